// oscar_quantize_pack kernel: rotate -> clip -> INT2 quantise -> pack.
//
// Demotes tokens of one tensor (K or V) into 64-token INT2 pages.  The step
// order (rotate by the fixed R, clip with the per-layer threshold, quantise
// with a per-group scale/zero point, pack four 2-bit codes per byte) is the
// demotion step of the serving pipeline in the myzaker.com article on OSCAR;
// R and the threshold are the offline artefacts of the gist.science OSCAR
// technical summary, section 2.2A.
//
// Block = (tile of 32 tokens, one KV head).  R[g] columns are read once per
// block and reused for the tile.  The rotation accumulates in fp64 on the
// matrix cores (the bf16 x fp32 products are exact in fp64) and rounds once
// to fp32, so every later decision (clip, min/max, fp16 rounding of
// scale/zero, the code) is taken on the correctly rounded fp32 rotated value.
#include <algorithm>

#include "common.hpp"
#include "demote.hpp"

namespace oscar {
namespace {

constexpr int kQTok = 32;  // tokens per block

// fp64 sum over the 16 lanes of a DPP row, every lane receiving it (all lanes
// of the wave active)
__device__ __forceinline__ double group16_sum_f64(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  return v + dpp_f64<kDppMirror>(v);
}

typedef double v4d __attribute__((ext_vector_type(4)));

// Eight waves per SIMD (at most 64 VGPRs; 54 without spills): the loads of x
// and R and the fp64 products are latency-bound, and eight resident blocks
// per compute unit hide more of it than the six that 80 VGPRs allow.
template <int D>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(8, 8))) void quantize_pack_kernel(
    int kind, const uint16_t* __restrict__ x, int64_t n_src, int64_t tok_stride,
    int64_t head_stride, const int32_t* __restrict__ src_idx, int64_t n_tok, int n_kv,
    const float* __restrict__ rot, float clip, const int32_t* __restrict__ dst_slot,
    uint8_t* __restrict__ codes, uint32_t* __restrict__ sz, int64_t n_pages) {
  constexpr int kRowBytes = D / 4;       // code bytes per token
  constexpr int kPlane = D / 16;         // bytes per token in one K plane
  // The x tile (channel-major, padded so the transposed writes are conflict-free)
  // and, once every wave's products are done, the clipped rotated values share
  // one LDS buffer.
  constexpr int kXs = D * (kQTok + 1), kYs = kQTok * (D + 1);
  __shared__ float tile[kXs > kYs ? kXs : kYs];
  float (*xs)[kQTok + 1] = reinterpret_cast<float (*)[kQTok + 1]>(tile);
  float (*ys)[D + 1] = reinterpret_cast<float (*)[D + 1]>(tile);
  __shared__ int64_t src_s[kQTok];
  __shared__ int64_t dst_s[kQTok];       // -1: skip this token
  constexpr int kMaxGroups = D / 32;     // 32-channel groups per head
  __shared__ float zf[kQTok][kMaxGroups], sf[kQTok][kMaxGroups];   // per token and group

  const int g = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kQTok;
  const int tid = threadIdx.x;
  const bool lm = (kind & OSCAR_CODEBOOK_LLOYD_MAX) != 0;
  const int ng = kind_groups(kind, D);   // group k holds channels k*D/ng ..
  const bool k_layout = kind_is_k(kind);

  if (tid < kQTok) {
    const int64_t t = t0 + tid;
    int64_t s = -1, slot = -1;
    if (t < n_tok) {
      s = src_idx ? (int64_t)src_idx[t] : t;
      slot = dst_slot[t];
      if (s < 0 || s >= n_src || slot < 0 || slot >= n_pages * kPage) {
        s = -1;
        slot = -1;
      }
    }
    src_s[tid] = s;
    dst_s[tid] = slot;
  }
  __syncthreads();

  // x tile: thread (t, chunk) loads channels 8 chunk .. 8 chunk + 7 of token t
  // as one 16-byte vector when the row is 16-byte aligned, else element by element
  for (int e = tid; e < kQTok * (D / 8); e += kBlock) {
    const int t = e / (D / 8), c0 = 8 * (e % (D / 8));
    const int64_t s = src_s[t];
    float v[8];
    if (s < 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = 0.0f;
    } else {
      const uint16_t* src = x + s * tok_stride + (int64_t)g * head_stride + c0;
      if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) {
        const uint4 w = *reinterpret_cast<const uint4*>(src);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[2 * k] = bf16_to_f32(ww[k] & 0xffffu);
          v[2 * k + 1] = bf16_to_f32(ww[k] >> 16);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = bf16_to_f32(src[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) xs[c0 + k][t] = v[k];
  }
  __syncthreads();

  // y[t][j] = sum_i x[t][i] * R[i][j] in fp64 on the matrix cores
  // (v_mfma_f64_16x16x4_f64: A[row][k] in lane row + 16k, B[k][col] in lane
  // col + 16k, D[row][col] in element row / 4 of lane col + 16 (row % 4)).
  // The bf16 x fp32 products are exact in fp64, and the sums are fp64, then
  // rounded once to fp32.  Wave w computes both 16-token tiles for the NT
  // column tiles of 16 starting at NT w, so each element of R is read by one
  // wave of the block.
  constexpr int NT = D / 64;             // column tiles per wave (2 for d = 128, 1 for d = 64)
  static_assert(kQTok == 32 && kBlock == 256, "2 token tiles x 4 column quarters, one quarter per wave");
  {
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int nt0 = NT * wave;
    const int row = lane & 15, kk = lane >> 4;
    const float* R = rot + (size_t)g * D * D + 16 * nt0 + row;
    v4d acc[2][NT];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[m][n] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 4) {
      const double a0 = (double)xs[k0 + kk][row], a1 = (double)xs[k0 + kk][16 + row];
      const float* Rk = R + (size_t)(k0 + kk) * D;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const double b = (double)Rk[16 * n];
        acc[0][n] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b, acc[0][n], 0, 0, 0);
        acc[1][n] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b, acc[1][n], 0, 0, 0);
      }
    }
    __syncthreads();   // every wave has read the x tile: its LDS now takes the rotated values
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ys[16 * m + kk + 4 * r][16 * (nt0 + n) + row] = fminf(fmaxf((float)acc[m][n][r], -clip), clip);
  }
  __syncthreads();

  // per-token group statistics: zero = fp16(min), scale = fp16((max - min) / 3),
  // or the Lloyd-Max mean and deviation (fp64).  A 16-lane DPP row handles one
  // token (four tokens per wave at a time); lane c of the row holds channels
  // c + 16k, so with 64- or 32-channel groups elements k of one group are adjacent.
  {
    constexpr int KP = D / 16;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int gq = lane >> 4, c = lane & 15;
    const int per = KP / ng;     // elements of one group in this lane
    for (int rd = 0; rd < kQTok / 16; ++rd) {
      const int t = 16 * rd + 4 * wave + gq;
      float v[KP];
#pragma unroll
      for (int k = 0; k < KP; ++k) v[k] = ys[t][c + 16 * k];
      for (int j = 0; j < ng; ++j) {
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < KP; ++k) {
          if (k / per != j) continue;
          mn = fminf(mn, v[k]);
          mx = fmaxf(mx, v[k]);
        }
        mn = group16_min(mn);
        mx = group16_max(mx);
        __half z = __float2half_rn(mn);
        __half s = __float2half_rn(__fdiv_rn(mx - mn, 3.0f));
        if (lm) {
          double s1 = 0.0;
#pragma unroll
          for (int k = 0; k < KP; ++k)
            if (k / per == j) s1 += (double)v[k];
          const double mean = group16_sum_f64(s1) / (D / ng);
          double s2 = 0.0;
#pragma unroll
          for (int k = 0; k < KP; ++k) {
            if (k / per != j) continue;
            const double dv = (double)v[k] - mean;
            s2 = __dadd_rn(s2, __dmul_rn(dv, dv));
          }
          lm_scale_zero(mean, group16_sum_f64(s2), D / ng, s, z);
        }
        if (c == 0) {
          zf[t][j] = __half2float(z);
          sf[t][j] = __half2float(s);
          const int64_t slot = dst_s[t];
          if (slot >= 0) {
            const int64_t page = slot / kPage;
            const int o = (int)(slot % kPage);
            sz[((page * n_kv + g) * ng + j) * kPage + o] =
                (uint32_t)__half_as_ushort(s) | ((uint32_t)__half_as_ushort(z) << 16);
          }
        }
      }
    }
  }
  __syncthreads();

  // codes: rint((y - zero) / scale) clamped to [0, 3], 4 per byte, LSB first
  for (int e = tid; e < kQTok * kRowBytes; e += kBlock) {
    const int t = e / kRowBytes, i = e % kRowBytes;
    const int64_t slot = dst_s[t];
    if (slot < 0) continue;
    const int j = (4 * i) / (D / ng);   // the group of channels 4i..4i+3
    const float z = zf[t][j], s = sf[t][j];
    uint32_t byte = 0;
    if (lm) {
#pragma unroll
      for (int q = 0; q < 4; ++q) byte |= lm_code(ys[t][4 * i + q], z, s) << (2 * q);
    } else if (s != 0.0f) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v = rintf(__fdiv_rn(ys[t][4 * i + q] - z, s));
        v = fminf(fmaxf(v, 0.0f), 3.0f);
        byte |= (uint32_t)v << (2 * q);
      }
    }
    const int64_t page = slot / kPage;
    const int o = (int)(slot % kPage);
    uint8_t* blk = codes + (page * n_kv + g) * (int64_t)(kPage * kRowBytes);
    const int pos = k_layout ? (i / kPlane) * (kPage * kPlane) + o * kPlane + (i % kPlane) : i * kPage + o;
    blk[pos] = (uint8_t)byte;
  }
}

// ---------------------------------------------------------------------------
// Bulk path on the bf16 matrix cores (uniform codebook, head_dim 128).
//
// The rotation runs as y~ = x (R1 + R2 + R3) on v_mfma_f32_16x16x32_bf16, R^T
// as the A operand (rows = output channels) and the bf16 tokens as the B
// operand (columns = tokens).  R splits into three bf16 parts, R1 = bf16(R),
// R2 = bf16(R - R1), R3 = R - R1 - R2, whose sum is R exactly (each part takes
// the next 8 significant bits of R's 24; only entries below 2^-110 lose bits to
// the bf16 subnormal range).  Every product is exact in fp32.  For k-block kb
// (inputs 32kb .. 32kb+31) one chain computes
//   m_kb = x_kb R1_kb + (x_kb R2_kb + x_kb R3_kb)
// and y~ = ((m_0 + m_1) + m_2) + m_3.  With one instruction summing 32 products
// into its fp32 input, and every addition inside it keeping at least 24
// significant bits (rounded or truncated, in whatever order), an instruction
// errs by at most 32 * 2^-23 (|C| + sum|p|) = 2^-18 (|C| + sum|p|).  Summed
// over the chains and the three additions, for every channel j
//   |y~_j - y_j| <= 4.4e-6 S_j + (subnormal flushes, below 1e-30),
//   S_j = sum_i |x_i| |R_ij| <= ||x||_2 ||R_:j||_2,
// so E = 4.4e-6 ||x||_2 max_j ||R_:j||_2 + 1e-30 bounds every channel of a
// token.
//
// The exact fp32 rotated value RN(y_j) then lies in [RN(y~_j - E), RN(y~_j +
// E)] (rounding is monotone), and so do the clipped group minimum and
// maximum.  Every later step of the quantiser is monotone too (fp32
// subtraction, the division by 3, fp16 rounding), so
//  * zero = fp16(min) and scale = fp16((max - min) / 3) are certain when the
//    two ends of their interval round to the same fp16 value; the division
//    by 3 is bracketed by products with the fp32 neighbours of 1/3.  A group
//    whose interval straddles an fp16 rounding boundary (about one in ten)
//    recomputes the channels that can hold its minimum and maximum (those
//    within 2E of the approximate extreme, usually one each) as fp64 dot
//    products rounded once to fp32, and takes zero and scale from them
//    exactly as the reference quantiser does;
//  * a code is read off t = (y~ - zero) / scale unless t lies within the
//    error of y~, of the fp32 steps of the reference quantiser and of the
//    reciprocal used here, of a bin edge c + 1/2; those channels are
//    recomputed exactly and coded with the reference division.
//
// Layout: R's three parts sit in LDS as ready A operands (96 KB); a wave
// takes 32 tokens at a time (two 16-token column blocks), loads their bf16
// rows straight from HBM as B operands, and computes all 128 channels, so
// lane (n, q) ends up with channels 16 cb + 4 q + i (cb = 0..7, i = 0..3) of
// token n of each column block: the four lanes n, n + 16, n + 32, n + 48
// hold one token, and their statistics need two lane exchanges.  No wave
// waits for another after the set-up.
// ---------------------------------------------------------------------------
constexpr int kMWaves = 8;                 // waves per block
constexpr int kMThreads = kMWaves * kWave;
constexpr int kFragBytes = 1024;           // one A operand: 64 lanes x 8 bf16
constexpr float kRotErr = 4.4e-6f;         // E / (||x|| max_j ||R_:j||)
constexpr float kRotErrAbs = 1e-30f;       // subnormal flushes inside the matrix cores
constexpr uint32_t kUnsureMark = 0x7E00u;  // (scale, zero) of a token left to the exact pass: scale = fp16 NaN

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float clamp_sym(float v, float tau) { return __builtin_amdgcn_fmed3f(v, -tau, tau); }
__device__ __forceinline__ int frag_offset(int part, int cb, int kb) { return ((part * 8 + cb) * 4 + kb) * kFragBytes; }

// signed-integer keys that order like the (finite) floats, so that minima and
// maxima over lanes need no canonicalisation of the exchanged values
__device__ __forceinline__ int order_key(float f) {
  const int b = __float_as_int(f);
  return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float key_value(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7fffffff)); }

// Reductions over the four lanes of a token (lanes n, n + 16, n + 32, n + 48)
// with the gfx950 row swaps: v_permlane16_swap of a register with itself
// hands every lane its own row and the neighbouring row's value (rows 0/1,
// 2/3), v_permlane32_swap its own half and the other half's.  Combining the
// two results in the same order on every lane gives all four lanes the same
// value.  VALU only; every lane of the four must be active.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_t swap16(uint32_t v) { return __builtin_amdgcn_permlane16_swap(v, v, false, false); }
__device__ __forceinline__ u32x2_t swap32(uint32_t v) { return __builtin_amdgcn_permlane32_swap(v, v, false, false); }
__device__ __forceinline__ float tok_sum(float v) {
  u32x2_t r = swap16(__float_as_uint(v));
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = swap32(__float_as_uint(v));
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ int tok_imin(int k) {
  u32x2_t r = swap16((uint32_t)k);
  k = min((int)r[0], (int)r[1]);
  r = swap32((uint32_t)k);
  return min((int)r[0], (int)r[1]);
}
__device__ __forceinline__ int tok_imax(int k) {
  u32x2_t r = swap16((uint32_t)k);
  k = max((int)r[0], (int)r[1]);
  r = swap32((uint32_t)k);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ uint32_t tok_or(uint32_t v) {
  u32x2_t r = swap16(v);
  v = r[0] | r[1];
  r = swap32(v);
  return r[0] | r[1];
}
__device__ __forceinline__ double tok_sum_f64(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const u32x2_t lo = swap16((uint32_t)u), hi = swap16((uint32_t)(u >> 32));
  v = __longlong_as_double((long long)(((unsigned long long)hi[0] << 32) | lo[0])) +
      __longlong_as_double((long long)(((unsigned long long)hi[1] << 32) | lo[1]));
  const unsigned long long w = (unsigned long long)__double_as_longlong(v);
  const u32x2_t lo2 = swap32((uint32_t)w), hi2 = swap32((uint32_t)(w >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi2[0] << 32) | lo2[0])) +
         __longlong_as_double((long long)(((unsigned long long)hi2[1] << 32) | lo2[1]));
}

// next pending channel of each token: the lowest channel whose bit is set in
// the masks of its four lanes (bit 4 cb + i of lane q: channel 16 cb + 4 q + i);
// 128 when none is
__device__ __forceinline__ int tok_next(uint32_t mask, int q) {
  int c = 128;
  if (mask) {
    const int b = __builtin_ctz(mask);
    c = 16 * (b >> 2) + 4 * q + (b & 3);
  }
  return tok_imin(c);
}
__device__ __forceinline__ uint32_t channel_bit(int j) { return 1u << (4 * (j >> 4) + (j & 3)); }

// Exact rotated value of channel j of the lanes' token: sum_i x_i R[i][j] in
// fp64, lane q taking i = 32 kb + 8 q + e (the inputs it holds), rounded once
// to fp32.  R is the row-major copy in LDS (rows of 128 floats); all four
// lanes get the value.
__device__ __forceinline__ float exact_channel4(const uint4 (&xq)[4], const float* rl, int j, int q) {
  double acc = 0.0;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const float* col = rl + (32 * kb + 8 * q) * 128 + j;
    uint32_t w[4] = {xq[kb].x, xq[kb].y, xq[kb].z, xq[kb].w};
    // converted here on every call (hoisted, the 32 fp64 inputs would hold 64 registers)
    asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xv = (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : __uint_as_float(w[e >> 1] << 16);
      acc = fma((double)xv, (double)col[e * 128], acc);
    }
  }
  return (float)tok_sum_f64(acc);
}

// the reference quantiser's code of a clipped value (scale > 0)
__device__ __forceinline__ float ref_code(float yc, float z, float s) {
  return fminf(fmaxf(rintf(__fdiv_rn(yc - z, s)), 0.0f), 3.0f);
}

// Statistics, scale/zero and codes of one token: the lane holds channels
// 16 cb + 4 q + i in y[cb][i] (approximate) and the bf16 inputs 32 kb + 8 q ..
// + 7 in xq[kb].  Groups of 128 / NG channels (cb 0..7 / NG per group).
// Fast mode writes every token whose scale, zero and codes are all certain
// and marks the others (fp16 NaN as the first group's scale, which no token
// can have); exact mode (the marked tokens, with R^T in LDS) takes the
// extremes of every group and the uncertain codes from exact channels.
template <int NG, bool kExact>
__device__ __forceinline__ void mfma_token(const v4f_t (&y)[8], const uint4 (&xq)[4], int64_t slot, int q, int g,
                                           int n_kv, float tau, float nr, const float* rt,
                                           uint8_t* __restrict__ codes, uint32_t* __restrict__ sz, bool k_layout) {
  constexpr int kCbPerGroup = 8 / NG;
  float sq = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const uint32_t w[4] = {xq[kb].x, xq[kb].y, xq[kb].z, xq[kb].w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]), __builtin_bit_cast(bf16x2_t, w[e]), sq,
                                           false);
  }
  sq = tok_sum(sq);
  bool zero_tok = false;
  if (__any(sq == 0.0f)) {   // all-zero tokens (and skipped ones) are told apart exactly
    uint32_t o = 0;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) o |= xq[kb].x | xq[kb].y | xq[kb].z | xq[kb].w;
    zero_tok = tok_or(o & 0x7fff7fffu) == 0;
  }
  // the norm's fp32 evaluation: squares below the normal range add at most 2^-119; the
  // square root errs by one unit, well inside the constant's margin
  const float E = fmaf(kRotErr, __builtin_amdgcn_sqrtf(sq + 0x1p-119f) * nr, kRotErrAbs);
  float yc[8][4];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) yc[cb][i] = clamp_sym(y[cb][i], tau);
  float mn_c[NG], mx_c[NG];
  __half zh[NG], sh[NG];
  bool sure[NG];
  bool unsure_any = false;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    float lo = yc[gi * kCbPerGroup][0], hi = lo;
#pragma unroll
    for (int cb = gi * kCbPerGroup; cb < (gi + 1) * kCbPerGroup; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo = fminf(lo, yc[cb][i]);
        hi = fmaxf(hi, yc[cb][i]);
      }
    mn_c[gi] = key_value(tok_imin(order_key(lo)));
    mx_c[gi] = key_value(tok_imax(order_key(hi)));
    // intervals holding the exact clipped extremes, and the fp16 zero and scale at their ends
    // (the ends of the division by 3 from the fp32 neighbours of 1/3)
    const float mn_lo = clamp_sym(mn_c[gi] - E, tau), mn_hi = clamp_sym(mn_c[gi] + E, tau);
    const float mx_lo = clamp_sym(mx_c[gi] - E, tau), mx_hi = clamp_sym(mx_c[gi] + E, tau);
    zh[gi] = __float2half_rn(mn_lo);
    sh[gi] = __float2half_rn((mx_lo - mn_hi) * __uint_as_float(0x3EAAAAAAu));
    sure[gi] = zero_tok ||
               (__half_as_ushort(zh[gi]) == __half_as_ushort(__float2half_rn(mn_hi)) &&
                __half_as_ushort(sh[gi]) ==
                    __half_as_ushort(__float2half_rn((mx_hi - mn_lo) * __uint_as_float(0x3EAAAAABu))));
    if (zero_tok) {   // y = +0 exactly: zero and scale +0, every code 0
      zh[gi] = __ushort_as_half(0);
      sh[gi] = __ushort_as_half(0);
    }
    unsure_any |= !sure[gi];
  }
  if (kExact && __any(unsure_any)) {
    // exact extremes of the uncertain groups.  An extreme whose unclipped approximation lies
    // beyond the clip by more than E is the clip; otherwise the candidates are the clipped
    // channels within 2E of the clipped approximate extreme (clipping moves no value by more
    // than its error moves it).
    float mn[NG], mx[NG];
    bool mn_open[NG], mx_open[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      float lo = y[gi * kCbPerGroup][0], hi = lo;
#pragma unroll
      for (int cb = gi * kCbPerGroup; cb < (gi + 1) * kCbPerGroup; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lo = fminf(lo, y[cb][i]);
          hi = fmaxf(hi, y[cb][i]);
        }
      lo = key_value(tok_imin(order_key(lo)));
      hi = key_value(tok_imax(order_key(hi)));
      mn[gi] = lo + E < -tau ? -tau : INFINITY;
      mx[gi] = hi - E > tau ? tau : -INFINITY;
      mn_open[gi] = !sure[gi] && mn[gi] == INFINITY;
      mx_open[gi] = !sure[gi] && mx[gi] == -INFINITY;
    }
    uint32_t cmn = 0, cmx = 0;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int gi = cb / kCbPerGroup;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (mn_open[gi] && yc[cb][i] <= mn_c[gi] + 2.0f * E) cmn |= 1u << (4 * cb + i);
        if (mx_open[gi] && yc[cb][i] >= mx_c[gi] - 2.0f * E) cmx |= 1u << (4 * cb + i);
      }
    }
    // every round clears at least one bit of every token that has any (128 bits per token)
    for (int round = 0; round < 128 && __any((cmn | cmx) != 0); ++round) {
      const int jn = tok_next(cmn, q), jx = tok_next(cmx, q);
      if (jn < 128) {
        const float v = clamp_sym(exact_channel4(xq, rt, jn, q), tau);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
          if (jn / (128 / NG) == gi) mn[gi] = fminf(mn[gi], v);
        if (((jn >> 2) & 3) == q) cmn &= ~channel_bit(jn);
      }
      if (jx < 128) {
        const float v = clamp_sym(exact_channel4(xq, rt, jx, q), tau);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
          if (jx / (128 / NG) == gi) mx[gi] = fmaxf(mx[gi], v);
        if (((jx >> 2) & 3) == q) cmx &= ~channel_bit(jx);
      }
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
      if (!sure[gi]) {
        zh[gi] = __float2half_rn(mn[gi]);
        sh[gi] = __float2half_rn(__fdiv_rn(mx[gi] - mn[gi], 3.0f));
      }
  }

  // ---- codes from t = (yc~ - zero) / scale.  |t - T| for the reference quantiser's
  // T = RN(RN(yc - zero) / scale) is at most (E + 2^-21 (m + 2|zero| + scale)) / scale + 2^-21,
  // m bounding |yc| over the group (the error of y~, the two roundings of T, the reciprocal,
  // -zero/scale and the fma, with |t| <= 4 where it matters); a code is sure when t is farther
  // than that from every half-integer.
  float z[NG], s[NG], rs[NG], nzrs[NG], thr[NG], worst[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    z[gi] = __half2float(zh[gi]);
    s[gi] = __half2float(sh[gi]);
    rs[gi] = s[gi] > 0.0f ? __builtin_amdgcn_rcpf(s[gi]) : 0.0f;
    nzrs[gi] = -z[gi] * rs[gi];
    const float m = fmaxf(fabsf(mn_c[gi]), fabsf(mx_c[gi])) + E;
    const float dt = fmaf(fmaf(4.8e-7f, m + 2.0f * fabsf(z[gi]) + s[gi], E), rs[gi] * 1.0001f, 4.8e-7f);
    thr[gi] = 0.5f - dt;   // |t - rint(t)| below this: sure
    worst[gi] = 0.0f;
  }
  uint32_t bytes[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    const int gi = cb / kCbPerGroup;
    float p = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float t = fmaf(yc[cb][i], rs[gi], nzrs[gi]);
      const float r = rintf(t);
      worst[gi] = fmaxf(worst[gi], fabsf(t - r));
      p = fmaf(__builtin_amdgcn_fmed3f(r, 0.0f, 3.0f), (float)(1 << (2 * i)), p);
    }
    bytes[cb] = (uint32_t)p;
  }
  bool code_unsure = false;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) code_unsure = code_unsure || worst[gi] >= thr[gi];
  const int64_t page = slot / kPage;
  const int o = (int)(slot % kPage);
  if (!kExact) {
    if (tok_or((unsure_any || code_unsure) ? 1u : 0u)) {   // the exact pass finishes this token
      if (slot >= 0 && q == 0) sz[((page * n_kv + g) * NG) * kPage + o] = kUnsureMark;
      return;
    }
  } else if (__any(code_unsure)) {
    uint32_t um = 0;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int gi = cb / kCbPerGroup;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float t = fmaf(yc[cb][i], rs[gi], nzrs[gi]);
        if (fabsf(t - rintf(t)) >= thr[gi]) um |= 1u << (4 * cb + i);
      }
    }
    for (int round = 0; round < 128 && __any(um != 0); ++round) {
      const int j = tok_next(um, q);
      if (j < 128) {
        const float v = exact_channel4(xq, rt, j, q);
        if (((j >> 2) & 3) == q) {
          float zj = z[0], sj = s[0];
#pragma unroll
          for (int gi = 1; gi < NG; ++gi)
            if (j / (128 / NG) == gi) {
              zj = z[gi];
              sj = s[gi];
            }
          const uint32_t c = (uint32_t)ref_code(clamp_sym(v, tau), zj, sj);
          const int cbj = j >> 4, sh2 = 2 * (j & 3);
#pragma unroll
          for (int cb = 0; cb < 8; ++cb)
            if (cb == cbj) bytes[cb] = (bytes[cb] & ~(3u << sh2)) | (c << sh2);
          um &= ~channel_bit(j);
        }
      }
    }
  }
  if (slot >= 0 && q < NG) {   // lane q writes group q
    __half s16 = sh[0], z16 = zh[0];
#pragma unroll
    for (int gi = 1; gi < NG; ++gi)
      if (q == gi) {
        s16 = sh[gi];
        z16 = zh[gi];
      }
    sz[((page * n_kv + g) * NG + q) * kPage + o] =
        (uint32_t)__half_as_ushort(s16) | ((uint32_t)__half_as_ushort(z16) << 16);
  }
  if (slot >= 0) {
    uint8_t* blk = codes + (page * n_kv + g) * (int64_t)(kPage * 32);
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int m = 4 * cb + q;   // byte m of the token's row: channels 4m .. 4m+3
      blk[k_layout ? (m >> 3) * (kPage * 8) + o * 8 + (m & 7) : m * kPage + o] = (uint8_t)bytes[cb];
    }
  }
}

// Set-up shared by both kernels: A operand (cb, kb) of part p, lane (i, q),
// holds R[32 kb + 8 q + e][16 cb + i], e = 0..7, in bf16 part p of R.
__device__ __forceinline__ void build_fragments(const float* __restrict__ R, uint8_t* frag, int tid) {
  constexpr int D = 128;
  constexpr int kSlots = 32 * kWave / kMThreads;   // operand slots per thread
  float w8[kSlots][8];
#pragma unroll
  for (int k = 0; k < kSlots; ++k) {   // every load in flight at once
    const int s = tid + k * kMThreads, cb = s >> 8, kb = (s >> 6) & 3, fl = s & 63;
    const float* col = R + (size_t)(32 * kb + 8 * (fl >> 4)) * D + 16 * cb + (fl & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) w8[k][e] = col[(size_t)e * D];
  }
#pragma unroll
  for (int ks = 0; ks < kSlots; ++ks) {
    const int s = tid + ks * kMThreads, cb = s >> 8, kb = (s >> 6) & 3, fl = s & 63;
    u32x4_t p1, p2, p3;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t h[2], m[2], l[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float w = w8[ks][2 * k + e];
        h[e] = bf16_rne(w);
        const float r1 = w - bf16_val(h[e]);        // exact
        m[e] = bf16_rne(r1);
        l[e] = bf16_rne(r1 - bf16_val(m[e]));       // exact: at most 8 significant bits remain
      }
      p1[k] = h[0] | (h[1] << 16);
      p2[k] = m[0] | (m[1] << 16);
      p3[k] = l[0] | (l[1] << 16);
    }
    *reinterpret_cast<u32x4_t*>(frag + frag_offset(0, cb, kb) + 16 * fl) = p1;
    *reinterpret_cast<u32x4_t*>(frag + frag_offset(1, cb, kb) + 16 * fl) = p2;
    *reinterpret_cast<u32x4_t*>(frag + frag_offset(2, cb, kb) + 16 * fl) = p3;
  }
}

// max_j ||R_:j||_2 over the block (kMThreads = 512 threads): thread t sums the
// squares of rows 32 (t / 128) .. + 31 of column t % 128 (all its loads in
// flight at once), the partial sums meet in tmp (516 floats of LDS, free
// again when this returns).
__device__ __forceinline__ float max_column_norm(const float* __restrict__ R, float* tmp, int tid, int lane, int wave) {
  static_assert(kMThreads == 512, "one 32-row strip of one column per thread");
  const float* col = R + (size_t)(32 * (tid >> 7)) * 128 + (tid & 127);
  float v[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) v[r] = col[(size_t)r * 128];
  float sq = 0.0f;
#pragma unroll
  for (int r = 0; r < 32; ++r) sq = fmaf(v[r], v[r], sq);
  tmp[tid] = sq;
  __syncthreads();
  if (tid < 128) {
    const float c = ((tmp[tid] + tmp[tid + 128]) + tmp[tid + 256]) + tmp[tid + 384];
    const float m = wave_max(c);
    if (lane == 0) tmp[512 + wave] = m;
  }
  __syncthreads();
  const float nr = sqrtf(fmaxf(tmp[512], tmp[513]));
  __syncthreads();
  return nr;
}

// The 16 x 128 rotated blocks of TB 16-token column blocks: y[tb][cb] holds
// channels 16 cb + 4 q + i of token n (lane (n, q)) of column block tb, from
// the bf16 inputs xq[tb].  Each A operand is read once for all TB blocks.
template <int TB>
__device__ __forceinline__ void rotate_blocks(const uint8_t* fl, const uint4 (&xq)[TB][4], v4f_t (&y)[TB][8]) {
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(fl + frag_offset(0, cb, kb));
      const bf16x8_t a2 = *reinterpret_cast<const bf16x8_t*>(fl + frag_offset(1, cb, kb));
      const bf16x8_t a3 = *reinterpret_cast<const bf16x8_t*>(fl + frag_offset(2, cb, kb));
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xq[tb][kb]);
        v4f_t m = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a3, b, v4f_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        m = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, b, m, 0, 0, 0);
        m = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, m, 0, 0, 0);
        y[tb][cb] = kb == 0 ? m : y[tb][cb] + m;
      }
    }
    // one 16-channel block at a time: at most 12 A operands and 8 product chains in registers
    // (reading the next block's operands ahead spills)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Exact pass over the tokens t_begin .. t_end - 1 of one block (KV head g)
// that its fast pass marked: each wave scans its share of them for the mark
// and recomputes the marked ones sixteen at a time (one column block), with
// R's A operands in frag and R row-major in rt.
constexpr int kScanPerLane = 8;   // tokens each lane tests per scan step
template <int NG>
__device__ __forceinline__ void exact_pass(int kind, const uint16_t* __restrict__ x, int64_t n_src, int64_t tok_stride,
                                           int64_t head_stride, const int32_t* __restrict__ src_idx, int n_kv,
                                           float tau, float nr, const int32_t* __restrict__ dst_slot,
                                           uint8_t* __restrict__ codes, uint32_t* __restrict__ sz, int64_t n_pages,
                                           const uint8_t* frag, const float* rt, int g, int64_t t_begin,
                                           int64_t t_end, int lane, int wave) {
  const int n = lane & 15, q = lane >> 4;
  const bool k_layout = kind_is_k(kind);
  // a batch: lane (n, q) takes the queued token (source row qs, slot qd) when n < count
  auto batch = [&](int64_t qs, int64_t qd, int count) {
    const int64_t src = n < count ? qs : -1, slot = n < count ? qd : -1;
    uint4 xq[1][4];
    if (src < 0) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) xq[0][kb] = make_uint4(0, 0, 0, 0);
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(x + src * tok_stride + (int64_t)g * head_stride + 8 * q);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) xq[0][kb] = p[4 * kb];
    }
    v4f_t y[1][8];
    rotate_blocks<1>(frag + 16 * lane, xq, y);
    mfma_token<NG, true>(y[0], xq[0], slot, q, g, n_kv, tau, nr, rt, codes, sz, k_layout);
  };

  // the queue: lanes n < qn (all four of each) hold a marked token's source row and slot
  int64_t qs = -1, qd = -1;
  int qn = 0;
  constexpr int kStep = kWave * kScanPerLane;
  for (int64_t base = t_begin + (int64_t)wave * kStep; base < t_end; base += (int64_t)kMWaves * kStep) {
    // all loads of the step in flight together: indices clamped into range, results masked
    bool marked[kScanPerLane];
    int64_t slot_k[kScanPerLane], src_k[kScanPerLane];
#pragma unroll
    for (int k = 0; k < kScanPerLane; ++k) {
      const int64_t t = base + k * kWave + lane;
      const int64_t tc = t < t_end ? t : t_begin;
      const int64_t sr = src_idx ? (int64_t)src_idx[tc] : tc;
      const int64_t d = dst_slot[tc];
      const bool ok = t < t_end && sr >= 0 && sr < n_src && d >= 0 && d < n_pages * kPage;
      slot_k[k] = ok ? d : 0;
      src_k[k] = sr;
      marked[k] = ok;
    }
#pragma unroll
    for (int k = 0; k < kScanPerLane; ++k) {
      const int64_t page = slot_k[k] / kPage;
      const uint32_t v = sz[((page * n_kv + g) * NG) * kPage + slot_k[k] % kPage];
      marked[k] = marked[k] && v == kUnsureMark;
    }
    uint32_t mbits = 0;
#pragma unroll
    for (int k = 0; k < kScanPerLane; ++k) mbits |= (marked[k] ? 1u : 0u) << k;
#pragma unroll 1
    for (int k = 0; k < kScanPerLane; ++k) {   // rolled: one copy of the batch below
      uint64_t mask = __ballot((mbits >> k) & 1u);
      int64_t sk = src_k[0], dk = slot_k[0];
#pragma unroll
      for (int kk = 1; kk < kScanPerLane; ++kk)
        if (k == kk) {
          sk = src_k[kk];
          dk = slot_k[kk];
        }
      while (mask) {   // wave-uniform
        const int l = __builtin_ctzll(mask);
        mask &= mask - 1;
        const int64_t sl = ((int64_t)__builtin_amdgcn_readlane((int)(sk >> 32), l) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)sk, l);
        const int64_t dl = ((int64_t)__builtin_amdgcn_readlane((int)(dk >> 32), l) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)dk, l);
        if (n == qn) {
          qs = sl;
          qd = dl;
        }
        if (++qn == 16) {
          batch(qs, qd, 16);
          qn = 0;
        }
      }
    }
  }
  if (qn > 0) batch(qs, qd, qn);
}

// Fast pass.  Block: one KV head and tiles_per_block consecutive 32-token
// tiles; wave w takes tiles w, w + 8, ... of them.
template <int NG>
__global__ __launch_bounds__(kMThreads, 1) void quantize_mfma_kernel(
    int kind, const uint16_t* __restrict__ x, int64_t n_src, int64_t tok_stride, int64_t head_stride,
    const int32_t* __restrict__ src_idx, int64_t n_tok, int n_kv, const float* __restrict__ rot, float clip,
    const int32_t* __restrict__ dst_slot, uint8_t* __restrict__ codes, uint32_t* __restrict__ sz,
    int64_t n_pages, int tiles_per_block) {
  __shared__ __attribute__((aligned(16))) uint8_t frag[3 * 32 * kFragBytes];   // A operands of R1, R2, R3
  // per wave: the second column block's y~ while the first one's statistics run (8 KB)
  __shared__ __attribute__((aligned(16))) v4f_t ystash[kMWaves][8][kWave];
  const int g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const bool k_layout = kind_is_k(kind);
  const int64_t n_tiles = (n_tok + 31) / 32;
  const int64_t tile0 = (int64_t)blockIdx.x * tiles_per_block;
  if (tile0 >= n_tiles) return;   // block-uniform
  const int64_t tile_end = min(tile0 + (int64_t)tiles_per_block, n_tiles);
  const float* R = rot + (size_t)g * 128 * 128;
  const float nr = max_column_norm(R, reinterpret_cast<float*>(&ystash[0][0][0]), tid, lane, wave);
  build_fragments(R, frag, tid);
  __syncthreads();
  const float tau = clip;

  // token 16 tb + n of a tile, its source row and slot (-1: skipped)
  auto token_info = [&](int64_t tile, int tb, int64_t& src, int64_t& slot) {
    const int64_t t = tile * 32 + 16 * tb + n;
    src = -1;
    slot = -1;
    if (tile < tile_end && t < n_tok) {
      const int64_t sr = src_idx ? (int64_t)src_idx[t] : t;
      const int64_t d = dst_slot[t];
      if (sr >= 0 && sr < n_src && d >= 0 && d < n_pages * kPage) {
        src = sr;
        slot = d;
      }
    }
  };
  // lane (n, q): inputs 32 kb + 8 q .. + 7 of the token (the B operand of k-block kb)
  auto load_x = [&](int64_t src, uint4 (&xq)[4]) {
    if (src < 0) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) xq[kb] = make_uint4(0, 0, 0, 0);
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(x + src * tok_stride + (int64_t)g * head_stride + 8 * q);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) xq[kb] = p[4 * kb];
    }
  };

  int64_t tile = tile0 + wave;
  int64_t src_c[2], slot_c[2], src_n[2], slot_n[2];
  token_info(tile, 0, src_c[0], slot_c[0]);
  token_info(tile, 1, src_c[1], slot_c[1]);
  uint4 xc[2][4];
  load_x(src_c[0], xc[0]);
  load_x(src_c[1], xc[1]);
  token_info(tile + kMWaves, 0, src_n[0], slot_n[0]);
  token_info(tile + kMWaves, 1, src_n[1], slot_n[1]);
  for (; tile < tile_end; tile += kMWaves) {
    // the indices of the tile after next, in flight during this tile
    int64_t src_f[2], slot_f[2];
    token_info(tile + 2 * kMWaves, 0, src_f[0], slot_f[0]);
    token_info(tile + 2 * kMWaves, 1, src_f[1], slot_f[1]);
    // the A operands are re-read every tile: an opaque lane offset keeps the compiler from
    // hoisting all 96 of them (384 registers) out of the loop
    int fo = 16 * lane;
    asm volatile("" : "+v"(fo));
    const uint8_t* fl = frag + fo;
    v4f_t y[2][8];
    rotate_blocks<2>(fl, xc, y);
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) ystash[wave][cb][lane] = y[1][cb];
    // the next tile's inputs, in flight during the statistics
    uint4 xn[2][4];
    load_x(src_n[0], xn[0]);
    load_x(src_n[1], xn[1]);
    mfma_token<NG, false>(y[0], xc[0], slot_c[0], q, g, n_kv, tau, nr, nullptr, codes, sz, k_layout);
    {
      v4f_t y1[8];
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) y1[cb] = ystash[wave][cb][lane];
      mfma_token<NG, false>(y1, xc[1], slot_c[1], q, g, n_kv, tau, nr, nullptr, codes, sz, k_layout);
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) xc[tb][kb] = xn[tb][kb];
      slot_c[tb] = slot_n[tb];
      src_n[tb] = src_f[tb];
      slot_n[tb] = slot_f[tb];
    }
  }

  // ---- the exact pass over this block's marked tokens, as soon as its own
  // fast pass is done (other blocks may still be in theirs): the barrier
  // makes every wave's marks visible to the block and frees ystash, which
  // then holds R row-major for the exact channels
  if (n_pages <= 0) return;   // block-uniform: nothing was written
  __syncthreads();
  float* rt = reinterpret_cast<float*>(&ystash[0][0][0]);
  static_assert(sizeof(ystash) >= 128 * 128 * sizeof(float), "R must fit where the stash was");
  {
    constexpr int kPer = 128 * 128 / 4 / kMThreads;
    float4 r4[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) r4[k] = reinterpret_cast<const float4*>(R)[tid + k * kMThreads];
#pragma unroll
    for (int k = 0; k < kPer; ++k) reinterpret_cast<float4*>(rt)[tid + k * kMThreads] = r4[k];
  }
  __syncthreads();
  exact_pass<NG>(kind, x, n_src, tok_stride, head_stride, src_idx, n_kv, tau, nr, dst_slot, codes, sz, n_pages,
                 frag, rt, g, tile0 * 32, min(tile_end * 32, n_tok), lane, wave);
}

// Few tokens (the steady-state step demotes one token per request): one block
// per (token, KV head).
template <int D>
__global__ __launch_bounds__(kBlock) void quantize_token_kernel(
    int kind, const uint16_t* __restrict__ x, int64_t n_src, int64_t tok_stride, int64_t head_stride,
    const int32_t* __restrict__ src_idx, int n_kv, const float* __restrict__ rot, float clip,
    const int32_t* __restrict__ dst_slot, uint8_t* __restrict__ codes, uint32_t* __restrict__ sz, int64_t n_pages) {
  demote_token_block<D>(kind, x, n_src, tok_stride, head_stride, src_idx, blockIdx.x, blockIdx.y, n_kv, rot, clip,
                        dst_slot, codes, sz, n_pages);
}

}  // namespace

// below this many tokens one block per (token, head) beats 32-token tiles
constexpr int64_t kTokenKernelMax = 64;

hipError_t launch_quantize_pack(int kind, const uint16_t* x, int64_t n_src, int64_t tok_stride,
                                int64_t head_stride, const int32_t* src_idx, int64_t n_tok, int n_kv,
                                int d, const float* rot, float clip, const int32_t* dst_slot,
                                uint8_t* codes, uint16_t* scale_zero, int64_t n_pages,
                                hipStream_t stream) {
  if (n_tok == 0) return hipSuccess;
  uint32_t* sz = reinterpret_cast<uint32_t*>(scale_zero);
  if (n_tok <= kTokenKernelMax) {
    const dim3 grid((unsigned)n_tok, (unsigned)n_kv);
    if (d == 128)
      quantize_token_kernel<128><<<grid, kBlock, 0, stream>>>(kind, x, n_src, tok_stride, head_stride, src_idx,
                                                             n_kv, rot, clip, dst_slot, codes, sz, n_pages);
    else
      quantize_token_kernel<64><<<grid, kBlock, 0, stream>>>(kind, x, n_src, tok_stride, head_stride, src_idx,
                                                            n_kv, rot, clip, dst_slot, codes, sz, n_pages);
    return hipGetLastError();
  }
  // the bf16 matrix-core path: uniform codebook, head_dim 128, 16-byte aligned source rows
  const bool lm = (kind & OSCAR_CODEBOOK_LLOYD_MAX) != 0;
  if (d == 128 && !lm && (reinterpret_cast<uintptr_t>(x) & 15) == 0 && tok_stride % 8 == 0 &&
      head_stride % 8 == 0) {
    const int64_t n_tiles = (n_tok + 31) / 32;
    // about one block per compute unit: each block loads R once and walks its tiles
    const int64_t per_head = std::max<int64_t>(1, std::min<int64_t>(n_tiles, 256 / n_kv));
    const int64_t tiles = (n_tiles + per_head - 1) / per_head;
    const dim3 fgrid((unsigned)((n_tiles + tiles - 1) / tiles), (unsigned)n_kv);
    if (kind_groups(kind, d) == 4) {
      quantize_mfma_kernel<4><<<fgrid, kMThreads, 0, stream>>>(kind, x, n_src, tok_stride, head_stride, src_idx,
                                                              n_tok, n_kv, rot, clip, dst_slot, codes, sz,
                                                              n_pages, (int)tiles);
    } else if (kind_groups(kind, d) == 2) {
      quantize_mfma_kernel<2><<<fgrid, kMThreads, 0, stream>>>(kind, x, n_src, tok_stride, head_stride, src_idx,
                                                              n_tok, n_kv, rot, clip, dst_slot, codes, sz,
                                                              n_pages, (int)tiles);
    } else {
      quantize_mfma_kernel<1><<<fgrid, kMThreads, 0, stream>>>(kind, x, n_src, tok_stride, head_stride, src_idx,
                                                              n_tok, n_kv, rot, clip, dst_slot, codes, sz,
                                                              n_pages, (int)tiles);
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((n_tok + kQTok - 1) / kQTok), (unsigned)n_kv);
  if (d == 128)
    quantize_pack_kernel<128><<<grid, kBlock, 0, stream>>>(kind, x, n_src, tok_stride, head_stride,
                                                          src_idx, n_tok, n_kv, rot, clip, dst_slot,
                                                          codes, sz, n_pages);
  else
    quantize_pack_kernel<64><<<grid, kBlock, 0, stream>>>(kind, x, n_src, tok_stride, head_stride,
                                                         src_idx, n_tok, n_kv, rot, clip, dst_slot,
                                                         codes, sz, n_pages);
  return hipGetLastError();
}

}  // namespace oscar

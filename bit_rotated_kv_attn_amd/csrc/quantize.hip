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
  constexpr int kPer = D / kWave;        // 64-channel groups per head
  __shared__ float zf[kQTok][kPer], sf[kQTok][kPer];   // per token and group

  const int g = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kQTok;
  const int tid = threadIdx.x;
  const bool lm = (kind & OSCAR_CODEBOOK_LLOYD_MAX) != 0;
  const int ng = (kind & OSCAR_GROUPS_64) ? kPer : 1;   // 64-channel groups: group k holds channels 64k..
  const bool k_layout = (kind & ~(OSCAR_CODEBOOK_LLOYD_MAX | OSCAR_GROUPS_64)) == OSCAR_KIND_K;

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
  // c + 16k, so with 64-channel groups elements k of one group are adjacent.
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

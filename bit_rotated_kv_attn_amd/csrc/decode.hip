// Decode attention over the three-segment cache (BF16 sink | INT2 history |
// BF16 recent), and the BF16 paged comparator.
//
// Method: the myzaker.com article on OSCAR (serving-pipeline paragraphs)
// describes decode as an INT2 part (unpack, scale/zero-point dequantisation,
// float accumulation) and a BF16 part over the sink and recent windows,
// merged by an online softmax.  The gist.science OSCAR technical summary
// (section 2.2B) adds that INT2 history is inverse-rotated inside the
// attention kernel.  Since R is orthogonal,
//     q . (x_hat R^T) = (q R) . x_hat   and   sum_t p_t x_hat_t R^T = (sum_t p_t x_hat_t) R^T,
// so the rotation is applied once per query head: to q before the history
// scan and to the accumulated history output after the split merge.  With
// x_hat = zero + c*scale, a history logit is scale*(q_rot . c) + zero*sum(q_rot).
//
// Launches (all on the caller's stream):
//   1. qrot_kernel    q_rot = q R_K[g], qsum = sum_j q_rot[j]
//   2. decode_main    one grid: history splits (split-K over pages) and
//                     BF16 64-token chunks; each writes an (m, l, acc) partial
//   3. merge_kernel   LSE merge of the history partials, * R_V^T, LSE merge
//                     with the BF16 partials, normalise
// Softmax state uses base-2 exponents (logits pre-scaled by log2 e).
#include "common.hpp"

namespace oscar {
namespace {

struct DecodeDev {
  int B, Hq, n_kv, G, sink_cap, recent_cap, max_hist_len, max_pages;
  int splits, pps, chunks, sink_chunks;
  float sm_log2;
  int64_t n_pages;
  const uint16_t *q, *sink_k, *sink_v, *recent_k, *recent_v;
  const int32_t *sink_len, *recent_len, *hist_len, *block_table;
  const uint8_t *k_codes, *v_codes;
  const uint32_t *k_sz, *v_sz;
  const float *r_k, *r_v;
  float *out, *qrot, *qsum, *hpart, *bpart;
};

struct Bf16Dev {
  int B, Hq, n_kv, G, max_pages, max_ctx_len, splits, pps;
  float sm_log2;
  int64_t n_pages;
  const uint16_t *q, *k_pages, *v_pages;
  const int32_t *block_table, *ctx_len;
  float *out, *part;
};

// per-wave online-softmax state for G query heads; lane owns channels lane + 64k
template <int D, int G>
struct WaveAcc {
  float m[G], l[G], z[G];
  float a[G][D / kWave];
};

template <int D, int G>
__device__ __forceinline__ void acc_init(WaveAcc<D, G>& s) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s.m[h] = -INFINITY;
    s.l[h] = 0.0f;
    s.z[h] = 0.0f;
#pragma unroll
    for (int k = 0; k < D / kWave; ++k) s.a[h][k] = 0.0f;
  }
}

// Softmax update for one 64-token tile: lane = token.  lg: base-2 logits
// (-inf for invalid lanes).  Writes each token's weight p (times wscale) to
// wbuf[lane*G + h] and returns via st the rescaled state; zterm is the value
// added to every channel per unit weight (the history zero point), 0 for BF16.
template <int D, int G>
__device__ __forceinline__ void softmax_tile(WaveAcc<D, G>& st, const float (&lg)[G], bool valid,
                                             float wscale, float zterm, float* wbuf, int lane) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mt = wave_max(lg[h]);
    const float mn = fmaxf(st.m[h], mt);
    const float alpha = exp2_or_zero(st.m[h], mn);
    const float pr = valid ? exp2f(lg[h] - mn) : 0.0f;
    st.l[h] = st.l[h] * alpha + wave_sum(pr);
    st.z[h] = st.z[h] * alpha + wave_sum(pr * zterm);
#pragma unroll
    for (int k = 0; k < D / kWave; ++k) st.a[h][k] *= alpha;
    st.m[h] = mn;
    wbuf[lane * G + h] = pr * wscale;
  }
  __builtin_amdgcn_wave_barrier();
}

// One INT2 history page (64 tokens, n_valid of them used) for KV head g.
template <int D, int G>
__device__ __forceinline__ void int2_page(WaveAcc<D, G>& st, const float* qr, const float* qs,
                                          float sm_log2, const uint8_t* __restrict__ kblk,
                                          const uint8_t* __restrict__ vblk,
                                          const uint32_t* __restrict__ ksz,
                                          const uint32_t* __restrict__ vsz, int n_valid,
                                          float* wbuf, int lane) {
  constexpr int kPlane = D / 16;   // bytes per token per K plane
  constexpr int kWords = D / 16;   // 32-bit words per token code row
  const bool valid = lane < n_valid;
  uint32_t w[kWords];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(kblk + p * kPage * kPlane + lane * kPlane);
#pragma unroll
    for (int u = 0; u < kPlane / 4; ++u) w[p * (kPlane / 4) + u] = src[u];
  }
  const uint32_t szk = ksz[lane], szv = vsz[lane];
  const float sk = f16_to_f32(szk & 0xffffu), zk = f16_to_f32(szk >> 16);
  const float sv = f16_to_f32(szv & 0xffffu), zv = f16_to_f32(szv >> 16);

  // code field k of row word u is rotated channel 16u + k
  float dot[G];
#pragma unroll
  for (int h = 0; h < G; ++h) dot[h] = 0.0f;
#pragma unroll
  for (int u = 0; u < kWords; ++u) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float c = (float)((w[u] >> (2 * k)) & 3u);
#pragma unroll
      for (int h = 0; h < G; ++h) dot[h] = fmaf(qr[h * D + 16 * u + k], c, dot[h]);
    }
  }
  float lg[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lg[h] = valid ? sm_log2 * fmaf(sk, dot[h], zk * qs[h]) : -INFINITY;
  softmax_tile<D, G>(st, lg, valid, sv, zv, wbuf, lane);

  // PV in rotated space: a[h][c] += sum_t p_t * scale_t * code_t[c]; the zero
  // point's share sum_t p_t * zero_t is kept in st.z and added at the merge.
#pragma unroll
  for (int k = 0; k < D / kWave; ++k) {
    const int c = lane + kWave * k;
    const uint4* col = reinterpret_cast<const uint4*>(vblk + (c >> 2) * kPage);
    uint32_t bw[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = col[q];
      bw[4 * q] = v.x; bw[4 * q + 1] = v.y; bw[4 * q + 2] = v.z; bw[4 * q + 3] = v.w;
    }
    const int sh = 2 * (c & 3);
    for (int t = 0; t < n_valid; ++t) {
      const float cv = (float)((bw[t >> 2] >> (8 * (t & 3) + sh)) & 3u);
#pragma unroll
      for (int h = 0; h < G; ++h) st.a[h][k] = fmaf(wbuf[t * G + h], cv, st.a[h][k]);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// One tile of up to 64 BF16 tokens; token t's row at kbase + t*D.
template <int D, int G>
__device__ __forceinline__ void bf16_tile(WaveAcc<D, G>& st, const float* qu, float sm_log2,
                                          const uint16_t* __restrict__ kbase,
                                          const uint16_t* __restrict__ vbase, int n_valid,
                                          float* wbuf, int lane) {
  const bool valid = lane < n_valid;
  float dot[G];
#pragma unroll
  for (int h = 0; h < G; ++h) dot[h] = 0.0f;
  if (valid) {
    const uint16_t* krow = kbase + (size_t)lane * D;
#pragma unroll 4
    for (int c8 = 0; c8 < D; c8 += 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(krow + c8);
      const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float k0 = __uint_as_float(e[q] << 16), k1 = __uint_as_float(e[q] & 0xffff0000u);
#pragma unroll
        for (int h = 0; h < G; ++h)
          dot[h] = fmaf(qu[h * D + c8 + 2 * q + 1], k1, fmaf(qu[h * D + c8 + 2 * q], k0, dot[h]));
      }
    }
  }
  float lg[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lg[h] = valid ? sm_log2 * dot[h] : -INFINITY;
  softmax_tile<D, G>(st, lg, valid, 1.0f, 0.0f, wbuf, lane);
#pragma unroll
  for (int k = 0; k < D / kWave; ++k) {
    const int c = lane + kWave * k;
    for (int t = 0; t < n_valid; ++t) {
      const float v = bf16_to_f32(vbase[(size_t)t * D + c]);
#pragma unroll
      for (int h = 0; h < G; ++h) st.a[h][k] = fmaf(wbuf[t * G + h], v, st.a[h][k]);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// Wave-level partial: [G][D+2] = (m, l, acc[D]) per head; acc includes z.
template <int D, int G>
__device__ __forceinline__ void write_wave_partial(const WaveAcc<D, G>& st, bool poison, float* dst,
                                                   int lane) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float* ph = dst + h * (D + 2);
    if (lane == 0) {
      ph[0] = st.m[h];
      ph[1] = poison ? NAN : st.l[h];
    }
#pragma unroll
    for (int k = 0; k < D / kWave; ++k) ph[2 + lane + kWave * k] = st.a[h][k] + st.z[h];
  }
}

// Merge the 4 waves' states of a block and write one partial.
template <int D, int G>
__device__ __forceinline__ void block_merge_write(const WaveAcc<D, G>& st, bool poison, float* mrg,
                                                  int* flags, float* dst, int tid) {
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  float* mw = mrg + wave * G * (D + 2);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (lane == 0) {
      mw[h * (D + 2)] = st.m[h];
      mw[h * (D + 2) + 1] = st.l[h];
    }
#pragma unroll
    for (int k = 0; k < D / kWave; ++k) mw[h * (D + 2) + 2 + lane + kWave * k] = st.a[h][k] + st.z[h];
  }
  if (lane == 0) flags[wave] = poison ? 1 : 0;
  __syncthreads();
  const bool bad = flags[0] | flags[1] | flags[2] | flags[3];
  constexpr int kW = kBlock / kWave;
  for (int e = tid; e < G * (D + 2); e += kBlock) {
    const int h = e / (D + 2), r = e % (D + 2);
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kW; ++v) M = fmaxf(M, mrg[v * G * (D + 2) + h * (D + 2)]);
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < kW; ++v) {
      const float f = exp2_or_zero(mrg[v * G * (D + 2) + h * (D + 2)], M);
      s += (r == 0) ? 0.0f : f * mrg[v * G * (D + 2) + e];
    }
    if (r == 0) dst[e] = M;
    else if (r == 1) dst[e] = bad ? NAN : s;
    else dst[e] = s;
  }
}

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void qrot_kernel(DecodeDev p) {
  __shared__ float qs[D];
  __shared__ float red[2];
  const int bh = blockIdx.x;
  const int h = bh % p.Hq, g = h / p.G;
  const int j = threadIdx.x;
  if (j < D) qs[j] = bf16_to_f32(p.q[(size_t)bh * D + j]);
  __syncthreads();
  float acc = 0.0f;
  if (j < D) {
    const float* R = p.r_k + (size_t)g * D * D;
    for (int i = 0; i < D; ++i) acc = fmaf(qs[i], R[i * D + j], acc);
    p.qrot[(size_t)bh * D + j] = acc;
  }
  const float s = wave_sum(j < D ? acc : 0.0f);
  if ((j & (kWave - 1)) == 0) red[j / kWave] = s;
  __syncthreads();
  if (j == 0) p.qsum[bh] = red[0] + red[1];
}

template <int D, int G>
__global__ __launch_bounds__(kBlock) void decode_main_kernel(DecodeDev p) {
  constexpr int kMrg = 4 * G * (D + 2);
  constexpr int kWbuf = 4 * kWave * G;
  __shared__ float q_s[G * D];
  __shared__ float qsum_s[G];
  __shared__ float scratch[kMrg > kWbuf ? kMrg : kWbuf];
  __shared__ int flags[4];
  const int b = blockIdx.z, g = blockIdx.y, x = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int h0 = g * G;
  const size_t part = (size_t)G * (D + 2);
  WaveAcc<D, G> st;
  acc_init(st);
  bool poison = false;
  float* wbuf = scratch + wave * kWave * G;

  if (x < p.splits) {  // ---- INT2 history split (block-uniform branch)
    for (int e = tid; e < G * D; e += kBlock) q_s[e] = p.qrot[((size_t)b * p.Hq + h0) * D + e];
    if (tid < G) qsum_s[tid] = p.qsum[(size_t)b * p.Hq + h0 + tid];
    __syncthreads();
    int hl = p.hist_len[b];
    if (hl < 0 || hl > p.max_hist_len) {
      poison = true;
      hl = 0;
    }
    const int hp = (hl + kPage - 1) / kPage;
    const int pb = x * p.pps;
    const int pe = min(pb + p.pps, hp);
    for (int pg = pb + wave; pg < pe; pg += kBlock / kWave) {
      const int pid = p.block_table[(size_t)b * p.max_pages + pg];
      if (pid < 0 || (int64_t)pid >= p.n_pages) {
        poison = true;
        continue;
      }
      const int nv = min(kPage, hl - pg * kPage);
      const size_t blk = (size_t)pid * p.n_kv + g;
      int2_page<D, G>(st, q_s, qsum_s, p.sm_log2, p.k_codes + blk * (kPage * D / 4),
                      p.v_codes + blk * (kPage * D / 4), p.k_sz + blk * kPage, p.v_sz + blk * kPage,
                      nv, wbuf, lane);
    }
    __syncthreads();  // wbuf and the merge area share scratch
    block_merge_write<D, G>(st, poison, scratch, flags,
                            p.hpart + (((size_t)b * p.n_kv + g) * p.splits + x) * part, tid);
  } else {  // ---- BF16 sink / recent chunks, one per wave
    for (int e = tid; e < G * D; e += kBlock) q_s[e] = bf16_to_f32(p.q[((size_t)b * p.Hq + h0) * D + e]);
    __syncthreads();
    const int c = (x - p.splits) * (kBlock / kWave) + wave;
    if (c < p.chunks) {
      const uint16_t *kb, *vb;
      int nv;
      if (c < p.sink_chunks) {
        int sl = p.sink_len[b];
        if (sl < 0 || sl > p.sink_cap) {
          poison = true;
          sl = 0;
        }
        const int t0 = c * kPage;
        nv = min(kPage, sl - t0);
        const size_t off = (((size_t)b * p.n_kv + g) * p.sink_cap + t0) * D;
        kb = p.sink_k + off;
        vb = p.sink_v + off;
      } else {
        int rl = p.recent_len[b];
        if (rl < 0 || rl > p.recent_cap) {
          poison = true;
          rl = 0;
        }
        const int t0 = (c - p.sink_chunks) * kPage;
        nv = min(kPage, rl - t0);
        const size_t off = (((size_t)b * p.n_kv + g) * p.recent_cap + t0) * D;
        kb = p.recent_k + off;
        vb = p.recent_v + off;
      }
      if (nv > 0) bf16_tile<D, G>(st, q_s, p.sm_log2, kb, vb, nv, wbuf, lane);
      write_wave_partial<D, G>(st, poison, p.bpart + (((size_t)b * p.n_kv + g) * p.chunks + c) * part,
                               lane);
    }
  }
}

template <int D>
__global__ __launch_bounds__(128) void merge_kernel(DecodeDev p) {
  __shared__ float arot[D];
  const int bh = blockIdx.x;
  const int b = bh / p.Hq, h = bh % p.Hq, g = h / p.G, kh = h % p.G;
  const int c = threadIdx.x;
  const size_t stride = (size_t)p.G * (D + 2);
  // history partials (rotated space)
  const float* hp = p.hpart + ((size_t)b * p.n_kv + g) * p.splits * stride + (size_t)kh * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, hp[s * stride]);
  float L = 0.0f, A = 0.0f;
  for (int s = 0; s < p.splits; ++s) {
    const float f = exp2_or_zero(hp[s * stride], M);
    L += f * hp[s * stride + 1];
    if (c < D) A += f * hp[s * stride + 2 + c];
  }
  if (c < D) arot[c] = A;
  __syncthreads();
  float oh = 0.0f;
  if (c < D && p.splits > 0) {
    const float* Rrow = p.r_v + ((size_t)g * D + c) * D;  // out[c] = sum_j arot[j] * R_V[c][j]
    for (int j2 = 0; j2 < D; ++j2) oh = fmaf(arot[j2], Rrow[j2], oh);
  }
  // BF16 partials (unrotated)
  const float* bp = p.bpart + ((size_t)b * p.n_kv + g) * p.chunks * stride + (size_t)kh * (D + 2);
  float Mb = -INFINITY;
  for (int s = 0; s < p.chunks; ++s) Mb = fmaxf(Mb, bp[s * stride]);
  float Lb = 0.0f, Ab = 0.0f;
  for (int s = 0; s < p.chunks; ++s) {
    const float f = exp2_or_zero(bp[s * stride], Mb);
    Lb += f * bp[s * stride + 1];
    if (c < D) Ab += f * bp[s * stride + 2 + c];
  }
  const float Mt = fmaxf(M, Mb);
  const float fh = exp2_or_zero(M, Mt), fb = exp2_or_zero(Mb, Mt);
  const float den = fh * L + fb * Lb;
  float o;
  if (isnan(den)) o = NAN;
  else o = (den > 0.0f) ? (fh * oh + fb * Ab) / den : 0.0f;
  if (c < D) p.out[(size_t)bh * D + c] = o;
}

// ---- BF16 paged comparator ---------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(kBlock) void bf16_paged_kernel(Bf16Dev p) {
  constexpr int kMrg = 4 * G * (D + 2);
  constexpr int kWbuf = 4 * kWave * G;
  __shared__ float q_s[G * D];
  __shared__ float scratch[kMrg > kWbuf ? kMrg : kWbuf];
  __shared__ int flags[4];
  const int b = blockIdx.z, g = blockIdx.y, x = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int h0 = g * G;
  WaveAcc<D, G> st;
  acc_init(st);
  bool poison = false;
  float* wbuf = scratch + wave * kWave * G;
  for (int e = tid; e < G * D; e += kBlock) q_s[e] = bf16_to_f32(p.q[((size_t)b * p.Hq + h0) * D + e]);
  __syncthreads();
  int cl = p.ctx_len[b];
  if (cl < 0 || cl > p.max_ctx_len) {
    poison = true;
    cl = 0;
  }
  const int np = (cl + kPage - 1) / kPage;
  const int pb = x * p.pps, pe = min(pb + p.pps, np);
  for (int pg = pb + wave; pg < pe; pg += kBlock / kWave) {
    const int pid = p.block_table[(size_t)b * p.max_pages + pg];
    if (pid < 0 || (int64_t)pid >= p.n_pages) {
      poison = true;
      continue;
    }
    const size_t off = ((size_t)pid * p.n_kv + g) * kPage * D;
    bf16_tile<D, G>(st, q_s, p.sm_log2, p.k_pages + off, p.v_pages + off, min(kPage, cl - pg * kPage),
                    wbuf, lane);
  }
  __syncthreads();
  block_merge_write<D, G>(st, poison, scratch, flags,
                          p.part + (((size_t)b * p.n_kv + g) * p.splits + x) * (size_t)G * (D + 2), tid);
}

template <int D>
__global__ __launch_bounds__(128) void merge_plain_kernel(Bf16Dev p) {
  const int bh = blockIdx.x;
  const int b = bh / p.Hq, h = bh % p.Hq, g = h / p.G, kh = h % p.G;
  const int c = threadIdx.x;
  const size_t stride = (size_t)p.G * (D + 2);
  const float* pp = p.part + ((size_t)b * p.n_kv + g) * p.splits * stride + (size_t)kh * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, pp[s * stride]);
  float L = 0.0f, A = 0.0f;
  for (int s = 0; s < p.splits; ++s) {
    const float f = exp2_or_zero(pp[s * stride], M);
    L += f * pp[s * stride + 1];
    if (c < D) A += f * pp[s * stride + 2 + c];
  }
  float o;
  if (isnan(L)) o = NAN;
  else o = (L > 0.0f) ? A / L : 0.0f;
  if (c < D) p.out[(size_t)bh * D + c] = o;
}

template <int D, int G>
void launch_main(const DecodeDev& dv, hipStream_t stream) {
  const unsigned nbf = (unsigned)((dv.chunks + 3) / 4);
  const dim3 grid((unsigned)dv.splits + nbf, (unsigned)dv.n_kv, (unsigned)dv.B);
  if (grid.x == 0) return;
  decode_main_kernel<D, G><<<grid, kBlock, 0, stream>>>(dv);
}

template <int D>
void launch_main_g(const DecodeDev& dv, hipStream_t stream) {
  switch (dv.G) {
    case 1: launch_main<D, 1>(dv, stream); break;
    case 2: launch_main<D, 2>(dv, stream); break;
    case 4: launch_main<D, 4>(dv, stream); break;
    case 8: launch_main<D, 8>(dv, stream); break;
    default: launch_main<D, 16>(dv, stream); break;
  }
}

template <int D, int G>
void launch_bf16(const Bf16Dev& dv, hipStream_t stream) {
  const dim3 grid((unsigned)dv.splits, (unsigned)dv.n_kv, (unsigned)dv.B);
  bf16_paged_kernel<D, G><<<grid, kBlock, 0, stream>>>(dv);
}

template <int D>
void launch_bf16_g(const Bf16Dev& dv, hipStream_t stream) {
  switch (dv.G) {
    case 1: launch_bf16<D, 1>(dv, stream); break;
    case 2: launch_bf16<D, 2>(dv, stream); break;
    case 4: launch_bf16<D, 4>(dv, stream); break;
    case 8: launch_bf16<D, 8>(dv, stream); break;
    default: launch_bf16<D, 16>(dv, stream); break;
  }
}

}  // namespace

namespace {
DecodeDev make_dev(const oscar_decode_args& a, const DecodePlan& plan, char* ws) {
  DecodeDev dv{};
  dv.B = a.batch; dv.Hq = a.n_q_heads; dv.n_kv = a.n_kv_heads; dv.G = a.n_q_heads / a.n_kv_heads;
  dv.sink_cap = a.sink_cap; dv.recent_cap = a.recent_cap;
  dv.max_hist_len = a.max_hist_len; dv.max_pages = a.max_pages;
  dv.splits = plan.splits; dv.pps = plan.pages_per_split;
  dv.chunks = plan.chunks; dv.sink_chunks = plan.sink_chunks;
  dv.sm_log2 = a.sm_scale * kLog2e;
  dv.n_pages = a.n_pages;
  dv.q = a.q; dv.sink_k = a.sink_k; dv.sink_v = a.sink_v; dv.recent_k = a.recent_k; dv.recent_v = a.recent_v;
  dv.sink_len = a.sink_len; dv.recent_len = a.recent_len; dv.hist_len = a.hist_len;
  dv.block_table = a.block_table;
  dv.k_codes = a.k_codes; dv.v_codes = a.v_codes;
  dv.k_sz = reinterpret_cast<const uint32_t*>(a.k_sz);
  dv.v_sz = reinterpret_cast<const uint32_t*>(a.v_sz);
  dv.r_k = a.r_k; dv.r_v = a.r_v; dv.out = a.out;
  dv.qrot = reinterpret_cast<float*>(ws + plan.off_qrot);
  dv.qsum = reinterpret_cast<float*>(ws + plan.off_qsum);
  dv.hpart = reinterpret_cast<float*>(ws + plan.off_hpart);
  dv.bpart = reinterpret_cast<float*>(ws + plan.off_bpart);
  return dv;
}
}  // namespace

hipError_t launch_decode_phase(int phase, const oscar_decode_args& a, const DecodePlan& plan, char* ws,
                               hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  const DecodeDev dv = make_dev(a, plan, ws);
  const unsigned nbh = (unsigned)a.batch * (unsigned)a.n_q_heads;
  const bool d128 = a.head_dim == 128;
  if (phase == kPhaseRotate) {
    if (plan.splits > 0) {
      if (d128) qrot_kernel<128><<<nbh, 128, 0, stream>>>(dv);
      else qrot_kernel<64><<<nbh, 128, 0, stream>>>(dv);
    }
  } else if (phase == kPhaseScan) {
    if (d128) launch_main_g<128>(dv, stream);
    else launch_main_g<64>(dv, stream);
  } else {
    if (d128) merge_kernel<128><<<nbh, 128, 0, stream>>>(dv);
    else merge_kernel<64><<<nbh, 128, 0, stream>>>(dv);
  }
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const oscar_bf16_decode_args& a, const Bf16Plan& plan, char* ws,
                              hipStream_t stream) {
  Bf16Dev dv{};
  dv.B = a.batch; dv.Hq = a.n_q_heads; dv.n_kv = a.n_kv_heads; dv.G = a.n_q_heads / a.n_kv_heads;
  dv.max_pages = a.max_pages; dv.max_ctx_len = a.max_ctx_len;
  dv.splits = plan.splits; dv.pps = plan.pages_per_split;
  dv.sm_log2 = a.sm_scale * kLog2e;
  dv.n_pages = a.n_pages;
  dv.q = a.q; dv.k_pages = a.k_pages; dv.v_pages = a.v_pages;
  dv.block_table = a.block_table; dv.ctx_len = a.ctx_len;
  dv.out = a.out;
  dv.part = reinterpret_cast<float*>(ws + plan.off_part);
  if (a.batch == 0) return hipSuccess;
  const unsigned nbh = (unsigned)a.batch * (unsigned)a.n_q_heads;
  if (plan.splits > 0) {
    if (a.head_dim == 128) launch_bf16_g<128>(dv, stream);
    else launch_bf16_g<64>(dv, stream);
  }
  if (a.head_dim == 128) merge_plain_kernel<128><<<nbh, 128, 0, stream>>>(dv);
  else merge_plain_kernel<64><<<nbh, 128, 0, stream>>>(dv);
  return hipGetLastError();
}

}  // namespace oscar

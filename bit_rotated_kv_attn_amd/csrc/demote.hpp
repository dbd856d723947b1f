// One-token INT2 demotion (rotate -> clip -> quantise -> pack) by one
// 256-thread block, shared by oscar_quantize_pack's few-token path and the
// fused decode step.  Same arithmetic as the tiled kernel: the rotated value is
// an fp64 dot product rounded once to fp32; zero = fp16(min), scale =
// fp16((max - min) / 3); code = rint((y - zero) / scale) clamped to [0, 3]
// (or the Lloyd-Max statistics and thresholds of oscar.h when kind carries
// OSCAR_CODEBOOK_LLOYD_MAX), over the whole head or over each 64-channel group
// (OSCAR_GROUPS_64; the scale/zero block of a (page, head) is then
// group-planar).
// Source: the demotion step of the serving pipeline in the myzaker.com article
// on OSCAR; R and the clip threshold from the gist.science OSCAR technical
// summary, section 2.2A.
#pragma once

#include "common.hpp"

namespace oscar {

// Thread (jq, part) loads its IP rows of columns 4jq..4jq+3 of R as 16-byte
// vectors, all in flight at once, and computes four partial fp64 dots; the P
// partials of a column are added in fp64 and rounded once to fp32.
template <int D>
__device__ __forceinline__ void demote_token_block(int kind, const uint16_t* __restrict__ x, int64_t n_src,
                                                   int64_t tok_stride, int64_t head_stride,
                                                   const int32_t* __restrict__ src_idx, int64_t t, int g, int n_kv,
                                                   const float* __restrict__ rot, float clip,
                                                   const int32_t* __restrict__ dst_slot, uint8_t* __restrict__ codes,
                                                   uint32_t* __restrict__ sz, int64_t n_pages) {
  constexpr int QPR = D / 4;             // column quads per row
  constexpr int P = kBlock / QPR;        // row parts of the dot product
  constexpr int IP = D / P;              // rows per part
  constexpr int kRowBytes = D / 4;
  constexpr int kPlane = D / 16;
  __shared__ float xs[D];
  __shared__ double parts[P][D];
  __shared__ float ys[D];
  __shared__ float red[2][kBlock / kWave];
  __shared__ double dred[2][kBlock / kWave];
  __shared__ float gzs[2][D / kWave];   // (zero, scale) of each group
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const bool lm = (kind & OSCAR_CODEBOOK_LLOYD_MAX) != 0;
  const bool grouped = (kind & OSCAR_GROUPS_64) != 0;   // 64-channel groups
  const bool k_layout = (kind & ~(OSCAR_CODEBOOK_LLOYD_MAX | OSCAR_GROUPS_64)) == OSCAR_KIND_K;
  const int64_t src = src_idx ? (int64_t)src_idx[t] : t;
  const int64_t slot = dst_slot[t];
  if (src < 0 || src >= n_src || slot < 0 || slot >= n_pages * kPage) return;   // block-uniform

  const int jq = tid % QPR, part = tid / QPR;
  const float4* R = reinterpret_cast<const float4*>(rot + (size_t)g * D * D + (size_t)part * IP * D) + jq;
  float4 r[IP];
#pragma unroll
  for (int k = 0; k < IP; ++k) r[k] = R[(size_t)k * QPR];
  if (tid < D) xs[tid] = bf16_to_f32(x[src * tok_stride + (int64_t)g * head_stride + tid]);
  __syncthreads();
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll
  for (int k = 0; k < IP; ++k) {
    const double xv = (double)xs[part * IP + k];
    a0 = fma(xv, (double)r[k].x, a0);
    a1 = fma(xv, (double)r[k].y, a1);
    a2 = fma(xv, (double)r[k].z, a2);
    a3 = fma(xv, (double)r[k].w, a3);
  }
  parts[part][4 * jq] = a0;
  parts[part][4 * jq + 1] = a1;
  parts[part][4 * jq + 2] = a2;
  parts[part][4 * jq + 3] = a3;
  __syncthreads();

  float mn = INFINITY, mx = -INFINITY;
  if (tid < D) {
    double y = parts[0][tid];
#pragma unroll
    for (int q = 1; q < P; ++q) y += parts[q][tid];
    const float yc = fminf(fmaxf((float)y, -clip), clip);
    ys[tid] = yc;
    mn = yc;
    mx = yc;
  }
  // per-wave (64-channel) extremes; a group is GW consecutive waves
  constexpr int kWaves = D / kWave;
  const int ng = grouped ? kWaves : 1, gw = kWaves / ng;
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) {
    red[0][wave] = mn;
    red[1][wave] = mx;
  }
  if (lm) {   // block-uniform: the group means, then the sums of squared deviations, in fp64
    const double v = wave_sum_f64(tid < D ? (double)ys[tid] : 0.0);
    if (lane == 0) dred[0][wave] = v;
    __syncthreads();
    double tot = 0.0;
    const int g0 = (wave < kWaves ? wave / gw : 0) * gw;   // first wave of this thread's group
    for (int w = g0; w < g0 + gw; ++w) tot += dred[0][w];
    const double dv = tid < D ? (double)ys[tid] - tot / (D / ng) : 0.0;
    const double sq = wave_sum_f64(__dmul_rn(dv, dv));
    if (lane == 0) dred[1][wave] = sq;
  }
  __syncthreads();
  if (tid < ng) {   // thread j: (scale, zero) of group j
    float gmn = INFINITY, gmx = -INFINITY;
    double sum = 0.0, sq = 0.0;
    for (int w = tid * gw; w < (tid + 1) * gw; ++w) {
      gmn = fminf(gmn, red[0][w]);
      gmx = fmaxf(gmx, red[1][w]);
      if (lm) {
        sum += dred[0][w];
        sq += dred[1][w];
      }
    }
    __half zh = __float2half_rn(gmn);
    __half sh = __float2half_rn(__fdiv_rn(gmx - gmn, 3.0f));
    if (lm) lm_scale_zero(sum / (D / ng), sq, D / ng, sh, zh);
    gzs[0][tid] = __half2float(zh);
    gzs[1][tid] = __half2float(sh);
    const int64_t page = slot / kPage;
    const int o = (int)(slot % kPage);
    sz[((page * n_kv + g) * ng + tid) * kPage + o] =
        (uint32_t)__half_as_ushort(sh) | ((uint32_t)__half_as_ushort(zh) << 16);
  }
  __syncthreads();
  if (tid < kRowBytes) {
    const int i = tid;
    const int j = (4 * i) / (D / ng);   // the group of channels 4i..4i+3
    const float z = gzs[0][j], s = gzs[1][j];
    const int64_t page = slot / kPage;
    const int o = (int)(slot % kPage);
    uint32_t byte = 0;
    if (lm) {
#pragma unroll
      for (int q = 0; q < 4; ++q) byte |= lm_code(ys[4 * i + q], z, s) << (2 * q);
    } else if (s != 0.0f) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v = rintf(__fdiv_rn(ys[4 * i + q] - z, s));
        v = fminf(fmaxf(v, 0.0f), 3.0f);
        byte |= (uint32_t)v << (2 * q);
      }
    }
    uint8_t* blk = codes + (page * n_kv + g) * (int64_t)(kPage * kRowBytes);
    const int pos = k_layout ? (i / kPlane) * (kPage * kPlane) + o * kPlane + (i % kPlane) : i * kPage + o;
    blk[pos] = (uint8_t)byte;
  }
}

}  // namespace oscar

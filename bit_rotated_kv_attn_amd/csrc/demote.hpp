// One-token INT2 demotion (rotate -> clip -> quantise -> pack) by one
// 256-thread block, shared by oscar_quantize_pack's few-token path and the
// fused decode step.  Same arithmetic as the tiled kernel: the rotated value is
// an fp64 dot product rounded once to fp32; zero = fp16(min), scale =
// fp16((max - min) / 3); code = rint((y - zero) / scale) clamped to [0, 3]
// (or the Lloyd-Max statistics and thresholds of oscar.h when kind carries
// OSCAR_CODEBOOK_LLOYD_MAX), over the whole head or over each 64- or
// 32-channel group (OSCAR_GROUPS_64, OSCAR_GROUPS_32; the scale/zero block of a
// (page, head) is then group-planar).
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
  constexpr int kUnits = D / 32;         // 32-channel units (half a wave each)
  __shared__ float red[2][kUnits];
  __shared__ double dred[2][kUnits];
  __shared__ float gzs[2][kUnits];      // (zero, scale) of each group
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const bool lm = (kind & OSCAR_CODEBOOK_LLOYD_MAX) != 0;
  const int ng = kind_groups(kind, D), gu = kUnits / ng;   // groups; units per group
  const bool k_layout = kind_is_k(kind);
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
  // extremes and sums of each 32-channel unit: the 16-lane row results of
  // rows (0, 1) and (2, 3) of a wave; a group is gu consecutive units.  The
  // sums of a group add its unit pairs first, as a whole-wave sum would.
  // Every lane read happens with the whole wave active (outside the
  // branches that store the results): a lane outside the branch would not
  // have finished the row reduction the read expects.
  auto group_sum = [&](const double* u, int j) {
    if (gu == 1) return u[j];
    double tot = 0.0;
    for (int k = j * gu; k < (j + 1) * gu; k += 2) tot += u[k] + u[k + 1];
    return tot;
  };
  constexpr int kWaves = D / kWave;
  mn = group16_min(mn);
  mx = group16_max(mx);
  const float mn0 = fminf(lane_value(mn, 0), lane_value(mn, 16)), mn1 = fminf(lane_value(mn, 32), lane_value(mn, 48));
  const float mx0 = fmaxf(lane_value(mx, 0), lane_value(mx, 16)), mx1 = fmaxf(lane_value(mx, 32), lane_value(mx, 48));
  if (wave < kWaves && lane == 0) {
    red[0][2 * wave] = mn0;
    red[0][2 * wave + 1] = mn1;
    red[1][2 * wave] = mx0;
    red[1][2 * wave + 1] = mx1;
  }
  if (lm) {   // block-uniform: the group means, then the sums of squared deviations, in fp64
    auto row_sum = [](double v) {
      v += dpp_f64<kDppXor1>(v);
      v += dpp_f64<kDppXor2>(v);
      v += dpp_f64<kDppHalfMirror>(v);
      return v + dpp_f64<kDppMirror>(v);
    };
    const double v = row_sum(tid < D ? (double)ys[tid] : 0.0);
    const double u0 = lane_value_f64(v, 0) + lane_value_f64(v, 16), u1 = lane_value_f64(v, 32) + lane_value_f64(v, 48);
    if (wave < kWaves && lane == 0) {
      dred[0][2 * wave] = u0;
      dred[0][2 * wave + 1] = u1;
    }
    __syncthreads();
    const int j = tid < D ? (tid / 32) / gu : 0;   // this thread's group
    const double dv = tid < D ? (double)ys[tid] - group_sum(dred[0], j) / (D / ng) : 0.0;
    const double w = row_sum(__dmul_rn(dv, dv));
    const double w0 = lane_value_f64(w, 0) + lane_value_f64(w, 16), w1 = lane_value_f64(w, 32) + lane_value_f64(w, 48);
    if (wave < kWaves && lane == 0) {
      dred[1][2 * wave] = w0;
      dred[1][2 * wave + 1] = w1;
    }
  }
  __syncthreads();
  if (tid < ng) {   // thread j: (scale, zero) of group j
    float gmn = INFINITY, gmx = -INFINITY;
    for (int k = tid * gu; k < (tid + 1) * gu; ++k) {
      gmn = fminf(gmn, red[0][k]);
      gmx = fmaxf(gmx, red[1][k]);
    }
    __half zh = __float2half_rn(gmn);
    __half sh = __float2half_rn(__fdiv_rn(gmx - gmn, 3.0f));
    if (lm) lm_scale_zero(group_sum(dred[0], tid) / (D / ng), group_sum(dred[1], tid), D / ng, sh, zh);
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

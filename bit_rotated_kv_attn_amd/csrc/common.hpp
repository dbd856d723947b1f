// Internal helpers shared by the liboscar kernels (gfx950, wave64).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "oscar.h"

namespace oscar {

constexpr int kPage = OSCAR_PAGE_TOKENS;  // tokens per page
constexpr int kWave = 64;                 // CDNA wavefront width
constexpr int kBlock = 256;               // threads per block (4 waves)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(bits16)));
}

// Reductions over the 16 lanes of a DPP row (lanes 16k..16k+15), every lane
// receiving the result: quad permutes (lane ^ 1, lane ^ 2), then the half-row
// and row mirrors.  VALU data movement, no LDS round trips.  The wave_*
// reductions add the four rows through scalar lane reads.  All of them need
// every lane of the wave active.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ float group16_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f32<kDppMirror>(v));
}

__device__ __forceinline__ float group16_min(float v) {
  v = fminf(v, dpp_f32<kDppXor1>(v));
  v = fminf(v, dpp_f32<kDppXor2>(v));
  v = fminf(v, dpp_f32<kDppHalfMirror>(v));
  return fminf(v, dpp_f32<kDppMirror>(v));
}

__device__ __forceinline__ float group16_sum(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  return v + dpp_f32<kDppMirror>(v);
}

__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_max(float v) {
  v = group16_max(v);
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

__device__ __forceinline__ float wave_min(float v) {
  v = group16_min(v);
  return fminf(fminf(lane_value(v, 0), lane_value(v, 16)), fminf(lane_value(v, 32), lane_value(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = group16_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// fp64: the two halves of each value move through the same DPP lanes
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)u, kCtrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), kCtrl, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

__device__ __forceinline__ double lane_value_f64(double v, int l) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), l);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
  return (lane_value_f64(v, 0) + lane_value_f64(v, 16)) + (lane_value_f64(v, 32) + lane_value_f64(v, 48));
}

// Lloyd-Max codebook (oscar.h): levels (-10, -3, 3, 10) in scale units, the
// scale per unit of deviation and the decision thresholds between the levels
constexpr double kLmUnit = 0.15104;
constexpr float kLmThreshold = 6.5f;

// fp16 (scale, zero) of a Lloyd-Max group from its fp64 sum and sum of
// squared deviations over n values: zero = fp16(fp32(mean)), scale =
// fp16(fp32(kLmUnit * deviation))
__device__ __forceinline__ void lm_scale_zero(double mean, double sq, int n, __half& sh, __half& zh) {
  zh = __float2half_rn((float)mean);
  sh = __float2half_rn((float)(kLmUnit * sqrt(sq / n)));
}

// Lloyd-Max code: the number of thresholds fp32(z + s*t), t in (-6.5, 0, 6.5), that y reaches
__device__ __forceinline__ uint32_t lm_code(float y, float z, float s) {
  return (uint32_t)(y >= fmaf(s, -kLmThreshold, z)) + (uint32_t)(y >= z) + (uint32_t)(y >= fmaf(s, kLmThreshold, z));
}

// exp2 that maps a -inf difference to 0 (empty partials carry m = -inf)
__device__ __forceinline__ float exp2_or_zero(float m, float ref) {
  return (m == -INFINITY) ? 0.0f : exp2f(m - ref);
}

// ---------------------------------------------------------------------------
// decode plan: splits and workspace layout (host and device agree on it)
// ---------------------------------------------------------------------------
struct DecodePlan {
  int hist_pages;    // ceil(max_hist_len / 64)
  int splits;        // history splits per (request, KV head)
  int pages_per_split;
  int chunks;        // BF16 64-token chunks per (request, KV head)
  int sink_chunks;   // the first sink_chunks chunks cover the sink window
  size_t off_qdig, off_qa, off_qb, off_hpart, off_bpart, total;
};

#ifndef OSCAR_RESIDENT_BLOCKS
#define OSCAR_RESIDENT_BLOCKS 512
#endif
// Blocks of the scan launch that are resident at once on MI355X (256 CUs,
// two 4-wave scan blocks per CU).  The split policy sizes the history splits
// so that history and BF16 blocks together fill them in one round: every wave
// then pays the latency of its first page once, and no second round of
// blocks runs on a partly idle chip.  Scan variants that fit one block per
// CU (scan_resident_blocks) plan with half as many.
constexpr int kResidentBlocks = OSCAR_RESIDENT_BLOCKS;
#ifndef OSCAR_SCAN_WAVES_PER_SIMD
#define OSCAR_SCAN_WAVES_PER_SIMD 2
#endif
// the most scan blocks any variant keeps resident (kResidentBlocks counts two
// per CU; a variant holds at most OSCAR_SCAN_WAVES_PER_SIMD): the workspace
// query plans with it, so its splits and workspace bound every launch's
constexpr long kMaxResidentBlocks = (long)kResidentBlocks * OSCAR_SCAN_WAVES_PER_SIMD / 2;
// at most 64 pages per wave (one page id per lane), which also bounds the
// rounding of the fp32 PV sums a wave accumulates
constexpr int kMaxPagesPerSplit = 4 * 64;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// (scale, zero) groups per head of a demotion kind's group flag (oscar.h)
constexpr int kGroupFlags = OSCAR_GROUPS_64 | OSCAR_GROUPS_32;
__host__ __device__ constexpr int kind_groups(int kind, int d) {
  return (kind & OSCAR_GROUPS_32) ? d / 32 : (kind & OSCAR_GROUPS_64) ? d / 64 : 1;
}
// the in-page code layout of a kind: K planes or V byte columns
__host__ __device__ constexpr bool kind_is_k(int kind) {
  return (kind & ~(OSCAR_CODEBOOK_LLOYD_MAX | kGroupFlags)) == OSCAR_KIND_K;
}

// One head's partial softmax state in the workspace: (m, l, two pad floats,
// acc[d]).  The pad puts acc on a 16-byte boundary for vector loads.
constexpr int kPartAcc = 4;
__host__ __device__ constexpr int part_row(int d) { return d + kPartAcc; }

// Shared-prefix cascade blocks read each page of a split for up to 16 requests
// with every wave covering the whole split, one page id per lane: their splits
// hold at most 64 pages.
constexpr int kCascadeMaxPagesPerSplit = 64;

// Partials of a head the per-unit merge requests in one round.
constexpr int kUnitRound = 16;

// Splits a launch that reads its shared prefix in packs of four requests takes
// at least: enough that the pack blocks of the prefix splits alone come near
// the resident blocks, so the packed waves, the longest of the launch, spread
// over every compute unit and end together; at most as many as keep every
// head's partials (history splits and BF16 chunks) within one merge round.
inline long pack_min_splits(int B, int n_kv, int chunks, long resident) {
  const long units = (long)(B / 4) * n_kv;   // pack blocks per prefix split
  if (units <= 0) return 0;
  const long want = (resident + units - 1) / units, cap = kUnitRound - chunks;
  return want < cap ? want : cap;
}

// resident: scan blocks resident at once; max_pps: pages per split at most;
// quad_prefix: the launch packs a shared prefix four requests at a time.  The
// workspace query plans with the largest count, the smallest cap and packing
// that any launch of these sizes can use, so its splits and workspace bound
// every other plan's.
inline DecodePlan make_decode_plan(int B, int Hq, int n_kv, int d, int max_hist_len, int sink_cap,
                                   int recent_cap, long resident = kMaxResidentBlocks,
                                   int max_pps = kMaxPagesPerSplit, bool quad_prefix = false) {
  DecodePlan p{};
  const int G = Hq / n_kv;
  const int NB = (G + 3) / 4;
  p.hist_pages = (max_hist_len + kPage - 1) / kPage;
  p.sink_chunks = (sink_cap + kPage - 1) / kPage;
  p.chunks = p.sink_chunks + (recent_cap + kPage - 1) / kPage;
  if (p.hist_pages > 0) {
    const long units = (long)(B > 0 ? B : 1) * n_kv;
    long target = resident - units * p.chunks;   // blocks left for history (one BF16 block per chunk)
    if (target < units) target = units;
    long s0 = (target + units - 1) / units;
    const long s_min = (p.hist_pages + max_pps - 1) / max_pps;
    if (s0 < s_min) s0 = s_min;
    if (quad_prefix) {
      const long s_pack = pack_min_splits(B, n_kv, p.chunks, resident);
      if (s0 < s_pack) s0 = s_pack;
    }
    if (s0 > p.hist_pages) s0 = p.hist_pages;
    p.pages_per_split = (int)((p.hist_pages + s0 - 1) / s0);
    p.splits = (p.hist_pages + p.pages_per_split - 1) / p.pages_per_split;
  }
  const size_t part = (size_t)G * part_row(d) * sizeof(float);
  size_t off = 0;
  p.off_qdig = off;  off = align256(off + (size_t)B * n_kv * NB * (d / 64) * 64 * 16);
  p.off_qa = off;    off = align256(off + (size_t)B * Hq * sizeof(float));
  p.off_qb = off;    off = align256(off + (size_t)B * Hq * 4 * sizeof(float));   // per quarter of the head
  p.off_hpart = off; off = align256(off + (size_t)B * n_kv * p.splits * part);
  p.off_bpart = off; off = align256(off + (size_t)B * n_kv * p.chunks * part);
  p.total = off;
  return p;
}

struct Bf16Plan {
  int ctx_pages, splits, pages_per_split;
  size_t off_part, total;
};

inline Bf16Plan make_bf16_plan(int B, int Hq, int n_kv, int d, int max_ctx_len) {
  Bf16Plan p{};
  const int G = Hq / n_kv;
  p.ctx_pages = (max_ctx_len + kPage - 1) / kPage;
  if (p.ctx_pages > 0) {
    const long units = (long)(B > 0 ? B : 1) * n_kv;
    long s0 = (kResidentBlocks + units - 1) / units;
    if (s0 < 1) s0 = 1;
    if (s0 > p.ctx_pages) s0 = p.ctx_pages;
    p.pages_per_split = (int)((p.ctx_pages + s0 - 1) / s0);
    p.splits = (p.ctx_pages + p.pages_per_split - 1) / p.pages_per_split;
  }
  p.off_part = 0;
  p.total = align256((size_t)B * n_kv * p.splits * G * part_row(d) * sizeof(float));
  return p;
}

// ---------------------------------------------------------------------------
// launchers (defined in quantize.hip / decode.hip); arguments already validated
// ---------------------------------------------------------------------------
hipError_t launch_quantize_pack(int kind, const uint16_t* x, int64_t n_src, int64_t tok_stride,
                                int64_t head_stride, const int32_t* src_idx, int64_t n_tok, int n_kv,
                                int d, const float* rot, float clip, const int32_t* dst_slot,
                                uint8_t* codes, uint16_t* scale_zero, int64_t n_pages,
                                hipStream_t stream);

// decode phases: rotate the query, scan history and BF16 windows, merge
constexpr int kPhaseRotate = 0, kPhaseScan = 1, kPhaseMerge = 2;
// demote_k / demote_v (or NULL): a decode step's demotions, run in the merge phase
hipError_t launch_decode_phase(int phase, const oscar_decode_args& a, const DecodePlan& plan, char* ws,
                               hipStream_t stream, const oscar_demote_args* demote_k = nullptr,
                               const oscar_demote_args* demote_v = nullptr);

hipError_t launch_decode_bf16(const oscar_bf16_decode_args& a, const Bf16Plan& plan, char* ws,
                              hipStream_t stream);

// scan blocks of the variant these (validated) args launch that are resident at
// once: kResidentBlocks scaled by its blocks per compute unit (two or one)
long scan_resident_blocks(const oscar_decode_args& a);

// Whether a launch reads its declared shared prefix in packs of four requests
// (else two): group size 4, head_dim 128, the uniform codebook, whole-head
// groups and four or more requests.
inline bool quad_packs(const oscar_decode_args& a) {
  return a.batch >= 4 && a.n_kv_heads > 0 && a.n_q_heads == 4 * a.n_kv_heads && a.head_dim == 128 &&
         a.codebook == OSCAR_CODEBOOK_UNIFORM && (a.group_channels == 0 || a.group_channels >= a.head_dim);
}

// Whether a launch with these (validated) args reads its shared prefix in
// cascade blocks, and whether any launch of these sizes can (the workspace
// query's bound): group size 4, head_dim 128, 16 or more requests; the launch
// also needs the caller's request, the uniform codebook, whole-head groups and
// a declared prefix of at least one cascade split.
inline bool cascade_sizes(int batch, int n_q_heads, int n_kv_heads, int head_dim) {
  return n_kv_heads > 0 && n_q_heads == 4 * n_kv_heads && head_dim == 128 && batch >= 16;
}
// the plan of the workspace query: the most splits any launch of these sizes can use
inline DecodePlan sizing_plan(int B, int Hq, int n_kv, int d, int max_hist_len, int sink_cap, int recent_cap) {
  const bool quad_sizes = B >= 4 && n_kv > 0 && Hq == 4 * n_kv && d == 128;
  return make_decode_plan(B, Hq, n_kv, d, max_hist_len, sink_cap, recent_cap, kMaxResidentBlocks,
                          cascade_sizes(B, Hq, n_kv, d) ? kCascadeMaxPagesPerSplit : kMaxPagesPerSplit, quad_sizes);
}
inline bool decode_cascade(const oscar_decode_args& a) {
  return a.prefix_cascade == 1 && cascade_sizes(a.batch, a.n_q_heads, a.n_kv_heads, a.head_dim) &&
         a.codebook == OSCAR_CODEBOOK_UNIFORM &&
         (a.group_channels == 0 || a.group_channels >= a.head_dim) && a.shared_pages >= kCascadeMaxPagesPerSplit;
}

}  // namespace oscar

// C ABI of liboscar: argument validation (host only, before any HIP call),
// workspace sizing and dispatch to the kernel launchers.
#include <atomic>
#include <cmath>
#include <mutex>

#include "common.hpp"

using namespace oscar;

namespace {

constexpr int kMaxCap = 4096;

bool supported_dim(int d) { return d == 64 || d == 128; }
bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

oscar_status hip_status(hipError_t e) { return e == hipSuccess ? OSCAR_OK : OSCAR_EHIP; }

// shape checks shared by the decode workspace query and the decode call
oscar_status check_decode_shape(int32_t B, int32_t Hq, int32_t n_kv, int32_t d, int32_t max_hist_len,
                                int32_t sink_cap, int32_t recent_cap) {
  if (B < 0 || B > 65535 || n_kv < 1 || n_kv > 65535 || Hq < 1 || Hq % n_kv) return OSCAR_EINVAL;
  if (max_hist_len < 0 || sink_cap < 0 || sink_cap > kMaxCap || recent_cap < 0 || recent_cap > kMaxCap)
    return OSCAR_EINVAL;
  if (!supported_dim(d) || !supported_group(Hq / n_kv)) return OSCAR_EUNSUPPORTED;
  if ((int64_t)B * Hq > (int64_t)0x7fffffff) return OSCAR_EINVAL;
  return OSCAR_OK;
}

}  // namespace

extern "C" {

int oscar_abi_version(void) { return OSCAR_ABI_VERSION; }

const char* oscar_status_str(int status) {
  switch (status) {
    case OSCAR_OK: return "ok";
    case OSCAR_EINVAL: return "invalid argument";
    case OSCAR_EUNSUPPORTED: return "unsupported shape (head_dim must be 64 or 128; query heads per KV head 1, 2, 4, 8 or 16)";
    case OSCAR_EWORKSPACE: return "workspace missing, misaligned or smaller than the size query returned";
    case OSCAR_EHIP: return "HIP runtime error";
    case OSCAR_ESCRATCH:
      return "the decode needs more scratch than the static buffer of oscar_decode_step_static holds "
             "(OSCAR_STATIC_SCRATCH_BYTES); call oscar_decode_step with a workspace";
    default: return "unknown status";
  }
}

oscar_status oscar_quantize_pack(int32_t kind, const uint16_t* x, int64_t n_src, int64_t x_tok_stride,
                                 int64_t x_head_stride, const int32_t* src_idx, int64_t n_tok,
                                 int32_t n_kv, int32_t head_dim, const float* rot, float clip,
                                 const int32_t* dst_slot, uint8_t* codes, uint16_t* scale_zero,
                                 int64_t n_pages, hipStream_t stream) {
  const int32_t layout = kind & ~(OSCAR_CODEBOOK_LLOYD_MAX | kGroupFlags);
  if (layout != OSCAR_KIND_K && layout != OSCAR_KIND_V) return OSCAR_EINVAL;
  if ((kind & kGroupFlags) == kGroupFlags) return OSCAR_EINVAL;
  if (n_tok < 0 || n_src < 0 || n_pages < 0 || n_kv < 1 || n_kv > 65535) return OSCAR_EINVAL;
  if (!supported_dim(head_dim)) return OSCAR_EUNSUPPORTED;
  if (!std::isfinite(clip) || !(clip > 0.0f) || clip > 65504.0f) return OSCAR_EINVAL;
  if (x_tok_stride < 0 || x_head_stride < 0) return OSCAR_EINVAL;
  if (n_tok > (int64_t)0x7fffffff * 16) return OSCAR_EINVAL;
  if (n_pages > ((int64_t)1 << 40)) return OSCAR_EINVAL;
  if (n_tok == 0) return OSCAR_OK;
  if (!x || !rot || !dst_slot || !codes || !scale_zero) return OSCAR_EINVAL;
  return hip_status(launch_quantize_pack(kind, x, n_src, x_tok_stride, x_head_stride, src_idx, n_tok,
                                         n_kv, head_dim, rot, clip, dst_slot, codes, scale_zero,
                                         n_pages, stream));
}

size_t oscar_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t head_dim, int32_t max_hist_len, int32_t sink_cap,
                                    int32_t recent_cap) {
  if (check_decode_shape(batch, n_q_heads, n_kv_heads, head_dim, max_hist_len, sink_cap, recent_cap) !=
      OSCAR_OK)
    return 0;
  return sizing_plan(batch, n_q_heads, n_kv_heads, head_dim, max_hist_len, sink_cap, recent_cap).total;
}

}  // extern "C"

namespace {
// Validate decode arguments and workspace; on success fill the plan.
oscar_status check_decode(const oscar_decode_args* a, void* workspace, size_t workspace_bytes,
                          DecodePlan* plan) {
  if (!a) return OSCAR_EINVAL;
  oscar_status st = check_decode_shape(a->batch, a->n_q_heads, a->n_kv_heads, a->head_dim,
                                       a->max_hist_len, a->sink_cap, a->recent_cap);
  if (st != OSCAR_OK) return st;
  if (!std::isfinite(a->sm_scale) || !(a->sm_scale > 0.0f)) return OSCAR_EINVAL;
  if (a->shared_pages < 0 || (int64_t)a->shared_pages * OSCAR_PAGE_TOKENS > a->max_hist_len)
    return OSCAR_EINVAL;
  if (a->codebook != OSCAR_CODEBOOK_UNIFORM && a->codebook != OSCAR_CODEBOOK_LLOYD_MAX) return OSCAR_EINVAL;
  if (a->group_channels != 0 && a->group_channels != 64 && a->group_channels != 32) return OSCAR_EINVAL;
  if (a->prefix_cascade != 0 && a->prefix_cascade != 1) return OSCAR_EINVAL;
  *plan = make_decode_plan(a->batch, a->n_q_heads, a->n_kv_heads, a->head_dim, a->max_hist_len,
                           a->sink_cap, a->recent_cap, scan_resident_blocks(*a),
                           decode_cascade(*a) ? kCascadeMaxPagesPerSplit : kMaxPagesPerSplit,
                           quad_packs(*a) && a->shared_pages > 0 && !decode_cascade(*a));
  if (a->batch == 0) return OSCAR_OK;
  if (!a->q || !a->out || !a->sink_len || !a->recent_len || !a->hist_len) return OSCAR_EINVAL;
  if (a->sink_cap > 0 && (!a->sink_k || !a->sink_v)) return OSCAR_EINVAL;
  if (a->recent_cap > 0 && (!a->recent_k || !a->recent_v)) return OSCAR_EINVAL;
  if (a->max_hist_len > 0) {
    if (!a->k_codes || !a->v_codes || !a->k_sz || !a->v_sz || !a->block_table || !a->r_k || !a->r_v)
      return OSCAR_EINVAL;
    if (a->n_pages < 1 || a->n_pages > ((int64_t)1 << 40) || a->max_pages < 1) return OSCAR_EINVAL;
    if ((int64_t)a->max_pages * OSCAR_PAGE_TOKENS < a->max_hist_len) return OSCAR_EINVAL;
  }
  if (plan->total > 0 &&
      (!workspace || workspace_bytes < plan->total || (reinterpret_cast<uintptr_t>(workspace) & 255)))
    return OSCAR_EWORKSPACE;
  return OSCAR_OK;
}

oscar_status check_demote(const oscar_demote_args* d, int32_t n_kv) {
  if (!d || d->n_tok == 0) return OSCAR_OK;
  if (d->n_tok < 0 || d->n_tok > ((int64_t)1 << 24) / n_kv) return OSCAR_EINVAL;
  if (d->n_src < 0 || d->x_tok_stride < 0 || d->x_head_stride < 0) return OSCAR_EINVAL;
  if (d->n_pages < 0 || d->n_pages > ((int64_t)1 << 40)) return OSCAR_EINVAL;
  if (!std::isfinite(d->clip) || !(d->clip > 0.0f) || d->clip > 65504.0f) return OSCAR_EINVAL;
  if (!d->x || !d->rot || !d->dst_slot || !d->codes || !d->scale_zero) return OSCAR_EINVAL;
  return OSCAR_OK;
}

// Static scratch of oscar_decode_step_static: one copy per GPU in the code
// object's device memory.  In host code `scratch` is only a symbol handle;
// the buffer's address on a device comes from hipGetSymbolAddress, looked up
// once per device (with that device current) and kept in scratch_ptr.
__device__ __attribute__((aligned(256))) uint8_t scratch[OSCAR_STATIC_SCRATCH_BYTES];
constexpr int kMaxDevices = 256;
std::atomic<void*> scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

oscar_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return OSCAR_EHIP;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return OSCAR_EHIP;
      scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return OSCAR_OK;
}

oscar_status run_phases(const oscar_decode_args* a, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, int first, int last, const oscar_demote_args* dk = nullptr,
                        const oscar_demote_args* dv = nullptr, bool use_static = false) {
  DecodePlan plan;
  oscar_status st;
  if (use_static) {
    // every check first (the workspace one with a stand-in address), then the
    // scratch address, the one HIP call before the launches
    if (!a) return OSCAR_EINVAL;
    if (check_decode_shape(a->batch, a->n_q_heads, a->n_kv_heads, a->head_dim, a->max_hist_len, a->sink_cap,
                           a->recent_cap) == OSCAR_OK &&
        sizing_plan(a->batch, a->n_q_heads, a->n_kv_heads, a->head_dim, a->max_hist_len, a->sink_cap,
                    a->recent_cap).total > OSCAR_STATIC_SCRATCH_BYTES)
      return OSCAR_ESCRATCH;
    st = check_decode(a, reinterpret_cast<void*>(uintptr_t(256)), OSCAR_STATIC_SCRATCH_BYTES, &plan);
  } else {
    st = check_decode(a, workspace, workspace_bytes, &plan);
  }
  if (st != OSCAR_OK) return st;
  if ((st = check_demote(dk, a->n_kv_heads)) != OSCAR_OK || (st = check_demote(dv, a->n_kv_heads)) != OSCAR_OK)
    return st;
  if (use_static && (st = static_scratch(&workspace)) != OSCAR_OK) return st;
  const bool demote = (dk && dk->n_tok > 0) || (dv && dv->n_tok > 0);
  if (a->batch == 0 && !demote) return OSCAR_OK;
  for (int ph = first; ph <= last; ++ph) {
    const hipError_t e = launch_decode_phase(ph, *a, plan, static_cast<char*>(workspace), stream, dk, dv);
    if (e != hipSuccess) return OSCAR_EHIP;
  }
  return OSCAR_OK;
}
}  // namespace

extern "C" {

oscar_status oscar_decode_attn(const oscar_decode_args* a, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return run_phases(a, workspace, workspace_bytes, stream, kPhaseRotate, kPhaseMerge);
}

oscar_status oscar_decode_step(const oscar_decode_args* a, const oscar_demote_args* demote_k,
                               const oscar_demote_args* demote_v, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return run_phases(a, workspace, workspace_bytes, stream, kPhaseRotate, kPhaseMerge, demote_k, demote_v);
}

oscar_status oscar_decode_step_static(const oscar_decode_args* a, const oscar_demote_args* demote_k,
                                      const oscar_demote_args* demote_v, hipStream_t stream) {
  return run_phases(a, nullptr, 0, stream, kPhaseRotate, kPhaseMerge, demote_k, demote_v, true);
}

oscar_status oscar_decode_rotate_query(const oscar_decode_args* a, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  return run_phases(a, workspace, workspace_bytes, stream, kPhaseRotate, kPhaseRotate);
}

oscar_status oscar_decode_scan(const oscar_decode_args* a, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return run_phases(a, workspace, workspace_bytes, stream, kPhaseScan, kPhaseScan);
}

oscar_status oscar_decode_merge(const oscar_decode_args* a, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  return run_phases(a, workspace, workspace_bytes, stream, kPhaseMerge, kPhaseMerge);
}

size_t oscar_decode_bf16_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                         int32_t head_dim, int32_t max_ctx_len) {
  if (check_decode_shape(batch, n_q_heads, n_kv_heads, head_dim, max_ctx_len, 0, 0) != OSCAR_OK) return 0;
  return make_bf16_plan(batch, n_q_heads, n_kv_heads, head_dim, max_ctx_len).total;
}

oscar_status oscar_decode_attn_bf16(const oscar_bf16_decode_args* a, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  if (!a) return OSCAR_EINVAL;
  oscar_status st = check_decode_shape(a->batch, a->n_q_heads, a->n_kv_heads, a->head_dim,
                                       a->max_ctx_len, 0, 0);
  if (st != OSCAR_OK) return st;
  if (!std::isfinite(a->sm_scale) || !(a->sm_scale > 0.0f)) return OSCAR_EINVAL;
  if (a->batch == 0) return OSCAR_OK;
  if (!a->q || !a->out || !a->ctx_len) return OSCAR_EINVAL;
  if (a->max_ctx_len > 0) {
    if (!a->k_pages || !a->v_pages || !a->block_table) return OSCAR_EINVAL;
    if (a->n_pages < 1 || a->max_pages < 1 ||
        (int64_t)a->max_pages * OSCAR_PAGE_TOKENS < a->max_ctx_len)
      return OSCAR_EINVAL;
  }
  const Bf16Plan plan = make_bf16_plan(a->batch, a->n_q_heads, a->n_kv_heads, a->head_dim, a->max_ctx_len);
  if (plan.total > 0 &&
      (!workspace || workspace_bytes < plan.total || (reinterpret_cast<uintptr_t>(workspace) & 255)))
    return OSCAR_EWORKSPACE;
  return hip_status(launch_decode_bf16(*a, plan, static_cast<char*>(workspace), stream));
}

}  // extern "C"

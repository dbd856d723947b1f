/*
 * oscar.h - C ABI of liboscar: INT2 three-segment decode attention and the
 * INT2 demotion (rotate -> clip -> quantise -> pack) kernel, for AMD gfx950.
 *
 * Method sources (cited by page title and section):
 *  - gist.science, "OSCAR: Offline Spectral Covariance-Aware Rotation for
 *    2-bit KV Cache Quantization", technical summary section 2.2A (fixed
 *    per-head rotations R_K = U_Q H P_br, R_V = U_S H P_br and per-layer clip
 *    thresholds, computed offline) and section 2.2B (paged hybrid-precision
 *    cache; INT2 history is unpacked, dequantised and inverse-rotated inside
 *    the attention kernel).
 *  - myzaker.com article on OSCAR, serving-pipeline paragraphs: a token pool
 *    of BF16 sink (64 tokens) | INT2 history | BF16 recent (256 tokens); the
 *    oldest recent token is rotated, clipped, quantised and packed (four
 *    2-bit values per byte) into history; decode runs an INT2 part (unpack,
 *    scale/zero-point dequantisation, float accumulation) and a BF16 part
 *    and merges them with an online softmax.
 *
 * Conventions shared by every entry point:
 *  - Pointers named in a signature are DEVICE pointers owned by the caller,
 *    unless documented as host.  The library allocates, frees and
 *    synchronises nothing.  It keeps no mutable global state, except the
 *    static per-device scratch buffer of oscar_decode_step_static.  Work is
 *    enqueued on `stream` (NULL = the default stream); results are valid
 *    after the caller synchronises that stream.
 *  - All argument checks run on the host BEFORE any HIP call.  A failed
 *    check returns OSCAR_EINVAL / OSCAR_EUNSUPPORTED / OSCAR_EWORKSPACE
 *    and enqueues nothing.  A kernel launch failure returns OSCAR_EHIP.
 *  - Rotations use row vectors: a rotated vector is y = x R; its inverse is
 *    x = y R^T.  R is fp32 [n_kv][d][d] row-major, one matrix per KV head.
 *  - bf16 and fp16 values are passed as their 16-bit patterns.
 *  - Pages hold 64 tokens.  One (page, KV head) block of an INT2 pool is:
 *      K codes : d/4*64 bytes in 4 planes.  Plane p (p = 0..3) holds bytes
 *                [p*d/16, (p+1)*d/16) of every token's code row, token-major:
 *                byte i of token o is at (i/(d/16))*64*(d/16) + o*(d/16) + i%(d/16).
 *      V codes : byte-column-major: byte i of token o is at i*64 + o.
 *      A token's code row has d/4 bytes; byte i holds rotated channels
 *      4i..4i+3, channel 4i+j in bits 2j..2j+1.
 *      scale/zero: fp16 pairs (scale, zero) per token: [64][2].
 *    Pools: codes uint8 [n_pages][n_kv][64*d/4]; scale_zero uint16
 *    [n_pages][n_kv][64][2].  A K pool and a V pool are separate buffers.
 *  - Dequantisation of a code c is zero + c*scale (rotated space) with the
 *    default codebook, zero + L[c]*scale with the Lloyd-Max one (below).
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OSCAR_ABI_VERSION 5
#define OSCAR_PAGE_TOKENS 64

#ifndef OSCAR_API
#define OSCAR_API __attribute__((visibility("default")))
#endif

typedef enum oscar_status {
  OSCAR_OK = 0,
  OSCAR_EINVAL = 1,        /* a pointer, size or scalar argument is invalid */
  OSCAR_EUNSUPPORTED = 2,  /* a valid shape this build has no kernel for   */
  OSCAR_EWORKSPACE = 3,    /* workspace missing, misaligned or too small    */
  OSCAR_EHIP = 4,          /* the HIP runtime reported an error             */
  OSCAR_ESCRATCH = 5       /* the call needs more than the static scratch
                              buffer of oscar_decode_step_static holds      */
} oscar_status;

typedef enum oscar_kind { OSCAR_KIND_K = 0, OSCAR_KIND_V = 1 } oscar_kind;

/* INT2 codebooks: how a 2-bit code c of a (token, head) group dequantises with
 * the group's fp16 (scale, zero), and how the demotion chooses them.
 *  UNIFORM    zero + c*scale; zero = fp16(min), scale = fp16((max - min)/3),
 *             c = rint((y - zero)/scale) clamped to [0, 3] (the pages' scale /
 *             zero-point quantiser).
 *  LLOYD_MAX  zero + L[c]*scale, L = (-10, -3, 3, 10): the 4-level quantiser
 *             with the least mean squared error for a Gaussian (levels at
 *             +-0.4528 and +-1.5104 deviations, here in the ratio 3:10).  The
 *             gist.science summary says the authors' code pairs a Lloyd-Max
 *             codebook with the rotation and gives no levels.  zero = fp16(fp32(mean)),
 *             scale = fp16(fp32(0.15104 * deviation)), mean and population
 *             deviation of the clipped group in fp64; c = the number of
 *             thresholds fp32(zero + scale*t), t in (-6.5, 0, 6.5), that y reaches.
 * The pools of a layer hold one codebook; demotion and decode must agree. */
#define OSCAR_CODEBOOK_UNIFORM 0
#define OSCAR_CODEBOOK_LLOYD_MAX 0x100

/* Quantisation groups: by default one group is all head_dim channels of a
 * (token, head).  With 64-channel groups every block of 64 consecutive
 * channels has its own (scale, zero) (head_dim 128: two groups; head_dim 64:
 * one, the same as the default); with 32-channel groups every block of 32
 * (head_dim 128: four groups; head_dim 64: two).  Sub-head groups are where
 * the bit-reversal permutation of R balances the groups (gist.science
 * summary, section 2.2A; the myzaker.com article on OSCAR, its paragraph on
 * aligning the rotation with attention).  With ng
 * groups per head the scale/zero pool is [n_pages][n_kv][64*ng][2],
 * group-planar: group j of token o at j*64 + o.  At most one of the two flags
 * is OR'ed into a demotion's kind; the decode args carry the group size. */
#define OSCAR_GROUPS_64 0x200
#define OSCAR_GROUPS_32 0x400

/* ABI version of the loaded library (OSCAR_ABI_VERSION). */
OSCAR_API int oscar_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
OSCAR_API const char* oscar_status_str(int status);

/*
 * oscar_quantize_pack - demote tokens of ONE tensor (K or V) of one layer
 * into INT2 history pages.  Follows the demotion step of the serving pipeline
 * (myzaker.com article) with the rotation and clip threshold of the
 * gist.science technical summary, section 2.2A:
 *   y = x R (fp32, accumulated exactly and rounded once); y_c = clamp(y, -clip, clip);
 *   over the d channels of each (token, head): zero = fp16(min y_c),
 *   scale = fp16((max y_c - min y_c) / 3) (fp32 subtract and divide);
 *   code = clamp(rint((y_c - zero) / scale), 0, 3) in fp32, round half to
 *   even, all codes 0 when scale is 0 (the Lloyd-Max codebook replaces these
 *   three steps with its own, above); pack 4 codes per byte; write the code
 *   row and (scale, zero) into slot dst_slot = page*64 + offset.
 *
 *  kind          OSCAR_KIND_K or OSCAR_KIND_V (selects the in-page layout),
 *                optionally OR'ed with OSCAR_CODEBOOK_LLOYD_MAX and / or one of
 *                OSCAR_GROUPS_64, OSCAR_GROUPS_32 (then scale_zero holds 64*ng
 *                pairs per head, ng = head_dim/64 or head_dim/32); both group
 *                flags together: OSCAR_EINVAL
 *  x             bf16; element (token s, head g, channel c) is at
 *                x[s*x_tok_stride + g*x_head_stride + c]; the caller
 *                guarantees that address is valid for every s in [0, n_src)
 *  src_idx       int32 [n_tok] source token of each demoted token, or NULL
 *                for tokens 0..n_tok-1; entries outside [0, n_src) are skipped
 *  n_tok         tokens to demote (0 is a no-op)
 *  n_kv, head_dim  head_dim in {64, 128}; n_kv >= 1
 *  rot           fp32 [n_kv][head_dim][head_dim] (R_K or R_V)
 *  clip          per-layer threshold, finite, 0 < clip <= 65504 (host scalar)
 *  dst_slot      int32 [n_tok]; slots outside [0, n_pages*64) are skipped
 *  codes         uint8 pool [n_pages][n_kv][64*head_dim/4]
 *  scale_zero    uint16 pool [n_pages][n_kv][64*ng][2] (ng = 1 without a group flag)
 *  Two demoted tokens must not share a slot (the result would be unspecified).
 */
OSCAR_API oscar_status oscar_quantize_pack(int32_t kind, const uint16_t* x, int64_t n_src,
                                 int64_t x_tok_stride, int64_t x_head_stride,
                                 const int32_t* src_idx, int64_t n_tok, int32_t n_kv,
                                 int32_t head_dim, const float* rot, float clip,
                                 const int32_t* dst_slot, uint8_t* codes,
                                 uint16_t* scale_zero, int64_t n_pages, hipStream_t stream);

/*
 * Decode attention over a three-segment cache (one new query per request).
 * Context of request b, in order: sink tokens [0, sink_len[b]) (BF16,
 * unrotated), history tokens [0, hist_len[b]) (INT2, stored rotated; history
 * token t is in page block_table[b][t/64] at offset t%64), recent tokens
 * [0, recent_len[b]) (BF16, unrotated, any ring order).  Query head h uses KV
 * head h / (n_q_heads / n_kv_heads).  Every query attends to its whole
 * context: out = softmax(sm_scale * q.k) . v, with INT2 history keys and
 * values inverse-rotated (x = (zero + c*scale) R^T).  The rotation is applied
 * once per query head (q R_K before the history scan, accumulated values times
 * R_V^T after it).  The INT2 and BF16 parts merge through an online softmax.
 * A request whose segments are all empty gets a zero output row.  Device
 * lengths outside [0, cap] / [0, max_hist_len], or a block-table entry outside
 * [0, n_pages) for a used page, make that request's output rows NaN (no
 * out-of-bounds access happens).
 */
typedef struct oscar_decode_args {
  int32_t batch;            /* B >= 0 (0 is a no-op)                               */
  int32_t n_q_heads;        /* multiple of n_kv_heads; G = n_q_heads/n_kv_heads in {1,2,4,8,16} */
  int32_t n_kv_heads;       /* >= 1                                                */
  int32_t head_dim;         /* 64 or 128                                           */
  float sm_scale;           /* finite, > 0 (normally 1/sqrt(head_dim))             */
  const uint16_t* q;        /* bf16 [B][n_q_heads][head_dim]                       */
  const uint16_t* sink_k;   /* bf16 [B][n_kv][sink_cap][head_dim]                  */
  const uint16_t* sink_v;
  const uint16_t* recent_k; /* bf16 [B][n_kv][recent_cap][head_dim]                */
  const uint16_t* recent_v;
  int32_t sink_cap;         /* 0..4096 (64 in OSCAR)                               */
  int32_t recent_cap;       /* 0..4096 (256 in OSCAR)                              */
  const int32_t* sink_len;  /* int32 [B]                                           */
  const int32_t* recent_len;/* int32 [B]                                           */
  const int32_t* hist_len;  /* int32 [B]                                           */
  int32_t max_hist_len;     /* host upper bound on hist_len[b]; sizes the grid     */
  const uint8_t* k_codes;   /* INT2 K pool (layout above)                          */
  const uint8_t* v_codes;   /* INT2 V pool                                         */
  const uint16_t* k_sz;     /* fp16 (scale, zero) pools                            */
  const uint16_t* v_sz;
  int64_t n_pages;          /* pages in each pool                                  */
  const int32_t* block_table; /* int32 [B][max_pages]                              */
  int32_t max_pages;        /* >= ceil(max_hist_len/64)                            */
  const float* r_k;         /* fp32 [n_kv][d][d], the R used to quantise K         */
  const float* r_v;         /* fp32 [n_kv][d][d], the R used to quantise V         */
  float* out;               /* fp32 [B][n_q_heads][head_dim]                       */
  int32_t shared_pages;     /* 0, or the length in pages of a history prefix that every
                               request holds at the same physical pages: block_table[b][i]
                               is one id for all b when i < shared_pages, and every
                               hist_len[b] >= 64*shared_pages (0 <= shared_pages and
                               64*shared_pages <= max_hist_len).  A prefix cache makes such
                               tables.  With n_q_heads/n_kv_heads = 4 the scan then reads
                               the history splits that lie inside the prefix once for each
                               pack of requests: four (4i .. 4i+3; uniform codebook,
                               whole-head groups, head_dim 128, batch >= 4) or two (2i,
                               2i+1) per pack.  Other group sizes ignore it.  The scan
                               checks the pages it reads for every request of a pack (of
                               a cascade group, below): if a row's ids differ there from
                               the others', or a history ends before them, every output
                               row of that pack (group) is NaN.                         */
  int32_t codebook;         /* OSCAR_CODEBOOK_UNIFORM or OSCAR_CODEBOOK_LLOYD_MAX: the
                               codebook the pools were demoted with (a decode step also
                               demotes with it)                                        */
  int32_t group_channels;   /* 0 (a group is the whole head), 64 (OSCAR_GROUPS_64 pools)
                               or 32 (OSCAR_GROUPS_32 pools); a decode step demotes with
                               the same groups                                         */
  int32_t prefix_cascade;   /* 0 or 1 (else OSCAR_EINVAL).  1: where the packs above
                               apply with four requests, batch >= 16 and shared_pages >=
                               64, the splits inside the prefix run as cascade blocks
                               instead: each page of such a split is read once for a
                               group of up to four packs (requests 16i .. 16i+15), whose
                               rows the block's four waves score from that one copy
                               (splits of at most 64 pages).  Ignored elsewhere.  Same
                               results as 0 up to rounding order; it cuts the page reads
                               of the prefix by up to four but makes more history splits
                               for the merge to combine.                                */
} oscar_decode_args;

/* Workspace bytes oscar_decode_attn needs for these sizes (0 on invalid sizes).
 * Depends only on its arguments, so results do not depend on the device. */
OSCAR_API size_t oscar_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t head_dim, int32_t max_hist_len, int32_t sink_cap,
                                    int32_t recent_cap);

/* Enqueue decode attention.  workspace: device buffer of at least
 * oscar_decode_workspace_bytes(...) bytes, 256-byte aligned; its contents on
 * entry do not matter and are overwritten. */
OSCAR_API oscar_status oscar_decode_attn(const oscar_decode_args* args, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * The three phases oscar_decode_attn runs, in this order, on one stream; a
 * caller may enqueue them separately (to time or overlap a phase).  The
 * workspace carries the state between phases, so the same args and
 * workspace must be passed to all three.
 *   oscar_decode_rotate_query  q_rot = q R_K (and its channel sum) per query head
 *   oscar_decode_scan          INT2 history split-K scan and BF16 sink/recent
 *                              tiles; one online-softmax partial per history
 *                              split and per BF16 block (a 64-token tile, or
 *                              all of a (request, KV head)'s tiles when the
 *                              call has 128 or more of those)
 *   oscar_decode_merge         log-sum-exp merge of the history partials, times
 *                              R_V^T, merge with the BF16 partials, normalise
 *                              (one block per query head, or per (request, KV
 *                              head) when each head has at most 16 partials, or
 *                              at most 64 with 128 or more (request, KV head)s)
 * Same validation and status codes as oscar_decode_attn.
 */
OSCAR_API oscar_status oscar_decode_rotate_query(const oscar_decode_args* args, void* workspace,
                                                 size_t workspace_bytes, hipStream_t stream);
OSCAR_API oscar_status oscar_decode_scan(const oscar_decode_args* args, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);
OSCAR_API oscar_status oscar_decode_merge(const oscar_decode_args* args, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream);

/*
 * One tensor's demotion inside a decode step: the arguments of
 * oscar_quantize_pack except kind, n_kv and head_dim (taken from the step:
 * demote_k is K and demote_v is V, both with the step's args->codebook and
 * args->group_channels).
 * n_tok in [0, 2^24 / n_kv]; the other rules are those of oscar_quantize_pack.
 */
typedef struct oscar_demote_args {
  const uint16_t* x;          /* bf16 source: element (s, g, c) at x[s*x_tok_stride + g*x_head_stride + c] */
  int64_t n_src;
  int64_t x_tok_stride;
  int64_t x_head_stride;
  const int32_t* src_idx;     /* int32 [n_tok] or NULL */
  int64_t n_tok;
  const float* rot;           /* fp32 [n_kv][head_dim][head_dim] */
  float clip;
  const int32_t* dst_slot;    /* int32 [n_tok] */
  uint8_t* codes;             /* INT2 code pool */
  uint16_t* scale_zero;       /* fp16 (scale, zero) pool */
  int64_t n_pages;
} oscar_demote_args;

/*
 * One steady-state decode step (the serving pipeline of the myzaker.com
 * article on OSCAR): demote the step's K and V tokens into INT2 history and
 * run decode attention, with the demotions folded into the decode's last
 * launch (three launches in all instead of five).  demote_k / demote_v may
 * be NULL.  They may write into the pools this decode reads, but only into
 * slots the decode does not attend (at or past hist_len of their request): the
 * step attends the token it demotes in BF16 from the recent window, and the
 * caller's next step counts it in hist_len.  Otherwise the result is
 * unspecified.  Same workspace and status rules as oscar_decode_attn; with
 * batch 0 only the demotions run.
 */
OSCAR_API oscar_status oscar_decode_step(const oscar_decode_args* args, const oscar_demote_args* demote_k,
                                         const oscar_demote_args* demote_v, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/*
 * oscar_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, and serving loops
 * or harnesses that forbid hipMalloc.  The workspace lives in a static
 * device buffer of OSCAR_STATIC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends; its address on the current
 * device is looked up (hipGetSymbolAddress) on the first call there.
 * Arguments, results and the other status codes are those of
 * oscar_decode_step.  A call whose oscar_decode_workspace_bytes exceeds
 * OSCAR_STATIC_SCRATCH_BYTES returns OSCAR_ESCRATCH before any HIP call
 * (use oscar_decode_step with a workspace then).  The call allocates and
 * frees nothing.  Every call on one GPU uses the same buffer: calls that
 * can overlap on one GPU (on different streams, or concurrent host threads
 * on one stream) race and must be serialised by the caller.  Nothing in
 * the buffer needs clearing between calls; each call writes what it reads.
 */
#define OSCAR_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
OSCAR_API oscar_status oscar_decode_step_static(const oscar_decode_args* args,
                                                const oscar_demote_args* demote_k,
                                                const oscar_demote_args* demote_v, hipStream_t stream);

/*
 * BF16 comparator: plain decode attention with the whole context held in
 * BF16 pages (no rotation, no quantisation), same GQA mapping and output
 * rules.  Used to measure the INT2 path against a BF16 cache of the same
 * shape.  Context token t of request b is in page block_table[b][t/64] at
 * offset t%64 of k_pages/v_pages bf16 [n_pages][n_kv][64][head_dim].
 */
typedef struct oscar_bf16_decode_args {
  int32_t batch, n_q_heads, n_kv_heads, head_dim;
  float sm_scale;
  const uint16_t* q;          /* bf16 [B][n_q_heads][head_dim] */
  const uint16_t* k_pages;    /* bf16 [n_pages][n_kv][64][head_dim] */
  const uint16_t* v_pages;
  int64_t n_pages;
  const int32_t* block_table; /* int32 [B][max_pages] */
  int32_t max_pages;
  const int32_t* ctx_len;     /* int32 [B], each in [0, max_ctx_len] */
  int32_t max_ctx_len;        /* host bound, <= max_pages*64 */
  float* out;                 /* fp32 [B][n_q_heads][head_dim] */
} oscar_bf16_decode_args;

OSCAR_API size_t oscar_decode_bf16_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                         int32_t head_dim, int32_t max_ctx_len);
OSCAR_API oscar_status oscar_decode_attn_bf16(const oscar_bf16_decode_args* args, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* OSCAR_H */

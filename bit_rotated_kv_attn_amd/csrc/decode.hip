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
// x_hat = zero + c*scale, a history logit is scale*(q_rot . c) + zero*sum(q_rot)
// and a history output is sum_t p_t*scale_t*c_t + sum_t p_t*zero_t.
//
// History scan on the matrix cores.  QK is exact integer arithmetic
// (v_mfma_i32_16x16x64_i8): the 2-bit codes become int8 operands by masking
// (no conversion; with the Lloyd-Max codebook a byte permute maps each code to
// its int8 level, and c reads L[c] above), and the rotated query becomes a
// 30-bit fixed-point integer split into four balanced 8-bit digits, one MFMA
// row per (head, digit), so 4 heads fill the 16 rows; a query element is
// exact to 2^-25 of the query's norm.  PV runs on the fp16 matrix cores with
// fp32 sums (v_mfma_f32_16x16x32_f16): each weight p*scale_V is an fp16 pair
// (high part, and the remainder scaled by 2^11), so it is held to 2^-21 of
// itself with no fixed-point floor, and the V codes enter as fp16 subnormal
// integers masked in place (c * 4^f * 2^-24, multiplied exactly).  The
// softmax reference maximum is only raised when a logit exceeds it by 2^12;
// the raise then rescales the fp32 sums.
// Launches (all on the caller's stream):
//   1. prepare_kernel       q_rot = q R_K[g] per query head -> MFMA digit
//                           operands
//   2. decode_main_kernel   one grid: INT2 history splits (those inside a
//                           declared shared prefix read once per pack of
//                           two or four requests, or on request once per
//                           group of up to four packs in cascade blocks),
//                           then the BF16 sink / recent chunks; each block
//                           writes an (m, l, acc) partial per head
//   3. merge_kernel         LSE merge of the history partials, * R_V^T, LSE merge
//      (merge_unit_kernel)  with the BF16 partials, normalise (one block per
//                           head, or per (request, KV head) in large batches);
//                           in a decode step also the step's K / V demotions
// Softmax state uses base-2 exponents (logits pre-scaled by log2 e).
#include "common.hpp"
#include "demote.hpp"

namespace oscar {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr uint32_t kMask0 = 0x03030303u;  // code field 0 of each byte (x1)
constexpr uint32_t kMask1 = 0x0C0C0C0Cu;  // field 1 (x4)
constexpr uint32_t kMask2 = 0x30303030u;  // field 2 (x16); field 3 is shifted into it
// Raise the reference maximum only when a logit passes it by 2^kLazyThr.
// On the long-context workloads about one page in a hundred then takes the
// rescale path; the fp32 PV sums make that path a multiply per sum.
constexpr float kLazyThr = 12.0f;
constexpr float kScaleSlack = 1.75f;      // rescale when a V scale exceeds 1.75x the running max
constexpr float kWeightTop = 16384.0f;    // 2^14: largest weight p*scale_V*kap the thresholds allow
constexpr float kFix = 1073741824.0f;     // 2^30: fixed-point range of the query digits
constexpr int kBf16WaveTokens = 16;       // tokens of a BF16 chunk per wave (4 waves per chunk)

struct DecodeDev {
  int B, Hq, n_kv, G, NB, sink_cap, recent_cap, max_hist_len, max_pages;
  // bf_blocks: BF16 blocks (and partials) per unit, each taking bf_cpb consecutive chunks
  int splits, pps, chunks, sink_chunks, bf_blocks, bf_cpb;
  // shared-prefix packing (G = 4 only): the first n_pref splits lie inside the
  // prefix and are read once for each of the `packs` packs of `pack` requests
  // (requests pack*i .. pack*i + pack - 1; pack = 2 or 4); the requests past the
  // last whole pack read them on their own
  int n_pref, packs, pack;
  // cascade (group size 4, four-request packs, 16 or more requests): the prefix
  // splits run as one block per (split, group of up to four packs, KV head),
  // each page staged once for the group; pack_units = groups, else packs
  int casc, pack_units;
  int lm;   // the pools hold Lloyd-Max codes (oscar.h OSCAR_CODEBOOK_LLOYD_MAX)
  int ng;   // (scale, zero) groups per head: 1, 2 (64-channel groups at d = 128, 32 at d = 64) or 4
  float sm_log2;
  int64_t n_pages;
  const uint16_t *q, *sink_k, *sink_v, *recent_k, *recent_v;
  const int32_t *sink_len, *recent_len, *hist_len, *block_table;
  const uint8_t *k_codes, *v_codes;
  const uint32_t *k_sz, *v_sz;
  const float *r_k, *r_v;
  float* out;
  uint8_t* qdig;     // [B][n_kv][NB][D/64][64 lanes][16 bytes] QK A operands
  float *qa, *qb;    // logit constants: qa [B][Hq] = sm_log2/(16 kq); qb [B][Hq][2] = sm_log2 * sum(q_rot)
                     // over channels 0..D/2-1 and D/2..D-1 (the two 64-channel groups when D = 128)
  float *hpart, *bpart;
};

struct DemoteDev {   // one tensor's demotion inside a decode step (n_tok = 0: none)
  const uint16_t* x;
  int64_t n_src, tok_stride, head_stride;
  const int32_t* src_idx;
  int64_t n_tok;
  const float* rot;
  float clip;
  const int32_t* dst_slot;
  uint8_t* codes;
  uint32_t* sz;
  int64_t n_pages;
};

DemoteDev make_demote(const oscar_demote_args* d) {
  DemoteDev m{};
  if (!d) return m;
  m.x = d->x;
  m.n_src = d->n_src;
  m.tok_stride = d->x_tok_stride;
  m.head_stride = d->x_head_stride;
  m.src_idx = d->src_idx;
  m.n_tok = d->n_tok;
  m.rot = d->rot;
  m.clip = d->clip;
  m.dst_slot = d->dst_slot;
  m.codes = d->codes;
  m.sz = reinterpret_cast<uint32_t*>(d->scale_zero);
  m.n_pages = d->n_pages;
  return m;
}

struct Bf16Dev {
  int B, Hq, n_kv, G, max_pages, max_ctx_len, splits, pps;
  float sm_log2;
  int64_t n_pages;
  const uint16_t *q, *k_pages, *v_pages;
  const int32_t *block_table, *ctx_len;
  float *out, *part;
};

// operand mask p of a raw code word: bytes hold field p of each byte (x1, x4, x16, x16)
__device__ __forceinline__ int code_mask(uint32_t w, int p) {
  return (int)(p == 0 ? (w & kMask0) : p == 1 ? (w & kMask1) : p == 2 ? (w & kMask2) : ((w >> 2) & kMask2));
}

// Lloyd-Max levels (-10, -3, 3, 10) as the int8 bytes of one word, indexed by the code
constexpr uint32_t kLmLevels = 0x0A03FDF6u;

// MFMA operand p of a raw code word: the uniform codebook masks field p in
// place (x1, x4, x16, x16); the Lloyd-Max one moves field p to the low bits of
// each byte and replaces the code by its level with a byte permute
template <bool LM>
__device__ __forceinline__ int code_operand(uint32_t w, int p) {
  if constexpr (LM) return (int)__builtin_amdgcn_perm(kLmLevels, kLmLevels, (w >> (2 * p)) & kMask0);
  else return code_mask(w, p);
}

// c + f * a and f * a, per component
__device__ __forceinline__ float4 f4_fma(float f, float4 a, float4 c) {
  return make_float4(fmaf(f, a.x, c.x), fmaf(f, a.y, c.y), fmaf(f, a.z, c.z), fmaf(f, a.w, c.w));
}

__device__ __forceinline__ float4 f4_scale(float f, float4 a) { return make_float4(f * a.x, f * a.y, f * a.z, f * a.w); }

// a value equal in every lane, moved to a scalar register
__device__ __forceinline__ float wave_uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// issue priority of the wave (0 lowest .. 3 highest; the level is wave-uniform)
__device__ __forceinline__ void set_wave_priority(int level) {
  switch (level) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

__device__ __forceinline__ uint32_t balanced_digits(uint32_t x) {  // x in [-2^30, 2^30] two's complement
  return (x + 0x80808080u) ^ 0x80808080u;
}

// ---------------------------------------------------------------------------
// BF16 tiles (sink / recent windows and the BF16 comparator): 64 tokens of one
// KV head.  QK runs on the matrix cores (v_mfma_f32_16x16x32_bf16: q and K are
// bf16 already, so products are exact and sums fp32); PV runs on the VALU in
// fp32 from a V tile staged in LDS.  All global loads of a tile are issued
// together (bf16_load) before any is used.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int D, int G>
struct WaveAcc {            // online-softmax state, replicated in every lane
  float m[G], l[G];
  float a[G][D / kWave];    // channels (D/64)*lane + k
};

template <int D, int G>
__device__ __forceinline__ void acc_init(WaveAcc<D, G>& s) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s.m[h] = -INFINITY;
    s.l[h] = 0.0f;
#pragma unroll
    for (int k = 0; k < D / kWave; ++k) s.a[h][k] = 0.0f;
  }
}

template <int D>
struct Bf16Tile {
  static constexpr int KK = D / 32;   // MFMA k-steps per token block
  static constexpr int VC = D / 8;    // 16-byte V chunks per lane
  uint4 k[4][KK];                     // B operands: token 16*tb + lane%16, channels 32kk + 8*(lane/16) ..+7
  uint4 v[VC];                        // V chunk lane + 64j of the [64][D] tile
};

// LDS bytes per wave for one BF16 tile: V tile, weights [64][G], reductions
template <int D, int G>
constexpr int bf16_lds_bytes() { return 32 * D * 2 + 64 * G * 4 + 3 * 16 * 4; }   // V staged 32 tokens at a time

// q rows of the G heads as MFMA A operands (rows >= G are zero)
template <int D, int G>
__device__ __forceinline__ void bf16_q_operands(bf16x8* qa, const uint16_t* __restrict__ qrows, int lane) {
  const int r = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const uint4 x = r < G ? *reinterpret_cast<const uint4*>(qrows + (size_t)r * D + 32 * kk + 8 * kg)
                          : make_uint4(0, 0, 0, 0);
    qa[kk] = __builtin_bit_cast(bf16x8, x);
  }
}

// a 16-byte load, non-temporal when STREAM: the sink and recent windows are
// read once per call, while the comparator's pages of a shared prefix are read
// for every request that holds them
template <bool STREAM>
__device__ __forceinline__ uint4 ld16(const uint16_t* ptr) {
  if constexpr (STREAM) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const uint4*>(ptr);
  }
}

// Tokens at or past nv are neither read nor used.
template <int D, bool STREAM>
__device__ __forceinline__ void bf16_load(Bf16Tile<D>& t, const uint16_t* __restrict__ kbase,
                                          const uint16_t* __restrict__ vbase, int nv, int lane) {
  const int r = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int tok = 16 * tb + r;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      t.k[tb][kk] = tok < nv ? ld16<STREAM>(kbase + (size_t)tok * D + 32 * kk + 8 * kg)
                             : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < D / 8; ++j) {
    const int ch = lane + kWave * j, tok = ch / (D / 8);
    t.v[j] = tok < nv ? ld16<STREAM>(vbase + (size_t)tok * D + 8 * (ch % (D / 8)))
                      : make_uint4(0, 0, 0, 0);
  }
}

template <int D, int G>
__device__ __forceinline__ void bf16_compute(WaveAcc<D, G>& st, const Bf16Tile<D>& t, const bf16x8* qa,
                                             float sm_log2, int nv, uint8_t* lds, int lane) {
  constexpr int CPL = D / kWave;
  uint16_t* vt = reinterpret_cast<uint16_t*>(lds);            // [32][D]: one half of the V tile
  float* w = reinterpret_cast<float*>(lds + 32 * D * 2);     // [64][G]
  float* red = w + 64 * G;                                    // [3][16]
  const int r = lane & 15, kg = lane >> 4;

  // QK: lane (r, kg) holds heads 4kg+i of token 16tb + r
  float lg[4][4], mloc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) mloc[i] = -INFINITY;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    v4f s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], __builtin_bit_cast(bf16x8, t.k[tb][kk]), s, 0, 0, 0);
    const bool ok = 16 * tb + r < nv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lg[tb][i] = ok ? sm_log2 * s[i] : -INFINITY;
      mloc[i] = fmaxf(mloc[i], lg[tb][i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mloc[i] = group16_max(mloc[i]);
    if (r == 0 && 4 * kg + i < G) red[4 * kg + i] = mloc[i];
  }
  __builtin_amdgcn_wave_barrier();
  float mnew[G], alpha[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mnew[h] = fmaxf(st.m[h], red[h]);
    alpha[h] = exp2_or_zero(st.m[h], mnew[h]);
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) red[16 + h] = mnew[h];
  }
  __builtin_amdgcn_wave_barrier();
  // weights p = exp2(logit - m) into w[token][head]; row sums per head
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * kg + i;
    if (4 * kg < G) {   // lane groups past the last head hold no rows
      const float m = red[16 + (h < G ? h : 0)];
      float ls = 0.0f;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const float pr = exp2_or_zero(lg[tb][i], m);
        ls += pr;
        if (h < G) w[(16 * tb + r) * G + h] = pr;
      }
      ls = group16_sum(ls);
      if (r == 0 && h < G) red[32 + h] = ls;
    }
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.l[h] = st.l[h] * alpha[h] + red[32 + h];
    st.m[h] = mnew[h];
#pragma unroll
    for (int k = 0; k < CPL; ++k) st.a[h][k] *= alpha[h];
  }
  // PV: lane holds channels CPL*lane .. CPL*lane + CPL-1; V chunks j < D/16
  // hold tokens 0..31, the rest tokens 32..63
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (32 * half >= nv) break;
#pragma unroll
    for (int j = 0; j < D / 16; ++j)
      *reinterpret_cast<uint4*>(vt + 8 * (lane + kWave * j)) = t.v[half * (D / 16) + j];
    __builtin_amdgcn_wave_barrier();
    const int tend = min(nv, 32 * half + 32);
#pragma unroll 4
    for (int tok = 32 * half; tok < tend; ++tok) {
      float v[CPL];
      const uint16_t* row = vt + (tok - 32 * half) * D;
      if constexpr (CPL == 2) {
        const uint32_t x = *reinterpret_cast<const uint32_t*>(row + 2 * lane);
        v[0] = bf16_to_f32(x & 0xffffu);
        v[1] = bf16_to_f32(x >> 16);
      } else {
        v[0] = bf16_to_f32(row[lane]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pr = w[tok * G + h];
#pragma unroll
        for (int k = 0; k < CPL; ++k) st.a[h][k] = fmaf(pr, v[k], st.a[h][k]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Wave state -> this wave's slot of the block merge area [G][D+2] = (m, l, acc).
template <int D, int G>
__device__ __forceinline__ void store_wave_state(const WaveAcc<D, G>& st, float* mw, int lane, bool poison) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (lane == 0) {
      mw[h * part_row(D)] = st.m[h];
      mw[h * part_row(D) + 1] = poison ? NAN : st.l[h];
    }
#pragma unroll
    for (int k = 0; k < D / kWave; ++k) mw[h * part_row(D) + kPartAcc + (D / kWave) * lane + k] = st.a[h][k];
  }
}

// Merge the 4 wave slots of a block (after a barrier; slot v starts at
// mrg + v*slot floats) into one partial.  kBlock/G threads serve each head, so
// a thread computes the four weights of its head once; every LDS read is
// issued before the first exponential.
// Heads h >= GH (a block that serves two requests) write to the next
// request's rows, ustride floats further on.
template <int G, int D, int GH = G>
__device__ __forceinline__ void combine_block(const float* mrg, int slot, const int* flags, float* dst, int tid,
                                              size_t ustride = 0) {
  constexpr int R = part_row(D), TPH = kBlock / G, IT = (R + TPH - 1) / TPH;
  const int h = tid / TPH, t = tid - h * TPH;
  if (h >= G) return;
  const bool bad = flags[0] | flags[1] | flags[2] | flags[3];
  const float* src = mrg + h * R;
  float m[4], x[IT][4];
#pragma unroll
  for (int v = 0; v < 4; ++v) m[v] = src[v * slot];
#pragma unroll
  for (int k = 0; k < IT; ++k) {
    const int r = min(t + TPH * k, R - 1);
#pragma unroll
    for (int v = 0; v < 4; ++v) x[k][v] = src[v * slot + r];
  }
  const float M = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
  float w[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) w[v] = exp2_or_zero(m[v], M);
#pragma unroll
  for (int k = 0; k < IT; ++k) {
    const int r = t + TPH * k;
    if (r < R) {
      float s = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) s = fmaf(w[v], x[k][v], s);
      dst[(h / GH) * ustride + (h % GH) * R + r] = (r == 0) ? M : (r == 1) ? (bad ? NAN : s) : (r < kPartAcc) ? 0.0f : s;
    }
  }
}

// ---------------------------------------------------------------------------
// INT2 history on the matrix cores
// ---------------------------------------------------------------------------
// ---- asynchronous page staging: global -> LDS copies (no VGPRs), one ring of
// stages per wave.  The copies are issued from inline assembly so that their
// completion is awaited explicitly (s_waitcnt vmcnt(n) before a stage is read)
// and pages ahead of the one being consumed stay in flight.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}

// address = scalar base + 32-bit lane offset (the global SADDR form).  No
// instruction offset: on these copies it also moves the LDS destination.
// STREAM marks the copy non-temporal (nt).  The per-request splits use it;
// pack and cascade blocks, whose prefix pages several packs read, keep the
// default cache policy.
template <bool STREAM>
__device__ __forceinline__ void copy16_to_lds(const void* sbase, uint32_t voff, uint32_t lds_base) {
  if constexpr (STREAM)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(lds_base)
                 : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
                 : "memory");
}

template <bool STREAM>
__device__ __forceinline__ void copy4_to_lds(const void* sbase, uint32_t voff, uint32_t lds_base) {
  if constexpr (STREAM)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(lds_base)
                 : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
                 : "memory");
}

// s_waitcnt immediate for vmcnt(0) with expcnt / lgkmcnt left at their maxima
constexpr int kWaitVmcnt0 = 0x0F70;

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait for the oldest staged page when `ahead` (wave-uniform, at most A) more
// pages of K copies each were staged after it
template <int K, int A>
__device__ __forceinline__ void wait_page(int ahead) {
  if constexpr (A == 0) {
    wait_vmem<0>();
  } else {
    if (ahead >= A) {
      wait_vmem<A * K>();
    } else {
      wait_page<K, A - 1>(ahead);
    }
  }
}

// Stage layout (one page of one KV head): K codes (16*D bytes), V codes
// (16*D bytes), K (scale, zero) [64] u32, V (scale, zero) [64] u32.  Each copy
// instruction moves 1 KB, lane l's 16 bytes landing at 16*l; every lane fetches
// exactly the 16 bytes that the same lane reads back as an MFMA operand, so the
// reads (16*l + 1024*c) are free of LDS bank conflicts:
//   K copy c, lane (q = l/16, n = l%16): plane q, tokens 4n..4n+3, bytes 16c..16c+15
//   V copy c, lane (q, n): byte column 16c + n, tokens 16q..16q+15
template <int D, int NG>
struct Stage {   // NG (scale, zero) groups per head, group-planar
  static constexpr int kK = 0, kV = 16 * D, kKsz = 32 * D, kVsz = 32 * D + 256 * NG, kBytes = 32 * D + 512 * NG;
  static constexpr int kCopies = 2 * (D / 64) + 2 * NG;   // copy instructions per page
};

// Lane byte offsets of the copies inside a (page, head) block (see Stage).
struct StageOffsets {
  uint32_t k, v, sz;
};

// V: lane (n, q) of LDS chunk c gets byte column 16c + n, tokens 16q..16q+15:
// the PV products of chunk c then cover channels 64c .. 64c + 63 (one
// 64-channel group), channel 64c + 4n + field in column n.
template <int D, int NG>
__device__ __forceinline__ StageOffsets stage_offsets(int lane) {
  constexpr int PLANE = D / 16;
  const int q = lane >> 4, n = lane & 15;
  return StageOffsets{(uint32_t)(q * kPage * PLANE + 4 * n * PLANE), (uint32_t)(n * kPage + 16 * q),
                      (uint32_t)(4 * lane)};
}

// blk (the (page, head) block index) is wave-uniform, so the block addresses
// stay in scalar registers; the second K / V copies of d = 128 differ only in
// their lane offsets
template <int D, int NG, bool STREAM>
__device__ __forceinline__ void stage_page(const DecodeDev& p, size_t blk, uint32_t stage_lds, StageOffsets o) {
  using S = Stage<D, NG>;
  // the stage address is wave-uniform (ring base and slot index); say so, so that
  // it stays in a scalar register for the copies' M0 operand
  stage_lds = __builtin_amdgcn_readfirstlane(stage_lds);
  const uint8_t* kb = p.k_codes + blk * (16 * D);
  const uint8_t* vb = p.v_codes + blk * (16 * D);
  copy16_to_lds<STREAM>(kb, o.k, stage_lds + S::kK);
  if constexpr (D == 128) copy16_to_lds<STREAM>(kb, o.k + 16, stage_lds + S::kK + 1024);
  copy16_to_lds<STREAM>(vb, o.v, stage_lds + S::kV);
  if constexpr (D == 128) copy16_to_lds<STREAM>(vb, o.v + 16 * kPage, stage_lds + S::kV + 1024);
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    copy4_to_lds<STREAM>(p.k_sz + (blk * NG + j) * kPage, o.sz, stage_lds + S::kKsz + 256 * j);
    copy4_to_lds<STREAM>(p.v_sz + (blk * NG + j) * kPage, o.sz, stage_lds + S::kVsz + 256 * j);
  }
}

// A quarter of stage_page for the waves of a cascade block (one KV head's page
// with whole-head groups): part 0 the K codes, 1 the V codes, 2 the K scales
// and zeros, 3 the V ones.  Every copy lands where stage_page puts it.
template <int D>
__device__ __forceinline__ void stage_page_part(const DecodeDev& p, size_t blk, uint32_t stage_lds, StageOffsets o,
                                                int part) {
  using S = Stage<D, 1>;
  stage_lds = __builtin_amdgcn_readfirstlane(stage_lds);
  if (part == 0) {
    const uint8_t* kb = p.k_codes + blk * (16 * D);
    copy16_to_lds<false>(kb, o.k, stage_lds + S::kK);
    if constexpr (D == 128) copy16_to_lds<false>(kb, o.k + 16, stage_lds + S::kK + 1024);
  } else if (part == 1) {
    const uint8_t* vb = p.v_codes + blk * (16 * D);
    copy16_to_lds<false>(vb, o.v, stage_lds + S::kV);
    if constexpr (D == 128) copy16_to_lds<false>(vb, o.v + 16 * kPage, stage_lds + S::kV + 1024);
  } else if (part == 2) {
    copy4_to_lds<false>(p.k_sz + blk * kPage, o.sz, stage_lds + S::kKsz);
  } else {
    copy4_to_lds<false>(p.v_sz + blk * kPage, o.sz, stage_lds + S::kVsz);
  }
}

// Softmax weights as PV A operands: one plane per (row block of 8 heads,
// group), 16 rows x 64 fp16 token slots.  Row 4g + 2e + part holds head
// 4e + g of the row block (e = head block within it, g = lane group), part 0
// the weight's high fp16 part and part 1 its low part.  The 16-byte chunk c
// of row r sits at chunk c ^ ((r >> 1) & 3): the eight rows read by one
// phase of a 128-bit load then fall in distinct banks.
constexpr int kPlaneRow = 128, kPlaneBytes = 16 * kPlaneRow;
__device__ __forceinline__ int plane_chunk(int r, int c) { return r * kPlaneRow + 16 * (c ^ ((r >> 1) & 3)); }

// Per-wave LDS: a ring of page stages and the weight planes (unless they
// reuse the consumed page slot).  Two stages: the page being processed and
// one page in flight.  With every wave of the chip one page ahead, about 9 MB
// of copies are outstanding, enough to keep HBM busy; deeper rings only
// lengthen the memory queues, and a wave then stalls issuing its copies
// instead of computing.
template <int D, int NB, int NG = 1>
struct Ring {
  static constexpr int PB = (NB + 1) / 2;   // PV row blocks
  // The planes reuse the slot of the page being processed.  With one or two
  // groups: all of them in its consumed K codes, when they fit there and every
  // row is written on every page (two head blocks per row block).  With four
  // groups: the first kSlotPlanes anywhere in the slot, since every word of it
  // (codes, scales and zeros) is in registers before the first plane store;
  // rows of an absent second head block then keep stale bytes, which only
  // reach PV result rows that are never read (MFMA rows are independent, and
  // the rescale and the fold skip absent head blocks).  The rest have their
  // own LDS, zeroed once, so rows of absent heads stay zero.
  static constexpr int kAllPlanes = PB * NG;
  static constexpr int kSlotFit = Stage<D, NG>::kBytes / kPlaneBytes;
  static constexpr int kSlotPlanes = NG == 4 ? (kAllPlanes < kSlotFit ? kAllPlanes : kSlotFit)
                                     : NB % 2 == 0 && kAllPlanes * kPlaneBytes <= 16 * D ? kAllPlanes : 0;
  static constexpr bool kPlanesInK = kSlotPlanes == kAllPlanes;   // no LDS of their own
#ifdef OSCAR_SCAN_STAGES
  static constexpr int kStages = OSCAR_SCAN_STAGES;
#else
  static constexpr int kStages = 2;
#endif
  static constexpr int kPlaneLds = (kAllPlanes - kSlotPlanes) * kPlaneBytes;
  static constexpr int kWaveBytes = kStages * Stage<D, NG>::kBytes + kPlaneLds;
};

// Lane roles (lane = 16*grp + n):
//  * QK:  D[(head, digit)][token] = sum_ch Qdigit[(head,digit)][ch] * code'[ch][token]
//         (v_mfma_i32_16x16x64_i8, exact).  A (q digits) comes from the
//         workspace; B lane (n, grp) holds, for token block tb, token 4n+tb and
//         the 16 channels of one code word of K plane grp.  The result lane
//         holds the 4 digit sums of head (4nb+grp) for token 4n+tb.
//  * PV:  D[(head, part)][channel] = sum_t W[(head, part)][t] * c[t][channel]
//         (v_mfma_f32_16x16x32_f16, fp32 sums).  A (fp16 weight parts) is
//         read from the LDS planes; B lane (n, grp) holds the fp16 operand of
//         8 tokens (of 16grp..16grp+15) of channel 64c + 4n + f: the 2-bit
//         code masked in place, i.e. the subnormal fp16 c * 4^f * 2^-24,
//         which the matrix cores multiply exactly.  The result lane holds
//         rows 4grp..4grp+3 (heads grp and 4 + grp, two parts each) of
//         column n.
// QK operands of a history wave: q digit A operands and the logit constants
template <int D, int G>
struct HistOperands {
  static constexpr int NB = (G + 3) / 4, NCH = D / 64;
  v4i qa[NB][NCH];
  float ca[NB], cb[NB][4];   // cb per (scale, zero) group (the first p.ng are used)
};

// The zero-point constants of one head: sm_log2 times the sum of q_rot over
// each group's channels, from the four quarter sums.
__device__ __forceinline__ void group_sums(const float* qb4, int ng, float sm_log2, float (&cb)[4]) {
  const float q0 = qb4[0], q1 = qb4[1], q2 = qb4[2], q3 = qb4[3];
  if (ng == 4) {
    cb[0] = sm_log2 * q0; cb[1] = sm_log2 * q1; cb[2] = sm_log2 * q2; cb[3] = sm_log2 * q3;
  } else if (ng == 2) {
    cb[0] = sm_log2 * (q0 + q1); cb[1] = sm_log2 * (q2 + q3); cb[2] = 0.0f; cb[3] = 0.0f;
  } else {
    cb[0] = sm_log2 * ((q0 + q1) + (q2 + q3)); cb[1] = 0.0f; cb[2] = 0.0f; cb[3] = 0.0f;
  }
}

template <int D, int G>
__device__ __forceinline__ void load_hist_operands(const DecodeDev& p, int b, int g, int lane, HistOperands<D, G>& o) {
  constexpr int NB = HistOperands<D, G>::NB, NCH = HistOperands<D, G>::NCH;
  const int n = lane & 15, grp = lane >> 4;
  const int h_base = b * p.Hq + g * G;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int hout = 4 * nb + grp;        // head whose results this lane holds
    o.ca[nb] = hout < G ? p.qa[h_base + hout] : 0.0f;
    group_sums(p.qb + 4 * (size_t)(h_base + (hout < G ? hout : 0)), p.ng, p.sm_log2, o.cb[nb]);
    const bool row_ok = 4 * nb + (n >> 2) < G;   // head of the A row this lane supplies
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const v4i* src = reinterpret_cast<const v4i*>(p.qdig) +
                       ((((size_t)b * p.n_kv + g) * NB + nb) * NCH + c) * kWave + lane;
      o.qa[nb][c] = row_ok ? *src : v4i{0, 0, 0, 0};
    }
  }
}

// The QK operands of a pack of PACK requests b .. b+PACK-1 at group size 4:
// head block nb of the 4*PACK-head wave is request b+nb's only head block.
template <int D, int PACK>
__device__ __forceinline__ void load_pack_operands(const DecodeDev& p, int b, int g, int lane,
                                                   HistOperands<D, 4 * PACK>& o) {
  constexpr int NCH = D / 64;
  const int grp = lane >> 4;
#pragma unroll
  for (int nb = 0; nb < PACK; ++nb) {
    const int unit = (b + nb) * p.n_kv + g;
    o.ca[nb] = p.qa[(size_t)(b + nb) * p.Hq + g * 4 + grp];
    group_sums(p.qb + 4 * ((size_t)(b + nb) * p.Hq + g * 4 + grp), p.ng, p.sm_log2, o.cb[nb]);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      o.qa[nb][c] = reinterpret_cast<const v4i*>(p.qdig)[((size_t)unit * NCH + c) * kWave + lane];
  }
}

// The PV B operand of field f for 8 tokens: bytes 0 and 2 of the code words
// w0, w1 and bytes 1 and 3 (s = w >> 8) hold tokens (0, 2), (4, 6) and
// (1, 3), (5, 7), one per 16-bit half.  Masked in place, each half is the
// fp16 subnormal c * 4^f * 2^-24.  With kHiBit only the field's high bit
// stays (2 * (c >> 1) * 4^f * 2^-24).
template <bool kHiBit>
__device__ __forceinline__ half8 pv_operand(uint32_t w0, uint32_t s0, uint32_t w1, uint32_t s1, int f) {
  const uint32_t m = (kHiBit ? 0x00020002u : 0x00030003u) << (2 * f);
  const u32x4 x = {w0 & m, s0 & m, w1 & m, s1 & m};
  return __builtin_bit_cast(half8, x);
}

// pv_operand restricted to the lanes whose mask lm is all ones (a column
// half of the product: the 32-channel groups of one 64-channel chunk)
template <bool kHiBit>
__device__ __forceinline__ half8 pv_operand_cols(uint32_t w0, uint32_t s0, uint32_t w1, uint32_t s1, int f,
                                                 uint32_t lm) {
  const uint32_t m = ((kHiBit ? 0x00020002u : 0x00030003u) << (2 * f)) & lm;
  const u32x4 x = {w0 & m, s0 & m, w1 & m, s1 & m};
  return __builtin_bit_cast(half8, x);
}

__device__ __forceinline__ uint32_t pack_rtz(float a, float b) {   // two fp16, toward zero: a low, b high
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// One wave's scan of history pages pg_begin .. pg_begin + count - 1.  pid_lane
// holds the page id of page pg_begin + lane, and qo the QK operands; both were
// loaded by the caller together with the history length, and this wave's
// vector loads have completed.
// CASC: the wave is one of the four of a cascade block, which all scan the
// same pages (count and pid_lane are the block's): ring is the block's shared
// two-stage ring, each wave issues its quarter of every page's copies, and a
// block barrier per page makes the page visible to all; own_planes are the
// wave's weight planes.  A wave with compute false only stages and keeps step.
// The fold into mw follows a last block barrier (mw may overlay the ring).
template <int D, int G, bool LM, int NG, bool CASC = false, bool STREAM = false>
__device__ __forceinline__ void hist_wave(const DecodeDev& p, int g, int pg_begin, int count, int hl, int pid_lane,
                                          const HistOperands<D, G>& qo, uint8_t* ring, float* mw, bool& poison,
                                          int lane, uint8_t* own_planes = nullptr, int wave = 0, bool compute = true) {
  constexpr int NB = (G + 3) / 4;
  constexpr int NCH = D / 64;   // code words per token per K plane; 64-channel chunks of V
  using S = Stage<D, NG>;
  using RG = Ring<D, NB, NG>;
  constexpr int PB = RG::PB;
  constexpr int NS = RG::kStages;
  constexpr int GC = D / NG;    // channels per (scale, zero) group
  static_assert(NG == 1 || NG == 2 || (NG == 4 && D == 128), "groups of the head, 64 or 32 channels");
  static_assert(!CASC || (NG == 1 && !LM && NS == 2), "cascade blocks: uniform codebook, whole-head groups");
  constexpr int kSlotPl = CASC ? 0 : RG::kSlotPlanes;                          // planes in the page slot
  constexpr int kOwnPlaneBytes = CASC ? PB * NG * kPlaneBytes : RG::kPlaneLds;   // planes of its own
  const int n = lane & 15, grp = lane >> 4;
  const auto& qa = qo.qa;
  const auto& ca = qo.ca;
  const auto& cb = qo.cb;
  // With (scale, zero) groups the QK dot is needed per group.  Operand block
  // grp (lanes 16grp .. 16grp + 15) of every chunk holds K plane grp, i.e.
  // channels grp*D/4 .. grp*D/4 + D/4 - 1, so a group is one block (32-channel
  // groups at d = 128) or two.  Two groups: group 0's q operand keeps blocks 0
  // and 1 and zeroes 2 and 3.  Four groups: the K operand of group j < 3
  // keeps block j only.  The last group's dot is the full one minus the
  // others (exact in int32).
  v4i qa0[NB][NCH];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int c = 0; c < NCH; ++c) qa0[nb][c] = (NG == 2 && grp < 2) ? qa[nb][c] : v4i{0, 0, 0, 0};
  const uint64_t page_ok = __ballot(pid_lane >= 0 && (int64_t)pid_lane < p.n_pages);

  // acc: fp32 PV sums of row block rb, chunk c, field f, rows 4grp..4grp+3
  // (Lloyd-Max: acc2 the sums over the codes' high bits).  mref: reference
  // maximum (log2 units) of each head block; logits are kept relative to it.
  // thr: rescale when a relative logit exceeds it (-inf until the first page
  // has set the references).  kap: weight scale putting the largest weight
  // the thresholds allow at 2^14 (0 until the first page).
  v4f acc[PB][NCH][4], acc2[PB][NCH][4];
  float mref[NB], lsum[NB], zsum[NB][NG];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    mref[nb] = 0.0f;
    lsum[nb] = 0.0f;
#pragma unroll
    for (int j = 0; j < NG; ++j) zsum[nb][j] = 0.0f;
  }
#pragma unroll
  for (int rb = 0; rb < PB; ++rb)
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        acc[rb][c][f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        acc2[rb][c][f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      }
  float thr = -INFINITY, smax = 0.0f, sthr = 0.0f, kap = 0.0f;

  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_offset(ring));
  uint8_t* planes = CASC ? own_planes : RG::kPlanesInK ? nullptr : ring + NS * S::kBytes;
  if constexpr (kOwnPlaneBytes > 0) {   // rows of absent heads are never written
#pragma unroll
    for (int o = 0; o < kOwnPlaneBytes; o += 16 * kWave)
      *reinterpret_cast<uint4*>(planes + o + 16 * lane) = make_uint4(0, 0, 0, 0);
  }
  // (page, head) block of each of the wave's pages, one per lane; an invalid
  // page id is staged from page 0 and skipped
  const size_t blk_lane = ((page_ok >> lane) & 1) ? (size_t)pid_lane * p.n_kv + g : (size_t)g;
  auto page_blk = [&](int i) -> size_t {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)blk_lane, i);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(blk_lane >> 32), i);
    return ((size_t)hi << 32) | lo;
  };
  const StageOffsets soff = stage_offsets<D, NG>(lane);
  const int pre = count < NS - 1 ? count : NS - 1;
  if constexpr (CASC) {
    if (count > 0) stage_page_part<D>(p, page_blk(0), ring_lds, soff, wave);
  } else {
    for (int i = 0; i < pre; ++i) stage_page<D, NG, STREAM>(p, page_blk(i), ring_lds + i * S::kBytes, soff);
  }
  int slot_use = 0, slot_fill = pre;   // ring slots of page i and of page i + NS - 1

  // Issue priority falls with the wave's relative progress through its range
  // (3 in the first quarter .. 0 in the last).  A SIMD otherwise issues
  // oldest-first: the older block's waves finish early and the younger ones
  // are left to run alone, one wave per SIMD, with their page latency
  // exposed.  This way the waves sharing a SIMD advance and finish together.
  int prio = 3, prio_next = (count + 3) / 4;   // page index of the next drop
  set_wave_priority(3);

  for (int i = 0; i < count; ++i) {
    const int pg = pg_begin + i;
    if (i == prio_next) {   // three times per wave
      prio = 3 - (4 * i) / count;
      set_wave_priority(prio);
      prio_next = ((4 - prio) * count + 3) / 4;
    }
    uint8_t* st;
    if constexpr (CASC) {
      // page i's copies (every wave's quarter) have landed, and every wave is
      // done with page i - 1, whose slot now takes page i + 1
      wait_vmem<0>();
      __syncthreads();
      if (i + 1 < count) stage_page_part<D>(p, page_blk(i + 1), ring_lds + ((i + 1) & 1) * S::kBytes, soff, wave);
      st = ring + (i & 1) * S::kBytes;
      if (!compute) continue;
    } else {
      if (i + NS - 1 < count) {
        stage_page<D, NG, STREAM>(p, page_blk(i + NS - 1), ring_lds + slot_fill * S::kBytes, soff);
        slot_fill = slot_fill == NS - 1 ? 0 : slot_fill + 1;
      }
      wait_page<S::kCopies, NS - 1>(count - 1 - i);
      st = ring + slot_use * S::kBytes;
      slot_use = slot_use == NS - 1 ? 0 : slot_use + 1;
    }
    if (!((page_ok >> i) & 1)) {
      poison = true;
      continue;
    }
    const int nv = min(kPage, hl - pg * kPage);
    if (nv < kPage) {
      // slots past the history end hold undefined bytes: give them zero
      // scales and zeros, so only the logit mask below has to exclude them
      if (lane >= nv) {
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          reinterpret_cast<uint32_t*>(st + S::kKsz + 256 * j)[lane] = 0u;
          reinterpret_cast<uint32_t*>(st + S::kVsz + 256 * j)[lane] = 0u;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }

    uint32_t kword[4 * NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint4 k4 = *reinterpret_cast<const uint4*>(st + S::kK + 1024 * c + 16 * lane);
      kword[4 * c] = k4.x; kword[4 * c + 1] = k4.y; kword[4 * c + 2] = k4.z; kword[4 * c + 3] = k4.w;
    }
    uint4 vpre[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) vpre[c] = *reinterpret_cast<const uint4*>(st + S::kV + 1024 * c + 16 * lane);
    // token 4n+tb, group j; the Lloyd-Max level 7c - 10 - (c >> 1) moves its -10 into the zero
    float sk[NG][4], zk[NG][4], sv[NG][4], zv[NG][4];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const uint4 ksz = *reinterpret_cast<const uint4*>(st + S::kKsz + 256 * j + 16 * n);
      const uint4 vsz = *reinterpret_cast<const uint4*>(st + S::kVsz + 256 * j + 16 * n);
      const uint32_t kw4[4] = {ksz.x, ksz.y, ksz.z, ksz.w};
      const uint32_t vw4[4] = {vsz.x, vsz.y, vsz.z, vsz.w};
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        sk[j][tb] = f16_to_f32(kw4[tb] & 0xffffu);
        zk[j][tb] = f16_to_f32(kw4[tb] >> 16);
        sv[j][tb] = f16_to_f32(vw4[tb] & 0xffffu);
        zv[j][tb] = f16_to_f32(vw4[tb] >> 16);
        if constexpr (LM) zv[j][tb] = fmaf(-10.0f, sv[j][tb], zv[j][tb]);
      }
    }

    // ---- QK, one head block at a time: token block tb holds token 4n+tb.
    // Relative logit (log2 units): scale*ca*dot + (zero*cb - mref).
    float lg[NB][4], lmax[NB];
    bool need = false;
    auto qk_block = [&](int nb, int tb) {
      const bool hok = 4 * nb + grp < G;
      v4i dq, dq0, dqg[3];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t w = kword[tb * NCH + c];
        const v4i bop = v4i{code_operand<LM>(w, 0), code_operand<LM>(w, 1), code_operand<LM>(w, 2),
                            code_operand<LM>(w, 3)};
        dq = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[nb][c], bop, c == 0 ? v4i{0, 0, 0, 0} : dq, 0, 0, 0);
        if constexpr (NG == 2)
          dq0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa0[nb][c], bop, c == 0 ? v4i{0, 0, 0, 0} : dq0, 0, 0, 0);
        if constexpr (NG == 4) {
#pragma unroll
          for (int j = 0; j < 3; ++j) {
            const v4i bj = grp == j ? bop : v4i{0, 0, 0, 0};
            dqg[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[nb][c], bj, c == 0 ? v4i{0, 0, 0, 0} : dqg[j], 0, 0, 0);
          }
        }
      }
      // digits: d0 + 2^8 d1 and d2 + 2^8 d3 are exact in int32
      auto dot_of = [](v4i v) {
        const int lo = v.x + v.y * 256, hi = v.z + v.w * 256;
        return fmaf((float)hi, 65536.0f, (float)lo);
      };
      if constexpr (NG == 1) {
        // an invalid head gets fma(0, dot, -inf) = -inf (dot is finite)
        const float off = hok ? fmaf(zk[0][tb], cb[nb][0], -mref[nb]) : -INFINITY;
        lg[nb][tb] = fmaf(sk[0][tb] * ca[nb], dot_of(dq), off);
      } else {
        // per-group digit sums, then the logit from the last group down
        v4i dg[NG];
        if constexpr (NG == 2) {
          dg[0] = dq0;
          dg[1] = dq - dq0;
        } else {
          dg[0] = dqg[0];
          dg[1] = dqg[1];
          dg[2] = dqg[2];
          dg[3] = dq - dqg[0] - dqg[1] - dqg[2];
        }
        float off = -mref[nb];
#pragma unroll
        for (int j = NG - 1; j >= 0; --j) off = fmaf(zk[j][tb], cb[nb][j], off);
        float l = hok ? off : -INFINITY;
#pragma unroll
        for (int j = NG - 1; j >= 0; --j) l = fmaf(sk[j][tb] * ca[nb], dot_of(dg[j]), l);
        lg[nb][tb] = l;
      }
    };
    if constexpr (NG == 4) {
      // one token block at a time: its K operands and four chains per head block
      // stay in registers, and the next block's MFMAs start after these results
      // are consumed (with every token block in flight at once, the chains' results
      // and masked operands overflow the VGPRs into the accumulation registers)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) qk_block(nb, tb);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) qk_block(nb, tb);
    }
    if (nv < kPage) {   // tokens past the history end (the last page only)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          if (4 * n + tb >= nv) lg[nb][tb] = -INFINITY;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      lmax[nb] = fmaxf(fmaxf(lg[nb][0], lg[nb][1]), fmaxf(lg[nb][2], lg[nb][3]));
      need |= lmax[nb] > thr;
    }
    float svmax = fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3]));
#pragma unroll
    for (int j = 1; j < NG; ++j) svmax = fmaxf(svmax, fmaxf(fmaxf(sv[j][0], sv[j][1]), fmaxf(sv[j][2], sv[j][3])));
    need |= svmax > sthr;

    __builtin_amdgcn_sched_barrier(0);
    if (__any(need)) {
      // raise the references and the V-scale bound; rescale the sums under the
      // new ones (the fp32 PV sums by the same factor as the weight sums, and
      // by the change of the weight scale)
      const bool first = !(kap > 0.0f);   // nothing accumulated yet
      const float s_new = fmaxf(smax, group16_max(svmax));
      float alpha[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float t = group16_max(lmax[nb]);
        // raise of the reference; the first page sets it (all -inf: head has no rows)
        const float delta = first ? (t == -INFINITY ? 0.0f : t) : fmaxf(t, 0.0f);
        alpha[nb] = exp2f(-delta);
        if (!first) {
          lsum[nb] *= alpha[nb];
#pragma unroll
          for (int j = 0; j < NG; ++j) zsum[nb][j] *= alpha[nb];
        }
        mref[nb] += delta;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) lg[nb][tb] -= delta;
      }
      thr = kLazyThr;
      // the page maximum of the V scales is the same in every lane: keep the
      // scale state in scalar registers
      smax = wave_uniform(s_new);
      sthr = wave_uniform(kScaleSlack * smax);
      // weights p*scale_V*kap stay below 2^14 (p < 2^kLazyThr, scale_V < kScaleSlack*smax)
      const float kap_new = wave_uniform(kWeightTop / (exp2f(kLazyThr) * kScaleSlack * (smax > 0.0f ? smax : 1.0f)));
      if (!first) {
        const float r = kap_new / kap;
#pragma unroll
        for (int rb = 0; rb < PB; ++rb)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            if (2 * rb + e >= NB) continue;   // rows of an absent head block are never read
            const float fct = alpha[2 * rb + e] * r;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
              for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int part = 0; part < 2; ++part) {
                  acc[rb][c][f][2 * e + part] *= fct;
                  if constexpr (LM) acc2[rb][c][f][2 * e + part] *= fct;
                }
          }
      }
      kap = kap_new;
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- weights w = p*scale_V*kap as an fp16 pair (high part, and the
    // remainder scaled by 2^11), into the planes of the PV A operands.  Lane
    // (n, grp) holds tokens 4n..4n+3, stored in slots 4n..4n+3 in the order
    // of the B operands' halves: tokens 0, 2, 1, 3.
    // plane k of (row block, group) index rb*NG + j
    auto plane_at = [&](int k) -> uint8_t* {
      return k < kSlotPl ? st + k * kPlaneBytes : planes + (k - kSlotPl) * kPlaneBytes;
    };
    float svk[NG][4];
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) svk[j][tb] = sv[j][tb] * kap;
    __builtin_amdgcn_wave_barrier();   // every lane has read the slot's words the planes may overlay
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float pr[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        pr[tb] = __builtin_amdgcn_exp2f(lg[nb][tb]);   // exp2(-inf) = 0
        lsum[nb] += pr[tb];
      }
      const int r = 4 * grp + 2 * (nb & 1);   // the head's high-part row
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        float w[4], u[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          zsum[nb][j] = fmaf(pr[tb], zv[j][tb], zsum[nb][j]);
          w[tb] = pr[tb] * svk[j][tb];
          u[tb] = w[tb] * 2048.0f;
        }
        const uint32_t h02 = pack_rtz(w[0], w[2]), h13 = pack_rtz(w[1], w[3]);
        const uint32_t l02 = pack_rtz(fmaf(f16_to_f32(h02 & 0xffffu), -2048.0f, u[0]),
                                      fmaf(f16_to_f32(h02 >> 16), -2048.0f, u[2]));
        const uint32_t l13 = pack_rtz(fmaf(f16_to_f32(h13 & 0xffffu), -2048.0f, u[1]),
                                      fmaf(f16_to_f32(h13 >> 16), -2048.0f, u[3]));
        uint8_t* plane = plane_at((nb >> 1) * NG + j) + 8 * (n & 1);
        *reinterpret_cast<uint2*>(plane + plane_chunk(r, n >> 1)) = make_uint2(h02, h13);
        *reinterpret_cast<uint2*>(plane + plane_chunk(r + 1, n >> 1)) = make_uint2(l02, l13);
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- PV: lane (n, grp) reads row n, token slots 16grp + 8ks .. + 7 of
    // each plane.  Column n of chunk c is channels 64c + 4n .. 64c + 4n + 3,
    // of group (64c + 4n) / GC: with 64-channel groups chunk c is group c;
    // with 32-channel groups columns 0..7 are group 2c and 8..15 group 2c + 1,
    // and each takes its own product with the other half's columns masked.
    half8 wa[PB][NG][2];
#pragma unroll
    for (int rb = 0; rb < PB; ++rb)
#pragma unroll
      for (int j = 0; j < NG; ++j)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          wa[rb][j][ks] = *reinterpret_cast<const half8*>(plane_at(rb * NG + j) + plane_chunk(n, 2 * grp + ks));
    const uint32_t cols_lo = n < 8 ? 0xffffffffu : 0u;   // column half of this lane
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint4 v4 = vpre[c];
      const uint32_t s0 = v4.x >> 8, s1 = v4.y >> 8, s2 = v4.z >> 8, s3 = v4.w >> 8;
      const int jp = GC >= 64 ? 64 * c / GC : 2 * c;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint32_t a0 = ks ? v4.z : v4.x, b0 = ks ? s2 : s0, a1 = ks ? v4.w : v4.y, b1 = ks ? s3 : s1;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          if constexpr (GC >= 64) {
            const half8 bop = pv_operand<false>(a0, b0, a1, b1, f);
#pragma unroll
            for (int rb = 0; rb < PB; ++rb)
              acc[rb][c][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[rb][jp][ks], bop, acc[rb][c][f], 0, 0, 0);
            if constexpr (LM) {
              const half8 bhi = pv_operand<true>(a0, b0, a1, b1, f);
#pragma unroll
              for (int rb = 0; rb < PB; ++rb)
                acc2[rb][c][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[rb][jp][ks], bhi, acc2[rb][c][f], 0, 0, 0);
            }
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t cm = h ? ~cols_lo : cols_lo;
              const half8 bop = pv_operand_cols<false>(a0, b0, a1, b1, f, cm);
#pragma unroll
              for (int rb = 0; rb < PB; ++rb)
                acc[rb][c][f] =
                    __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[rb][jp + h][ks], bop, acc[rb][c][f], 0, 0, 0);
              if constexpr (LM) {
                const half8 bhi = pv_operand_cols<true>(a0, b0, a1, b1, f, cm);
#pragma unroll
                for (int rb = 0; rb < PB; ++rb)
                  acc2[rb][c][f] =
                      __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[rb][jp + h][ks], bhi, acc2[rb][c][f], 0, 0, 0);
              }
            }
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  wait_vmem<0>();
  if constexpr (CASC) __syncthreads();   // no wave reads the shared ring or the planes any more
  set_wave_priority(3);   // the block's merge waits for this wave

  // ---- reduce the weight sums over the 16 lanes of each head; each head's
  // (m, l, acc) slot overlays the start of the wave's ring.  Channel value:
  // (high row + low row / 2^11) * 2^24 / (kap * 4^f), plus the zero-point sum.
  float lz[NB], zs[NB][NG];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    lz[nb] = group16_sum(lsum[nb]);
#pragma unroll
    for (int j = 0; j < NG; ++j) zs[nb][j] = group16_sum(zsum[nb][j]);
  }
  const float kinv = kap > 0.0f ? 16777216.0f / kap : 0.0f;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int h = 4 * nb + grp;
    if (h < G) {
      float* mh = mw + h * part_row(D);
      if (n == 0) {
        mh[0] = kap > 0.0f ? mref[nb] : -INFINITY;   // no page processed: empty partial
        mh[1] = lz[nb];
      }
      const int rb = nb >> 1, e = nb & 1;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        float z = zs[nb][0];   // the zero-point sum of column n's group
#pragma unroll
        for (int j = 1; j < NG; ++j)
          if ((64 * c + 4 * n) / GC == j) z = zs[nb][j];
        float o[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          float v = fmaf(acc[rb][c][f][2 * e + 1], 1.0f / 2048.0f, acc[rb][c][f][2 * e]);
          if constexpr (LM)
            v = fmaf(7.0f, v, -0.5f * fmaf(acc2[rb][c][f][2 * e + 1], 1.0f / 2048.0f, acc2[rb][c][f][2 * e]));
          o[f] = fmaf(v, kinv * (f == 0 ? 1.0f : f == 1 ? 0.25f : f == 2 ? 0.0625f : 0.015625f), z);
        }
        *reinterpret_cast<float4*>(mh + kPartAcc + 64 * c + 4 * n) = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 1. rotate the query: q_rot = q R_K[g]; MFMA digit operands and constants
// ---------------------------------------------------------------------------
// Two blocks per query head, one per half of the output channels (half = 0
// or 1): each reads half of R_K, and the digit scale needs no exchange
// between them (it comes from |q|_2).  qb[4 bh + 2 half + e] is the sum of
// q_rot over channels 32e .. 32e + 31 of the half (none for e = 1 when
// head_dim is 64): the sums of every 32-channel group, whose pairs give the
// 64-channel groups and the head.
template <int D>
__device__ __forceinline__ void rotate_query_block(const DecodeDev& p, int bh, int half) {
  constexpr int NCH = D / 64, PLANE = D / 16;
  constexpr int DH = D / 2;   // output channels of this block
  // thread (jq, part): columns 4jq..4jq+3 of the half, rows part*IP ..
  // part*IP+IP-1, loaded as IP 16-byte vectors all in flight at once
  constexpr int QPR = DH / 4, P = kBlock / QPR, IP = D / P;
  __shared__ float qs[D];
  __shared__ __attribute__((aligned(16))) float part_s[P][DH];
  const int b = bh / p.Hq, h = bh % p.Hq, g = h / p.G, hl = h % p.G;
  const int tid = threadIdx.x, jq = tid % QPR, part = tid / QPR;
  // q is requested before R, so waiting for it leaves the R loads in flight
  const float qv = tid < D ? bf16_to_f32(p.q[(size_t)bh * D + tid]) : 0.0f;
  const float4* R =
      reinterpret_cast<const float4*>(p.r_k + (size_t)g * D * D + (size_t)part * IP * D + half * DH) + jq;
  float4 r[IP];
#pragma unroll
  for (int k = 0; k < IP; ++k) r[k] = R[(size_t)k * (D / 4)];
  if (tid < D) qs[tid] = qv;
  __syncthreads();
  // Fixed-point scale of the digits, from |q|_2 while R is still arriving:
  // every |q_rot_j| <= |q|_2 |R e_j|_2 = |q|_2 for an orthogonal R, and the
  // factor 2 covers the rounding of R and of the sums.  The norm is taken as
  // 2^e |q 2^-e|_2 with 2^e <= max|q_i| < 2^(e+1), so its square neither
  // overflows nor underflows.  kq is the power of two with
  // 16 * 2|q|_2 * kq <= 2^30 (at most 2^100); products are clamped to that range.
  float qm = 0.0f;
#pragma unroll
  for (int i = tid % kWave; i < D; i += kWave) qm = fmaxf(qm, fabsf(qs[i]));
  qm = wave_max(qm);
  float kq = 1.0f;
  if (qm > 0.0f) {
    const int e = ilogbf(qm);
    float sq = 0.0f;
#pragma unroll
    for (int i = tid % kWave; i < D; i += kWave) {
      const float t = ldexpf(qs[i], -e);
      sq = fmaf(t, t, sq);
    }
    const float bound = 2.0f * ldexpf(sqrtf(wave_sum(sq)), e);
    kq = fminf(exp2f(floorf(log2f(kFix / (16.0f * bound)))), 0x1p100f);
    if (16.0f * bound * kq > kFix) kq *= 0.5f;
  }
  float4 a4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int k = 0; k < IP; ++k) a4 = f4_fma(qs[part * IP + k], r[k], a4);
  reinterpret_cast<float4*>(part_s[part])[jq] = a4;
  __syncthreads();
  float acc = 0.0f;
  if (tid < DH) {
    const int ch = half * DH + tid;             // output channel of this thread
#pragma unroll
    for (int q = 0; q < P; ++q) acc += part_s[q][tid];
    const int pp = ch & 3;                      // mask index of channel ch
    // the plane factor cancels the operand's in-place weight (Lloyd-Max operands carry none)
    const float scale = kq * ((pp == 0 || p.lm) ? 16.0f : pp == 1 ? 4.0f : 1.0f);
    const float fx = fminf(fmaxf(rintf(acc * scale), -kFix), kFix);
    const uint32_t U = balanced_digits((uint32_t)(int)fx);
    const int ib = ch >> 2;                     // code-row byte of channel ch
    const int kb = ib / PLANE, rem = ib % PLANE, c = rem >> 2, bb = rem & 3;
    const int nb = hl >> 2, hr = hl & 3;
    uint8_t* base = p.qdig + ((((size_t)b * p.n_kv + g) * p.NB + nb) * NCH + c) * kWave * 16;
#pragma unroll
    for (int dj = 0; dj < 4; ++dj) {
      const int lane = 16 * kb + 4 * hr + dj;
      base[lane * 16 + 4 * pp + bb] = (uint8_t)(U >> (8 * dj));
    }
  }
  // sums of q_rot over the half's 32-channel units (tid < DH <= 64: wave 0,
  // unit e in lanes 32e .. 32e + 31 of the 16-lane row sums), after the digit
  // stores
  const float rs = group16_sum(acc);
  const float s0 = lane_value(rs, 0) + lane_value(rs, 16), s1 = lane_value(rs, 32) + lane_value(rs, 48);
  if (tid == 0) {
    if (half == 0) p.qa[bh] = p.sm_log2 / (16.0f * kq);
    p.qb[4 * bh + 2 * half] = s0;
    p.qb[4 * bh + 2 * half + 1] = s1;
  }
}

// Launch 1 of a decode: two blocks per query head rotate q.
template <int D>
__global__ __launch_bounds__(kBlock) void prepare_kernel(DecodeDev p) {
  rotate_query_block<D>(p, blockIdx.x >> 1, blockIdx.x & 1);
}

// Block `id` of a decode step's demotions: the step's K tokens first, then
// its V tokens, one block per (token, KV head).  They run in the decode's
// last launch, on the compute units its merge leaves idle: the demoted slots
// lie past every hist_len, so no launch of this decode reads them.
template <int D>
__device__ __forceinline__ void demote_step_block(const DecodeDev& p, int id, const DemoteDev& dk,
                                                  const DemoteDev& dv) {
  const int64_t nk = dk.n_tok * p.n_kv;
  const DemoteDev& dm = id < nk ? dk : dv;
  const int gflag = p.ng == 1 ? 0 : D / p.ng == 64 ? OSCAR_GROUPS_64 : OSCAR_GROUPS_32;
  const int kind = (id < nk ? OSCAR_KIND_K : OSCAR_KIND_V) | (p.lm ? OSCAR_CODEBOOK_LLOYD_MAX : 0) | gflag;
  if (id >= nk) id -= (int)nk;
  demote_token_block<D>(kind, dm.x, dm.n_src, dm.tok_stride, dm.head_stride, dm.src_idx, id / p.n_kv, id % p.n_kv,
                        p.n_kv, dm.rot, dm.clip, dm.dst_slot, dm.codes, dm.sz, dm.n_pages);
}

// ---------------------------------------------------------------------------
// 2. scan: history splits, then one BF16 block per 64-token sink / recent chunk
// ---------------------------------------------------------------------------
// Waves per SIMD the scan is compiled for: the 16-head wave (G = 16, or four
// requests of group size 4 in one wave) fits two per SIMD without spills with
// the uniform codebook and whole-head groups, and one otherwise.  Four groups
// per head fit two with up to 8 heads per wave (the VGPR budget of two waves
// also keeps their MFMA results out of the accumulation registers) and one
// with 16.
template <int G, bool LM, int NG, int PACK>
constexpr int scan_waves_per_simd() {
  if constexpr (NG == 4) return G > 8 ? 1 : 2;
  return (G > 8 || PACK > 2) && (LM || NG == 2) ? 1 : OSCAR_SCAN_WAVES_PER_SIMD;
}

// LDS of a scan block: four history waves' rings (a group-4 kernel also runs
// 4*PACK-head waves, PACK requests, on shared-prefix splits) or four BF16
// chunk waves' tiles, whichever is larger
template <int D, int G, int NG, int PACK>
constexpr int scan_smem_bytes() {
  constexpr int own = 4 * Ring<D, (G + 3) / 4, NG>::kWaveBytes;
  constexpr int pack = G == 4 ? 4 * Ring<D, PACK, NG>::kWaveBytes : 0;
  constexpr int hist = own > pack ? own : pack;
  constexpr int bf16 = 4 * bf16_lds_bytes<D, G>();
  return hist > bf16 ? hist : bf16;
}

// Scan blocks one compute unit holds at once: the waves per SIMD the kernel is
// compiled for (a block has one wave per SIMD), or fewer if its LDS (plus the
// four block flags) does not fit that many times into the 160 KB of a CU.
constexpr int kLdsPerCu = 160 * 1024;
template <int D, int G, bool LM, int NG, int PACK>
constexpr int scan_blocks_per_cu() {
  constexpr int by_lds = kLdsPerCu / (scan_smem_bytes<D, G, NG, PACK>() + 16);
  constexpr int by_waves = scan_waves_per_simd<G, LM, NG, PACK>();
  return by_lds < by_waves ? by_lds : by_waves;
}

template <int D, int G, bool LM, int NG, int PACK = 2>
__global__ __launch_bounds__(kBlock, (scan_waves_per_simd<G, LM, NG, PACK>())) void decode_main_kernel(DecodeDev p) {
  constexpr int NB = (G + 3) / 4;
  using RG = Ring<D, NB, NG>;
  constexpr int kSmem = scan_smem_bytes<D, G, NG, PACK>();
  static_assert(4 * G * part_row(D) * 4 <= kSmem, "BF16 merge slots must fit");
  static_assert(G * part_row(D) * 4 <= RG::kWaveBytes, "merge slot must fit in the wave's ring");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
  __shared__ int flags[4];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int units = p.B * p.n_kv;
  const int id = blockIdx.x;
  // block ids: the history splits past the shared prefix (split, request, KV
  // head) and the prefix splits read for request packs (split, pack, KV head),
  // then the prefix splits of the requests past the last whole pack (split,
  // request, KV head), then the BF16 chunks.  The per-request splits come
  // before the pack blocks: they take the first round of resident slots
  // beside pack blocks and end early, and the pack blocks, the longest of the
  // launch, follow into their slots (dispatched the other way round, the
  // per-request splits ran after the pack blocks, at one wave per SIMD).
  // Cascade blocks, fewer and longer still, come first.
  const int n_packed = p.n_pref * p.pack_units * p.n_kv;
  const int n_rest = (p.splits - p.n_pref) * units;
  const int left = p.B - p.packs * p.pack;
  const int n_hist = n_packed + n_rest + p.n_pref * left * p.n_kv;
  const int rest0 = p.casc ? n_packed : 0;   // first id of the per-request splits
  const int pid = id - (p.casc ? 0 : n_rest);   // index among the pack (or cascade) blocks
  bool poison = false;

  if (id >= n_hist) {
    // ---- BF16 sink / recent chunks (block-uniform), after every history block:
    // bf_cpb consecutive chunks per block, 16 tokens of each per wave.  With
    // one chunk per block, spread this thin, a block's loads stay small next
    // to the history block that shares its CU; with many units, a block takes
    // all of its unit's chunks, so the launch's tail has fewer, fuller blocks.
    const int cid = id - n_hist;
    const int unit = cid % units, bc = cid / units;
    const int b = unit / p.n_kv, g = unit % p.n_kv;
    WaveAcc<D, G> st;
    acc_init(st);
    int sl = p.sink_len[b], rl = p.recent_len[b];
    if (sl < 0 || sl > p.sink_cap) {
      poison = true;
      sl = 0;
    }
    if (rl < 0 || rl > p.recent_cap) {
      poison = true;
      rl = 0;
    }
    bf16x8 qa[D / 32];
    bf16_q_operands<D, G>(qa, p.q + ((size_t)b * p.Hq + g * G) * D, lane);
    const int c_end = min(p.chunks, (bc + 1) * p.bf_cpb);
    for (int c = bc * p.bf_cpb; c < c_end; ++c) {   // block-uniform
      const uint16_t *kb, *vb;
      int nv;
      if (c < p.sink_chunks) {
        const int t0 = c * kPage + kBf16WaveTokens * wave;
        nv = min(kBf16WaveTokens, sl - t0);
        const size_t off = (((size_t)b * p.n_kv + g) * p.sink_cap + t0) * D;
        kb = p.sink_k + off;
        vb = p.sink_v + off;
      } else {
        const int t0 = (c - p.sink_chunks) * kPage + kBf16WaveTokens * wave;
        nv = min(kBf16WaveTokens, rl - t0);
        const size_t off = (((size_t)b * p.n_kv + g) * p.recent_cap + t0) * D;
        kb = p.recent_k + off;
        vb = p.recent_v + off;
      }
      if (nv > 0) {
        Bf16Tile<D> tile;
        bf16_load<D, true>(tile, kb, vb, nv, lane);
        bf16_compute<D, G>(st, tile, qa, p.sm_log2, nv, smem + wave * bf16_lds_bytes<D, G>(), lane);
      }
    }
    __syncthreads();   // the merge slots overlay the tiles' LDS
    float* mrg = reinterpret_cast<float*>(smem);
    store_wave_state<D, G>(st, mrg + wave * G * part_row(D), lane, false);
    if (lane == 0) flags[wave] = poison ? 1 : 0;
    __syncthreads();
    combine_block<G, D>(mrg, G * part_row(D), flags,
                        p.bpart + (((size_t)b * p.n_kv + g) * p.bf_blocks + bc) * (size_t)G * part_row(D), tid);
    return;
  }

  if constexpr (G == 4 && PACK == 4) {
    if (p.casc && id < n_packed) {
      // ---- a cascade block: one split inside the shared prefix, up to four
      // packs of four requests (wave w takes pack 4*group + w) reading every
      // page from one staged copy
      using S1 = Stage<D, 1>;
      constexpr int kRing = 2 * S1::kBytes, kPlanes = 2 * kPlaneBytes;   // shared ring; each wave's planes
      constexpr int kSlot = 16 * part_row(D) * 4;                        // each wave's 16-head merge slot
      static_assert(kRing + 4 * kPlanes <= kSmem && 4 * kSlot <= kSmem, "cascade LDS must fit");
      const int per_split = p.pack_units * p.n_kv;
      const int split = pid / per_split, grp_id = (pid % per_split) / p.n_kv, g = pid % p.n_kv;
      const int pk = 4 * grp_id + wave;                // this wave's pack
      const bool active = pk < p.packs;
      const int b = 4 * pk;                            // its first request
      const int ws0 = split * p.pps, count = p.pps;    // the whole split, inside the prefix
      const int full = (ws0 + count) * kPage;          // every history of the group must cover it
      const int32_t* row0 = p.block_table + (size_t)(16 * grp_id) * p.max_pages;   // the staged row
      const int pid_lane = lane < count ? row0[ws0 + lane] : -1;
      HistOperands<D, 16> qo;
      bool bad = false;
      if (active) {
        load_pack_operands<D, 4>(p, b, g, lane, qo);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pr = lane < count ? p.block_table[(size_t)(b + r) * p.max_pages + ws0 + lane] : -1;
          const int hr = p.hist_len[b + r];
          bad |= pr != pid_lane || hr < full || hr > p.max_hist_len;
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          qo.ca[nb] = 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) qo.cb[nb][j] = 0.0f;
#pragma unroll
          for (int c = 0; c < D / 64; ++c) qo.qa[nb][c] = v4i{0, 0, 0, 0};
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      // a row that differs from the staged one, or a history ending inside the
      // split, anywhere in the group poisons the whole group
      const bool wave_bad = __any(bad);
      if (lane == 0) flags[wave] = wave_bad ? 1 : 0;
      __syncthreads();
      poison = (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
      __syncthreads();   // flags are read before anything overlays them
      const int n_pages = poison ? 0 : count;        // block-uniform
      float* mw = reinterpret_cast<float*>(smem + wave * kSlot);
      hist_wave<D, 16, false, 1, true>(p, g, ws0, n_pages, full, pid_lane, qo, smem, mw, poison, lane,
                                      smem + kRing + wave * kPlanes, wave, active);
      if (active) {
        // each request's 4-head partial into its own slot: (m, l, 0, 0, acc)
        constexpr int R = part_row(D);
#pragma unroll 4
        for (int e = lane; e < 16 * R; e += kWave) {
          const int h = e / R, k = e - h * R;
          const float v = mw[e];
          float* dst = p.hpart + (((size_t)(b + h / 4) * p.n_kv + g) * p.splits + split) * (size_t)4 * R +
                       (size_t)(h % 4) * R + k;
          *dst = (k == 1) ? (poison ? NAN : v) : (k < kPartAcc && k > 1) ? 0.0f : v;
        }
      }
      return;
    }
  }
  if constexpr (G == 4) {
    if (pid >= 0 && pid < n_packed) {
      // ---- a split inside the shared prefix for requests b .. b+PACK-1: one
      // 4*PACK-head wave reads each page once for all of them
      constexpr int GP = 4 * PACK;
      using RP = Ring<D, PACK, NG>;
      static_assert(GP * part_row(D) * 4 <= RP::kWaveBytes, "merge slot must fit in the wave's ring");
      const int per_split = p.packs * p.n_kv;
      const int split = pid / per_split, pk = (pid % per_split) / p.n_kv, g = pid % p.n_kv;
      const int b = PACK * pk;
      const int per_wave = (p.pps + 3) / 4;
      const int ws0 = split * p.pps + wave * per_wave;
      const int pe = split * p.pps + p.pps;   // split end; the prefix holds it whole
      const bool mine = lane < per_wave && ws0 + lane < pe;
      const int32_t* row = p.block_table + (size_t)b * p.max_pages;
      const int pid_lane = mine ? row[ws0 + lane] : -1;
      int pid_other[PACK - 1], hlr[PACK];
#pragma unroll
      for (int r = 1; r < PACK; ++r) pid_other[r - 1] = mine ? row[(size_t)r * p.max_pages + ws0 + lane] : -1;
      HistOperands<D, GP> qo;
      load_pack_operands<D, PACK>(p, b, g, lane, qo);
#pragma unroll
      for (int r = 0; r < PACK; ++r) hlr[r] = p.hist_len[b + r];
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      const int full = pe * kPage;   // every history of the pack must cover the split
      bool bad = false;
#pragma unroll
      for (int r = 0; r < PACK; ++r) bad |= hlr[r] < full || hlr[r] > p.max_hist_len;
#pragma unroll
      for (int r = 1; r < PACK; ++r) bad |= pid_other[r - 1] != pid_lane;
      if (__any(bad)) poison = true;
      const int count =
          __builtin_amdgcn_readfirstlane(poison ? 0 : max(0, min(ws0 + per_wave, pe) - ws0));
      uint8_t* ring = smem + wave * RP::kWaveBytes;
      hist_wave<D, GP, LM, NG>(p, g, ws0, count, full, pid_lane, qo, ring, reinterpret_cast<float*>(ring), poison,
                               lane);
      if (lane == 0) flags[wave] = poison ? 1 : 0;
      __syncthreads();
      const size_t rows = (size_t)4 * part_row(D);
      combine_block<GP, D, 4>(reinterpret_cast<const float*>(smem), RP::kWaveBytes / 4, flags,
                              p.hpart + (((size_t)b * p.n_kv + g) * p.splits + split) * rows, tid,
                              (size_t)p.n_kv * p.splits * rows);
      return;
    }
  }

  // ---- INT2 history split of one request: waves take contiguous page ranges
  int b, g, split;
  if (id >= rest0 && id < rest0 + n_rest) {
    const int j = id - rest0, unit = j % units;
    split = p.n_pref + j / units;
    b = unit / p.n_kv;
    g = unit % p.n_kv;
  } else {   // the prefix splits of the requests past the last whole pack
    const int j = id - n_packed - n_rest;
    split = j / (left * p.n_kv);
    b = p.packs * p.pack + (j / p.n_kv) % left;
    g = j % p.n_kv;
  }
  const int per_wave = (p.pps + 3) / 4;   // at most 64
  const int ws0 = split * p.pps + wave * per_wave;   // the wave's first page, before the history length clips it
  // The page ids of the wave's whole static range, the QK operands and the
  // history length are requested together: one memory round trip before the
  // first page copy instead of two.  Table entries past the history end are
  // loaded (in bounds) but never used.
  const int pid_lane = (lane < per_wave && ws0 + lane < p.max_pages)
                           ? p.block_table[(size_t)b * p.max_pages + ws0 + lane] : -1;
  HistOperands<D, G> qo;
  load_hist_operands<D, G>(p, b, g, lane, qo);
  int hl = p.hist_len[b];
  // This wait must be visible to the compiler (builtin, not inline assembly):
  // otherwise it still counts these loads as pending inside the page loop and
  // inserts vmcnt waits there that also drain every page copy in flight.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  if (hl < 0 || hl > p.max_hist_len) {
    poison = true;
    hl = 0;
  }
  const int hp = (hl + kPage - 1) / kPage;
  const int pe = min(split * p.pps + p.pps, hp);
  const int count = max(0, min(ws0 + per_wave, pe) - ws0);
  uint8_t* ring = smem + wave * RG::kWaveBytes;
  // the wave's merge slot [G][D+2] = (m, l, acc) overlays its own ring once the scan is done
  hist_wave<D, G, LM, NG, false, true>(p, g, ws0, count, hl, pid_lane, qo, ring, reinterpret_cast<float*>(ring), poison,
                                       lane);
  if (lane == 0) flags[wave] = poison ? 1 : 0;
  __syncthreads();
  combine_block<G, D>(reinterpret_cast<const float*>(smem), RG::kWaveBytes / 4, flags,
                      p.hpart + (((size_t)b * p.n_kv + g) * p.splits + split) * (size_t)G * part_row(D), tid);
}

// ---------------------------------------------------------------------------
// 3. merge: LSE over history splits, * R_V^T, LSE with BF16 chunks, normalise
// ---------------------------------------------------------------------------
// Online LSE merge of one head's partials (m, l, acc[D]) by a 256-thread
// block.  Thread (q, grp) owns channels 4q..4q+3 of the partials s = grp,
// grp + NG, ... (NG = kBlock / (D/4) groups): it issues the loads of up to
// kMergeRound of them (a float2 (m, l) and a float4 of acc each) before the
// first use, folds them into a running (m, l, acc) and moves to the next round;
// the NG group states are then combined through LDS.  acc is split in two
// sums: partials s < n_rot (history, still rotated) and the rest.
constexpr int kMergeRound = 12;

template <int D>
struct MergeShared {
  static constexpr int NQ = D / 4, NG = kBlock / NQ;
  float m[NG], l[NG];
  float4 a_rot[NG][NQ], a_plain[NG][NQ];
  float rot[D], plain[D];   // combined channel sums
};

// part_ptr(s): the head's row of partial s (16-byte aligned).  Returns the
// block-wide (M, L) and leaves the channel sums in sh.rot / sh.plain.
template <int D, typename PartPtr>
__device__ __forceinline__ float2 merge_head(PartPtr part_ptr, int n_rot, int nt, MergeShared<D>& sh, int tid) {
  constexpr int NQ = MergeShared<D>::NQ, NG = MergeShared<D>::NG;
  const int q = tid % NQ, grp = tid / NQ;
  float m = -INFINITY, l = 0.0f;
  float4 ar = make_float4(0.0f, 0.0f, 0.0f, 0.0f), ap = ar;
  for (int s0 = grp; s0 < nt; s0 += NG * kMergeRound) {
    float2 ml[kMergeRound];
    float4 av[kMergeRound];
#pragma unroll
    for (int k = 0; k < kMergeRound; ++k) {
      const int s = s0 + NG * k;
      if (s < nt) {
        const float* pp = part_ptr(s);
        ml[k] = *reinterpret_cast<const float2*>(pp);
        av[k] = *reinterpret_cast<const float4*>(pp + kPartAcc + 4 * q);
      } else {
        ml[k] = make_float2(-INFINITY, 0.0f);
        av[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
    }
    float rm = m;
#pragma unroll
    for (int k = 0; k < kMergeRound; ++k) rm = fmaxf(rm, ml[k].x);
    const float alpha = exp2_or_zero(m, rm);
    l *= alpha;
    ar = f4_scale(alpha, ar);
    ap = f4_scale(alpha, ap);
#pragma unroll
    for (int k = 0; k < kMergeRound; ++k) {
      const float f = exp2_or_zero(ml[k].x, rm);
      const float fr = s0 + NG * k < n_rot ? f : 0.0f;
      l = fmaf(f, ml[k].y, l);
      ar = f4_fma(fr, av[k], ar);
      ap = f4_fma(f - fr, av[k], ap);
    }
    m = rm;
  }
  if (q == 0) {
    sh.m[grp] = m;
    sh.l[grp] = l;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < NG; ++k) M = fmaxf(M, sh.m[k]);
  float L = 0.0f;
#pragma unroll
  for (int k = 0; k < NG; ++k) L = fmaf(exp2_or_zero(sh.m[k], M), sh.l[k], L);
  const float f = exp2_or_zero(m, M);
  sh.a_rot[grp][q] = f4_scale(f, ar);
  sh.a_plain[grp][q] = f4_scale(f, ap);
  __syncthreads();
  if (tid < D) {
    const float* r0 = reinterpret_cast<const float*>(&sh.a_rot[0][0]);
    const float* p0 = reinterpret_cast<const float*>(&sh.a_plain[0][0]);
    float sr = 0.0f, sp = 0.0f;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      sr += r0[k * D + tid];
      sp += p0[k * D + tid];
    }
    sh.rot[tid] = sr;
    sh.plain[tid] = sp;
  }
  __syncthreads();
  return make_float2(M, L);
}

// The output rotation out_i = sum_j A_j R_V[i][j] for NR consecutive rows i
// of R_V, read in whole rows: thread t holds columns 4c..4c+3 (c = t % (D/4))
// of rows RPT*rb .. RPT*rb + RPT-1 (rb = t / (D/4)), so each load
// instruction of a wave covers whole 512-byte rows (per-thread row segments
// would put every lane of an instruction on its own cache line).  The dot
// products over a row's column quads are then summed through LDS.
template <int D, int NR = D>
struct RvRows {
  static constexpr int QPR = D / 4, RB = kBlock / QPR, RPT = NR / RB, TPO = kBlock / NR;
  static constexpr int kStride = NR + 1;   // red[c][row]: conflict-free writes and sums
  float4 v[RPT];
};

// rv: the first of the NR rows
template <int D, int NR>
__device__ __forceinline__ void load_rv_rows(RvRows<D, NR>& r, const float* __restrict__ rv, int tid) {
  using T = RvRows<D, NR>;
  const int c = tid % T::QPR, rb = tid / T::QPR;
  const float4* src = reinterpret_cast<const float4*>(rv + (size_t)(T::RPT * rb) * D) + c;
#pragma unroll
  for (int k = 0; k < T::RPT; ++k) r.v[k] = src[(size_t)k * T::QPR];
}

// out row i = tid / TPO (of the NR rows) of A (D floats in LDS) times R_V^T;
// every thread of the row gets the value.  red: QPR * (NR + 1) floats of
// LDS.  Contains one barrier; the caller synchronises before red or A is
// written again.
template <int D, int NR>
__device__ __forceinline__ float rv_product(const RvRows<D, NR>& r, const float* A, float* red, int tid) {
  using T = RvRows<D, NR>;
  const int c = tid % T::QPR, rb = tid / T::QPR;
  const float4 a = reinterpret_cast<const float4*>(A)[c];
  float* dst = red + c * T::kStride + T::RPT * rb;
#pragma unroll
  for (int k = 0; k < T::RPT; ++k)
    dst[k] = fmaf(a.x, r.v[k].x, fmaf(a.y, r.v[k].y, fmaf(a.z, r.v[k].z, a.w * r.v[k].w)));
  __syncthreads();
  const int i = tid / T::TPO, h = tid % T::TPO;
  constexpr int CPT = T::QPR / T::TPO;   // column quads summed per thread
  float o = 0.0f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) o += red[(h * CPT + j) * T::kStride + i];
#pragma unroll
  for (int off = 1; off < T::TPO; off <<= 1) o += __shfl_xor(o, off, kWave);
  return o;
}

// Two blocks per query head, one per half of the output channels (each
// applies half of R_V's rows; both merge all of the head's partials):
//   out = (sum_hist f_s acc_s R_V^T + sum_bf16 f_s acc_s) / sum_all f_s l_s,
//   f_s = exp2(m_s - M) with M the maximum over every partial.
// The R_V rows are requested first, so their loads overlap the partials'.
template <int D>
__global__ __launch_bounds__(kBlock) void merge_kernel(DecodeDev p, int n_merge, DemoteDev dk, DemoteDev dv) {
  constexpr int NR = D / 2;
  using RV = RvRows<D, NR>;
  __shared__ MergeShared<D> sh;
  __shared__ float red[RV::QPR * RV::kStride];
  if ((int)blockIdx.x >= n_merge) {
    demote_step_block<D>(p, blockIdx.x - n_merge, dk, dv);
    return;
  }
  const int bh = blockIdx.x >> 1, half = blockIdx.x & 1;
  const int b = bh / p.Hq, h = bh % p.Hq, g = h / p.G, kh = h % p.G;
  const int tid = threadIdx.x;
  const size_t stride = (size_t)p.G * part_row(D);
  const float* hp = p.hpart + ((size_t)b * p.n_kv + g) * p.splits * stride + (size_t)kh * part_row(D);
  const float* bp = p.bpart + ((size_t)b * p.n_kv + g) * p.bf_blocks * stride + (size_t)kh * part_row(D);
  const int n = p.splits, nt = p.splits + p.bf_blocks;
  RV rv;
  load_rv_rows<D, NR>(rv, p.r_v + ((size_t)g * D + (size_t)half * NR) * D, tid);
  const float2 ML = merge_head<D>(
      [&](int s) { return s < n ? hp + (size_t)s * stride : bp + (size_t)(s - n) * stride; }, n, nt, sh, tid);
  // out_hist[i] = sum_j A_hist[j] R_V[g][i][j] for the half's rows i
  const float o = rv_product<D, NR>(rv, sh.rot, red, tid);
  const int i = half * NR + tid / RV::TPO;
  if (tid % RV::TPO == 0) {
    const float L = ML.y;
    float out;
    if (isnan(L)) out = NAN;
    else out = (L > 0.0f) ? (o + sh.plain[i]) / L : 0.0f;
    p.out[(size_t)bh * D + i] = out;
  }
}

// One (request, KV head) per block, for launches whose heads have few partials
// each (large batches, few splits): the R_V rows are loaded once for the
// unit's G heads rather than once per head, and the partials of every head are
// requested kUnitRound at a time (one round up to 16 partials), the rounds
// combined online.  Thread (h, q) owns channels 4q..4q+3 of head h.
constexpr int kUnitMaxParts = 4 * kUnitRound;

template <int D, int G>
__global__ __launch_bounds__(kBlock) void merge_unit_kernel(DecodeDev p, int n_merge, DemoteDev dk, DemoteDev dv) {
  constexpr int QPR = D / 4, R = part_row(D), TPO = RvRows<D, D>::TPO;
  static_assert(G * QPR <= kBlock, "one (head, channel quad) per thread");
  __shared__ __attribute__((aligned(16))) float arot[G][D];
  __shared__ __attribute__((aligned(16))) float aplain[G][D];
  __shared__ float Ls[G];
  __shared__ float red[RvRows<D, D>::QPR * RvRows<D, D>::kStride];
  if ((int)blockIdx.x >= n_merge) {
    demote_step_block<D>(p, blockIdx.x - n_merge, dk, dv);
    return;
  }
  const int unit = blockIdx.x, b = unit / p.n_kv, g = unit % p.n_kv;
  const int tid = threadIdx.x;
  const int i = tid / TPO;   // output channel of this thread
  RvRows<D, D> rv;
  load_rv_rows<D, D>(rv, p.r_v + (size_t)g * D * D, tid);
  const size_t stride = (size_t)G * R;
  const int n = p.splits, nt = p.splits + p.bf_blocks;
  const float* hb = p.hpart + (size_t)unit * n * stride;
  const float* bb = p.bpart + (size_t)unit * p.bf_blocks * stride;
  if (tid < G * QPR) {
    const int h = tid / QPR, q = tid % QPR;
    float M = -INFINITY, L = 0.0f;
    float4 ar = make_float4(0.0f, 0.0f, 0.0f, 0.0f), ap = ar;
    for (int s0 = 0; s0 < nt; s0 += kUnitRound) {
      float2 ml[kUnitRound];
      float4 av[kUnitRound];
#pragma unroll
      for (int k = 0; k < kUnitRound; ++k) {
        const int s = s0 + k;
        if (s < nt) {
          const float* pp = (s < n ? hb + (size_t)s * stride : bb + (size_t)(s - n) * stride) + h * R;
          ml[k] = *reinterpret_cast<const float2*>(pp);
          av[k] = *reinterpret_cast<const float4*>(pp + kPartAcc + 4 * q);
        } else {
          ml[k] = make_float2(-INFINITY, 0.0f);
          av[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
      }
      // the round's maximum; the sums so far move to it (on the first round M
      // is -inf and they are still zero)
      float Mr = M;
#pragma unroll
      for (int k = 0; k < kUnitRound; ++k) Mr = fmaxf(Mr, ml[k].x);
      if (s0 > 0) {
        const float c = exp2_or_zero(M, Mr);
        L *= c;
        ar = f4_fma(c, ar, make_float4(0.0f, 0.0f, 0.0f, 0.0f));
        ap = f4_fma(c, ap, make_float4(0.0f, 0.0f, 0.0f, 0.0f));
      }
      M = Mr;
#pragma unroll
      for (int k = 0; k < kUnitRound; ++k) {
        const float f = exp2_or_zero(ml[k].x, M);
        const float fr = s0 + k < n ? f : 0.0f;   // history partials are still rotated
        L = fmaf(f, ml[k].y, L);
        ar = f4_fma(fr, av[k], ar);
        ap = f4_fma(f - fr, av[k], ap);
      }
    }
    *reinterpret_cast<float4*>(&arot[h][4 * q]) = ar;
    *reinterpret_cast<float4*>(&aplain[h][4 * q]) = ap;
    if (q == 0) Ls[h] = L;
  }
  __syncthreads();
  // out[h][i] = (sum_j A_hist[h][j] R_V[g][i][j] + A_bf16[h][i]) / L[h]
  for (int h = 0; h < G; ++h) {
    if (h > 0) __syncthreads();   // every thread has read red for head h - 1
    const float o = rv_product<D, D>(rv, arot[h], red, tid);
    if (tid % TPO == 0) {
      const float L = Ls[h];
      float out;
      if (isnan(L)) out = NAN;
      else out = (L > 0.0f) ? (o + aplain[h][i]) / L : 0.0f;
      p.out[((size_t)b * p.Hq + (size_t)g * G + h) * D + i] = out;
    }
  }
}

// The per-unit merge when each head's partials fit in one round and the G
// heads' channel quads fit in one block.  n_dem demotion blocks follow the
// merge blocks.
template <int D>
bool launch_merge_unit(const DecodeDev& dv, unsigned n_dem, const DemoteDev& mk, const DemoteDev& mv,
                       hipStream_t stream) {
  // one round, or several when the batch gives every compute unit a block of its own
  const int parts = dv.splits + dv.bf_blocks;
  if (dv.G * (D / 4) > kBlock || parts > kUnitMaxParts) return false;
  if (parts > kUnitRound && (long)dv.B * dv.n_kv < 128) return false;
  const int units = dv.B * dv.n_kv;
  const unsigned grid = (unsigned)units + n_dem;
  switch (dv.G) {
    case 1: merge_unit_kernel<D, 1><<<grid, kBlock, 0, stream>>>(dv, units, mk, mv); break;
    case 2: merge_unit_kernel<D, 2><<<grid, kBlock, 0, stream>>>(dv, units, mk, mv); break;
    case 4: merge_unit_kernel<D, 4><<<grid, kBlock, 0, stream>>>(dv, units, mk, mv); break;
    case 8: merge_unit_kernel<D, 8><<<grid, kBlock, 0, stream>>>(dv, units, mk, mv); break;
    default:
      if constexpr (16 * (D / 4) <= kBlock) merge_unit_kernel<D, 16><<<grid, kBlock, 0, stream>>>(dv, units, mk, mv);
      else return false;
      break;
  }
  return true;
}

// Launch 3: the merge (none with batch 0), then the step's demotions.
template <int D>
void launch_merge(const DecodeDev& dv, const DemoteDev& mk, const DemoteDev& mv, hipStream_t stream) {
  const unsigned n_dem = (unsigned)((mk.n_tok + mv.n_tok) * dv.n_kv);
  if (dv.B > 0 && launch_merge_unit<D>(dv, n_dem, mk, mv, stream)) return;
  const int n_merge = 2 * dv.B * dv.Hq;   // two blocks per query head
  if (n_merge + n_dem > 0) merge_kernel<D><<<(unsigned)n_merge + n_dem, kBlock, 0, stream>>>(dv, n_merge, mk, mv);
}

// ---- BF16 paged comparator ---------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(kBlock, (G > 8 ? 1 : 2)) void bf16_paged_kernel(Bf16Dev p) {
  constexpr int kWaveLds = bf16_lds_bytes<D, G>();
  constexpr int kMrg = 4 * G * part_row(D) * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kWaveLds > kMrg ? 4 * kWaveLds : kMrg];
  __shared__ int flags[4];
  const int b = blockIdx.z, g = blockIdx.y, x = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  WaveAcc<D, G> st;
  acc_init(st);
  bool poison = false;
  bf16x8 qa[D / 32];
  bf16_q_operands<D, G>(qa, p.q + ((size_t)b * p.Hq + g * G) * D, lane);
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
    const int nv = min(kPage, cl - pg * kPage);
    Bf16Tile<D> tile;
    bf16_load<D, false>(tile, p.k_pages + off, p.v_pages + off, nv, lane);
    bf16_compute<D, G>(st, tile, qa, p.sm_log2, nv, smem + wave * kWaveLds, lane);
  }
  __syncthreads();   // the merge area overlays the tiles' LDS
  float* mrg = reinterpret_cast<float*>(smem);
  store_wave_state<D, G>(st, mrg + wave * G * part_row(D), lane, false);
  if (lane == 0) flags[wave] = poison ? 1 : 0;
  __syncthreads();
  combine_block<G, D>(mrg, G * part_row(D), flags, p.part + (((size_t)b * p.n_kv + g) * p.splits + x) * (size_t)G * part_row(D),
                      tid);
}

template <int D>
__global__ __launch_bounds__(kBlock) void merge_plain_kernel(Bf16Dev p) {
  __shared__ MergeShared<D> sh;
  const int bh = blockIdx.x;
  const int b = bh / p.Hq, h = bh % p.Hq, g = h / p.G, kh = h % p.G;
  const int tid = threadIdx.x;
  const size_t stride = (size_t)p.G * part_row(D);
  const float* pp = p.part + ((size_t)b * p.n_kv + g) * p.splits * stride + (size_t)kh * part_row(D);
  const float2 ML = merge_head<D>([&](int s) { return pp + (size_t)s * stride; }, 0, p.splits, sh, tid);
  if (tid < D) {
    const float L = ML.y;
    float o;
    if (isnan(L)) o = NAN;
    else o = (L > 0.0f) ? sh.plain[tid] / L : 0.0f;
    p.out[(size_t)bh * D + tid] = o;
  }
}

template <int D, int G>
void launch_main(const DecodeDev& dv, hipStream_t stream) {
  const long units = (long)dv.B * dv.n_kv;
  const long blocks = (long)dv.n_pref * dv.pack_units * dv.n_kv + (long)(dv.splits - dv.n_pref) * units +
                      (long)dv.n_pref * (dv.B - dv.packs * dv.pack) * dv.n_kv + units * dv.bf_blocks;
  if (blocks == 0) return;
  const dim3 grid((unsigned)blocks);
  if (dv.ng == 2) {   // 64-channel groups at d = 128, 32-channel ones at d = 64
    if (dv.lm) decode_main_kernel<D, G, true, 2><<<grid, kBlock, 0, stream>>>(dv);
    else decode_main_kernel<D, G, false, 2><<<grid, kBlock, 0, stream>>>(dv);
    return;
  }
  if constexpr (D == 128) {
    if (dv.ng == 4) {   // 32-channel groups
      if (dv.lm) decode_main_kernel<D, G, true, 4><<<grid, kBlock, 0, stream>>>(dv);
      else decode_main_kernel<D, G, false, 4><<<grid, kBlock, 0, stream>>>(dv);
      return;
    }
    if constexpr (G == 4) {
      // four-request packs (uniform codebook, whole-head groups): the whole launch runs at the
      // 16-head waves' two waves per SIMD (their own launch, leaving three per SIMD to the other
      // blocks, measured 199 against 167 us per step on the 28-request layer)
      if (!dv.lm && dv.n_pref > 0 && dv.pack == 4) {
        decode_main_kernel<D, 4, false, 1, 4><<<grid, kBlock, 0, stream>>>(dv);
        return;
      }
    }
  }
  if (dv.lm) decode_main_kernel<D, G, true, 1><<<grid, kBlock, 0, stream>>>(dv);
  else decode_main_kernel<D, G, false, 1><<<grid, kBlock, 0, stream>>>(dv);
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

// (scale, zero) groups per head of the pools a decode reads
int decode_groups(const oscar_decode_args& a) {
  return a.group_channels > 0 && a.group_channels < a.head_dim ? a.head_dim / a.group_channels : 1;
}

// blocks per CU of the scan variant launch_main picks for these formats (the
// four-request packs of group size 4 included, whichever is smaller)
template <int D, int G>
int scan_blocks_per_cu_of(bool lm, int ng) {
  int b;
  if (ng == 2) {
    b = lm ? scan_blocks_per_cu<D, G, true, 2, 2>() : scan_blocks_per_cu<D, G, false, 2, 2>();
  } else if (ng == 4) {
    if constexpr (D == 128) b = lm ? scan_blocks_per_cu<D, G, true, 4, 2>() : scan_blocks_per_cu<D, G, false, 4, 2>();
    else b = 1;   // not reached: four groups need head_dim 128
  } else {
    b = lm ? scan_blocks_per_cu<D, G, true, 1, 2>() : scan_blocks_per_cu<D, G, false, 1, 2>();
    if constexpr (D == 128 && G == 4)
      if (!lm) b = std::min(b, scan_blocks_per_cu<D, 4, false, 1, 4>());
  }
  return b;
}

template <int D>
int scan_blocks_per_cu_g(int G, bool lm, int ng) {
  switch (G) {
    case 1: return scan_blocks_per_cu_of<D, 1>(lm, ng);
    case 2: return scan_blocks_per_cu_of<D, 2>(lm, ng);
    case 4: return scan_blocks_per_cu_of<D, 4>(lm, ng);
    case 8: return scan_blocks_per_cu_of<D, 8>(lm, ng);
    default: return scan_blocks_per_cu_of<D, 16>(lm, ng);
  }
}

DecodeDev make_dev(const oscar_decode_args& a, const DecodePlan& plan, char* ws) {
  DecodeDev dv{};
  dv.B = a.batch; dv.Hq = a.n_q_heads; dv.n_kv = a.n_kv_heads; dv.G = a.n_q_heads / a.n_kv_heads;
  dv.NB = (dv.G + 3) / 4;
  dv.sink_cap = a.sink_cap; dv.recent_cap = a.recent_cap;
  dv.max_hist_len = a.max_hist_len; dv.max_pages = a.max_pages;
  dv.splits = plan.splits; dv.pps = plan.pages_per_split;
  dv.chunks = plan.chunks; dv.sink_chunks = plan.sink_chunks;
  // with many units a BF16 block takes all of its unit's chunks, else one
  dv.bf_cpb = (long)a.batch * a.n_kv_heads >= 128 && plan.chunks > 0 ? plan.chunks : 1;
  dv.bf_blocks = (plan.chunks + dv.bf_cpb - 1) / dv.bf_cpb;
  dv.lm = a.codebook == OSCAR_CODEBOOK_LLOYD_MAX ? 1 : 0;
  dv.ng = decode_groups(a);
  // pack the splits that lie wholly inside a shared prefix (group size 4, two or
  // more requests): four requests per wave with the uniform codebook and
  // whole-head groups at d = 128 (the 16-head wave fits two per SIMD there),
  // else two
  const bool quad = quad_packs(a);
  dv.pack = quad ? 4 : 2;
  dv.packs = a.batch / dv.pack;
  dv.n_pref = (dv.G == 4 && dv.packs > 0 && plan.splits > 0) ? std::min(plan.splits, a.shared_pages / plan.pages_per_split)
                                                            : 0;
  // the cascade's plan keeps splits within 64 pages (abi.hip plans with decode_cascade too)
  dv.casc = quad && decode_cascade(a) && dv.n_pref > 0 && plan.pages_per_split <= kCascadeMaxPagesPerSplit ? 1 : 0;
  dv.pack_units = dv.casc ? (dv.packs + 3) / 4 : dv.packs;
  dv.sm_log2 = a.sm_scale * kLog2e;
  dv.n_pages = a.n_pages;
  dv.q = a.q; dv.sink_k = a.sink_k; dv.sink_v = a.sink_v; dv.recent_k = a.recent_k; dv.recent_v = a.recent_v;
  dv.sink_len = a.sink_len; dv.recent_len = a.recent_len; dv.hist_len = a.hist_len;
  dv.block_table = a.block_table;
  dv.k_codes = a.k_codes; dv.v_codes = a.v_codes;
  dv.k_sz = reinterpret_cast<const uint32_t*>(a.k_sz);
  dv.v_sz = reinterpret_cast<const uint32_t*>(a.v_sz);
  dv.r_k = a.r_k; dv.r_v = a.r_v; dv.out = a.out;
  dv.qdig = reinterpret_cast<uint8_t*>(ws + plan.off_qdig);
  dv.qa = reinterpret_cast<float*>(ws + plan.off_qa);
  dv.qb = reinterpret_cast<float*>(ws + plan.off_qb);
  dv.hpart = reinterpret_cast<float*>(ws + plan.off_hpart);
  dv.bpart = reinterpret_cast<float*>(ws + plan.off_bpart);
  return dv;
}

}  // namespace

hipError_t launch_decode_phase(int phase, const oscar_decode_args& a, const DecodePlan& plan, char* ws,
                               hipStream_t stream, const oscar_demote_args* demote_k,
                               const oscar_demote_args* demote_v) {
  const DecodeDev dv = make_dev(a, plan, ws);
  const unsigned nbh = (unsigned)a.batch * (unsigned)a.n_q_heads;
  const bool d128 = a.head_dim == 128;
  if (phase == kPhaseRotate) {
    if (plan.splits > 0 && nbh > 0) {
      if (d128) prepare_kernel<128><<<2 * nbh, kBlock, 0, stream>>>(dv);
      else prepare_kernel<64><<<2 * nbh, kBlock, 0, stream>>>(dv);
    }
  } else if (phase == kPhaseMerge) {
    const DemoteDev mk = make_demote(demote_k), mv = make_demote(demote_v);
    if (d128) launch_merge<128>(dv, mk, mv, stream);
    else launch_merge<64>(dv, mk, mv, stream);
  } else if (a.batch > 0) {
    if (d128) launch_main_g<128>(dv, stream);
    else launch_main_g<64>(dv, stream);
  }
  return hipGetLastError();
}

long scan_resident_blocks(const oscar_decode_args& a) {
  const int G = a.n_q_heads / a.n_kv_heads, ng = decode_groups(a);
  const bool lm = a.codebook == OSCAR_CODEBOOK_LLOYD_MAX;
  const int b = a.head_dim == 128 ? scan_blocks_per_cu_g<128>(G, lm, ng) : scan_blocks_per_cu_g<64>(G, lm, ng);
  return (long)kResidentBlocks * std::max(b, 1) / 2;
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
  if (a.head_dim == 128) merge_plain_kernel<128><<<nbh, kBlock, 0, stream>>>(dv);
  else merge_plain_kernel<64><<<nbh, kBlock, 0, stream>>>(dv);
  return hipGetLastError();
}

}  // namespace oscar

"""Seeded synthetic inputs for the three-segment INT2 decode path.

This module is shared by the oracle-side tests and by the HIP-side tests and
benchmark. It draws random numbers, converts them to the storage dtypes
(bf16 bit patterns), builds block tables, and produces the two offline
calibration artefacts that both sides take as *inputs*: the fixed per-head
rotations R_K, R_V and the per-layer clip thresholds tau_K, tau_V.

It computes none of the hot path: no clipping, no INT2 quantisation, no
packing, no attention.  The calibration stand-ins follow the description of
the offline phase in the gist.science technical summary of "OSCAR: Offline
Spectral Covariance-Aware Rotation for 2-bit KV Cache Quantization"
(section 2.2A): an eigenbasis U of a covariance, times a normalised Hadamard
matrix, times a bit-reversal permutation, and a clip threshold taken from
rotated calibration activations.  The covariance here is a seeded random SPD
matrix instead of a model's query / score-weighted value covariance (no model
weights or datasets are available), and the threshold is the 99.9th
percentile of the rotated |values|.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

PAGE = 64          # tokens per history page
SINK_CAP = 64      # BF16 sink window (myzaker article, serving pipeline section)
RECENT_CAP = 256   # BF16 recent window (same section)
BASE_SEED = 20260519


# --------------------------------------------------------------------------
# dtype helpers (storage conversions only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits.

    Inputs are finite (the generator never produces NaN/Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# offline-calibration stand-ins (inputs to both sides)
# --------------------------------------------------------------------------
def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (power of two), scaled by 1/sqrt(d)."""
    if d < 1 or d & (d - 1):
        raise ValueError("Hadamard order must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / math.sqrt(d)


def bit_reversal_perm(d: int) -> np.ndarray:
    """Permutation matrix P with P[i, br(i)] = 1, br reversing the log2(d) index bits."""
    nb = d.bit_length() - 1
    if 1 << nb != d:
        raise ValueError("bit reversal needs a power-of-two size")
    br = np.array([int(format(i, f"0{nb}b")[::-1], 2) if nb else 0 for i in range(d)])
    p = np.zeros((d, d), dtype=np.float64)
    p[np.arange(d), br] = 1.0
    return p


def spd_eigenbasis(d: int, rng: np.random.Generator):
    """Seeded random SPD covariance C = A A^T / d + 1e-3 I and its eigenbasis.

    Columns ordered by descending eigenvalue; each column's sign is fixed so its
    largest-magnitude entry is positive (stable across LAPACK builds)."""
    a = rng.standard_normal((d, d))
    c = a @ a.T / d + 1e-3 * np.eye(d)
    w, u = np.linalg.eigh(c)
    order = np.argsort(-w, kind="stable")
    w, u = w[order], u[:, order]
    idx = np.argmax(np.abs(u), axis=0)
    sign = np.sign(u[idx, np.arange(d)])
    u = u * sign
    return c, w, u


def make_rotation(d: int, rng: np.random.Generator) -> np.ndarray:
    """R = U . H . P_br as float32 (row-vector convention: y = x R)."""
    _, _, u = spd_eigenbasis(d, rng)
    return (u @ hadamard(d) @ bit_reversal_perm(d)).astype(np.float32)


def clip_threshold(x_bits: np.ndarray, rot: np.ndarray, max_tokens: int = 8192) -> np.float32:
    """99.9th percentile of |x R| over tokens, heads and channels (numpy linear
    interpolation).  x_bits: bf16 [n_tok][n_kv][d]; rot: [n_kv][d][d].  A
    deterministic prefix of at most ``max_tokens`` tokens is the calibration set."""
    xs = bf16_bits_to_f32(x_bits[:max_tokens]).astype(np.float64)
    vals = [np.abs(xs[:, g, :] @ rot[g].astype(np.float64)).ravel() for g in range(rot.shape[0])]
    return np.float32(np.percentile(np.concatenate(vals), 99.9))


# --------------------------------------------------------------------------
# activations
# --------------------------------------------------------------------------
def outlier_channels(rng: np.random.Generator, n_kv: int, d: int, k: int) -> np.ndarray:
    """k distinct channels per KV head, fixed for all tokens and requests."""
    return np.stack([rng.choice(d, size=k, replace=False) for _ in range(n_kv)])


def kv_tokens(rng: np.random.Generator, shape_prefix, n_kv: int, d: int,
              outl: np.ndarray, factor: float = 20.0) -> np.ndarray:
    """bf16 N(0,1) activations of shape prefix+(n_kv, d) with outlier channels scaled."""
    x = rng.standard_normal(tuple(shape_prefix) + (n_kv, d), dtype=np.float32)
    for g in range(n_kv):
        x[..., g, outl[g]] *= np.float32(factor)
    return f32_to_bf16_bits(x)


# --------------------------------------------------------------------------
# configurations (the five workloads)
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class DecodeShape:
    name: str
    batch: int
    n_q_heads: int
    n_kv: int
    head_dim: int
    context: int            # L per request = sink + history + recent
    shared_hist_pages: int = 0   # leading history pages shared by every request
    n_outliers: int = 3

    @property
    def hist_len(self) -> int:
        return max(0, self.context - SINK_CAP - RECENT_CAP)

    @property
    def hist_pages(self) -> int:
        return -(-self.hist_len // PAGE)


TINY = DecodeShape("tiny-1layer-b1-h4kv2-d64-L1024", 1, 4, 2, 64, 1024)
QWEN3_8B_32K = DecodeShape("qwen3-8b-layer-b1-h32kv8-d128-L32768", 1, 32, 8, 128, 32768)
QWEN3_32B_100K = DecodeShape("qwen3-32b-layer-b1-h64kv8-d128-L100000", 1, 64, 8, 128, 100000)
QWEN3_8B_B28_100K = DecodeShape("qwen3-8b-layer-b28-h32kv8-d128-L100000-prefix90k",
                                28, 32, 8, 128, 100000, shared_hist_pages=90000 // PAGE)

DECODE_SHAPES = {0: TINY, 1: QWEN3_8B_32K, 3: QWEN3_32B_100K, 4: QWEN3_8B_B28_100K}


def seeds(config_index: int, n: int = 10):
    return np.random.SeedSequence(BASE_SEED + config_index).spawn(n)


def _page_ids(shape: DecodeShape, rng: np.random.Generator):
    """Block table [B][max_pages] and number of physical pages.

    History token t of request b lives in page table[b][t // 64] at slot t % 64.
    With shared pages, the first ``shared_hist_pages`` entries of every row are
    the same physical ids (a prefix-cache hit).  Physical ids are a seeded
    shuffle of the pool."""
    hp = shape.hist_pages
    shared = min(shape.shared_hist_pages, hp)
    private = hp - shared
    n_pages = shared + shape.batch * private
    perm = rng.permutation(n_pages).astype(np.int32)
    table = np.empty((shape.batch, max(hp, 1)), dtype=np.int32)
    table[:, :] = -1
    for b in range(shape.batch):
        table[b, :shared] = perm[:shared]
        table[b, shared:hp] = perm[shared + b * private: shared + (b + 1) * private]
    return table, n_pages


def make_decode_config(index: int, materialize_history: bool = True,
                       shape: DecodeShape | None = None, seed_index: int | None = None):
    """Synthetic decode-layer inputs for one of the decode workloads.

    Returns a dict of numpy arrays.  ``hist_k``/``hist_v`` (bf16 [n_hist][n_kv][d])
    are the history tokens to be demoted, in the order of ``hist_slot`` (int32,
    physical page * 64 + offset).  With ``materialize_history=False`` no history
    activations are drawn (used for the 28-request workload, whose pages are
    synthesised directly by :func:`random_pages`)."""
    shape = shape or DECODE_SHAPES[index]
    ss = seeds(index if seed_index is None else seed_index)
    r_q, r_k, r_v, r_ok, r_ov, r_rk, r_rv, r_tab, r_ring, r_x = (np.random.default_rng(s) for s in ss)
    B, Hq, nkv, d = shape.batch, shape.n_q_heads, shape.n_kv, shape.head_dim
    outk = outlier_channels(r_ok, nkv, d, shape.n_outliers)
    outv = outlier_channels(r_ov, nkv, d, shape.n_outliers)
    q = f32_to_bf16_bits(r_q.standard_normal((B, Hq, d), dtype=np.float32))
    sink_k = kv_tokens(r_k, (B, SINK_CAP), nkv, d, outk).transpose(0, 2, 1, 3).copy()
    sink_v = kv_tokens(r_v, (B, SINK_CAP), nkv, d, outv).transpose(0, 2, 1, 3).copy()
    rec_k = kv_tokens(r_k, (B, RECENT_CAP), nkv, d, outk).transpose(0, 2, 1, 3).copy()
    rec_v = kv_tokens(r_v, (B, RECENT_CAP), nkv, d, outv).transpose(0, 2, 1, 3).copy()
    L = shape.context
    sink_len = np.full(B, min(L, SINK_CAP), dtype=np.int32)
    recent_len = np.full(B, min(max(L - SINK_CAP, 0), RECENT_CAP), dtype=np.int32)
    hist_len = np.full(B, shape.hist_len, dtype=np.int32)
    table, n_pages = _page_ids(shape, r_tab)
    r_kr = np.stack([make_rotation(d, r_rk) for _ in range(nkv)])
    r_vr = np.stack([make_rotation(d, r_rv) for _ in range(nkv)])
    cfg = dict(shape=shape, name=shape.name, batch=B, n_q_heads=Hq, n_kv=nkv, head_dim=d,
               sm_scale=np.float32(1.0 / math.sqrt(d)), q=q,
               sink_k=sink_k, sink_v=sink_v, recent_k=rec_k, recent_v=rec_v,
               sink_len=sink_len, recent_len=recent_len, hist_len=hist_len,
               block_table=table, n_pages=n_pages, r_k=r_kr, r_v=r_vr,
               outliers_k=outk, outliers_v=outv)
    if materialize_history:
        # unique history tokens: the shared prefix once, then each request's private part
        slots = []
        hp, shared = shape.hist_pages, min(shape.shared_hist_pages, shape.hist_pages)
        for b in range(B):
            t0 = 0 if b == 0 else shared * PAGE
            t = np.arange(t0, shape.hist_len)
            slots.append(table[b, t // PAGE] * PAGE + t % PAGE)
        hist_slot = np.concatenate(slots).astype(np.int32) if slots else np.zeros(0, np.int32)
        n_hist = hist_slot.size
        hist_k = kv_tokens(r_x, (n_hist,), nkv, d, outk)
        hist_v = kv_tokens(r_x, (n_hist,), nkv, d, outv)
        cfg.update(hist_k=hist_k, hist_v=hist_v, hist_slot=hist_slot,
                   tau_k=clip_threshold(hist_k, r_kr), tau_v=clip_threshold(hist_v, r_vr))
    return cfg


def random_pages(rng: np.random.Generator, n_pages: int, n_kv: int, d: int, sigma: float):
    """Directly synthesised INT2 pages (uniform random 2-bit codes in every
    byte, per-token fp16 scale/zero drawn around the statistics of rotated,
    clipped activations of standard deviation ``sigma``).  Random bytes are
    valid in any in-page layout.  Returns (codes uint8 [n_pages][n_kv][64*d/4],
    scale_zero uint16 [n_pages][n_kv][64][2])."""
    codes = rng.integers(0, 256, size=(n_pages, n_kv, PAGE * d // 4), dtype=np.uint8)
    zero = rng.uniform(-3.2 * sigma, -2.2 * sigma, size=(n_pages, n_kv, PAGE)).astype(np.float16)
    scale = rng.uniform(1.4 * sigma, 2.1 * sigma, size=(n_pages, n_kv, PAGE)).astype(np.float16)
    sz = np.stack([scale.view(np.uint16), zero.view(np.uint16)], axis=-1)
    return codes, sz


def make_bulk_demotion_config(n_tok: int = 131072, n_kv: int = 8, d: int = 128, seed_index: int = 2):
    """Bulk demotion workload: n_tok tokens x n_kv heads x d for K and V,
    bf16 N(0,1) with 2% outlier channels (ceil(0.02 d) = 3 per head at d=128)
    scaled x20, written into 64-token pages in a seeded shuffled page order."""
    ss = seeds(seed_index)
    r_k, r_v, r_ok, r_ov, r_rk, r_rv, r_tab = (np.random.default_rng(s) for s in ss[:7])
    n_out = max(1, math.ceil(0.02 * d))
    outk = outlier_channels(r_ok, n_kv, d, n_out)
    outv = outlier_channels(r_ov, n_kv, d, n_out)
    xk = kv_tokens(r_k, (n_tok,), n_kv, d, outk)
    xv = kv_tokens(r_v, (n_tok,), n_kv, d, outv)
    n_pages = -(-n_tok // PAGE)
    perm = r_tab.permutation(n_pages).astype(np.int64)
    t = np.arange(n_tok)
    dst = (perm[t // PAGE] * PAGE + t % PAGE).astype(np.int32)
    rk = np.stack([make_rotation(d, r_rk) for _ in range(n_kv)])
    rv = np.stack([make_rotation(d, r_rv) for _ in range(n_kv)])
    return dict(name=f"bulk-demotion-{n_tok}tok-kv{n_kv}-d{d}", x_k=xk, x_v=xv, dst_slot=dst,
                n_pages=n_pages, r_k=rk, r_v=rv, n_kv=n_kv, head_dim=d,
                tau_k=clip_threshold(xk, rk), tau_v=clip_threshold(xv, rv))


def bf16_context_pages(cfg: dict, rng: np.random.Generator | None = None):
    """The same layer held entirely in BF16 (for the BF16 decode comparator).

    The context of request b is its sink, its history (the unrotated bf16
    originals) and its recent window, in that order, stored in 64-token pages
    [n_pages][n_kv][64][d] behind a shuffled block table.  Shared INT2 history
    pages map to shared BF16 pages of the same tokens (context pages
    1 .. shared_hist_pages, since the 64-token sink fills context page 0).
    Needs the materialised history (``hist_k``/``hist_v``)."""
    rng = rng or np.random.default_rng(seeds(99)[0])
    shape: DecodeShape = cfg["shape"]
    B, nkv, d = cfg["batch"], cfg["n_kv"], cfg["head_dim"]
    L = shape.context
    S = min(shape.shared_hist_pages, shape.hist_pages)
    if S and SINK_CAP % PAGE:
        raise ValueError("shared prefix needs a page-aligned sink")
    n_ctx_pages = -(-L // PAGE)
    per_req = n_ctx_pages - S
    n_pages = S + B * per_req
    perm = rng.permutation(n_pages).astype(np.int32)
    s0 = SINK_CAP // PAGE
    table = np.empty((B, n_ctx_pages), dtype=np.int32)
    for b in range(B):
        own = perm[S + b * per_req: S + (b + 1) * per_req]
        table[b, :s0] = own[:s0]
        table[b, s0:s0 + S] = perm[:S]
        table[b, s0 + S:] = own[s0:]
    kp = np.zeros((n_pages, nkv, PAGE, d), dtype=np.uint16)
    vp = np.zeros_like(kp)
    shared_tok = S * PAGE
    private_tok = shape.hist_len - shared_tok
    t_hist = np.arange(shape.hist_len)
    for b in range(B):
        uniq = np.where(t_hist < shared_tok, t_hist,
                        shared_tok + b * private_tok + (t_hist - shared_tok))
        hk, hv = cfg["hist_k"][uniq], cfg["hist_v"][uniq]
        ks = np.concatenate([cfg["sink_k"][b].transpose(1, 0, 2)[: cfg["sink_len"][b]], hk,
                             cfg["recent_k"][b].transpose(1, 0, 2)[: cfg["recent_len"][b]]])
        vs = np.concatenate([cfg["sink_v"][b].transpose(1, 0, 2)[: cfg["sink_len"][b]], hv,
                             cfg["recent_v"][b].transpose(1, 0, 2)[: cfg["recent_len"][b]]])
        t = np.arange(ks.shape[0])
        pg, off = table[b, t // PAGE], t % PAGE
        kp[pg, :, off, :] = ks
        vp[pg, :, off, :] = vs
    ctx_len = np.full(B, L, dtype=np.int32)
    return dict(k_pages=kp, v_pages=vp, block_table=table, ctx_len=ctx_len, n_pages=n_pages)

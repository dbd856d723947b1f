"""Oracle: decode attention over the three-segment cache (test infrastructure only).

Follows [ZAKER]'s serving pipeline: a BF16 sink (up to 64 tokens), INT2
history and a BF16 recent window (up to 256 tokens) are attended by the one
new query, and the INT2 and BF16 parts combine through an online softmax.
It also follows [CSDN] 3.1 and [GIST] 2.2B: INT2 history is loaded,
dequantised with its scale/zero point and inverse-rotated before ordinary
attention.  The history is stored after the fixed rotation and clipping.  The
BF16 windows are stored unrotated.

The oracle takes the literal reading: it inverse-rotates every dequantised
history token (x_hat R^T) and then runs softmax attention in float64 over the
materialised keys and values.  Readings where the pages are silent:

* one decode query per request attends to every cached token of its request
  (no causal mask inside the cache); the new token is already in the recent
  window;
* logits are sm_scale * q.k with sm_scale passed in (1/sqrt(d) by default);
* grouped-query attention: query head h uses KV head h // (Hq / n_kv);
* a request with no cached tokens at all gets an all-zero output row;
* the output is float32.
"""
from __future__ import annotations

import numpy as np

from .quant import PAGE, UNIFORM, bf16_to_f64, code_levels, f16_bits_to_f64, read_history_codes


def attn_plain(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """softmax(sm_scale * q K^T) V for query rows q [h, d], keys K [n, d],
    values V [n, d], all float64.  Empty n gives zeros."""
    q = np.asarray(q, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros((q.shape[0], V.shape[1]), dtype=np.float64)
    logits = (q @ K.T) * np.float64(sm_scale)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    return (p @ V) / p.sum(axis=1, keepdims=True)


def attn_partial(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """Unnormalised partial over a subset of tokens: (m, l, acc) with
    m = max logit, l = sum exp(logit - m), acc = sum exp(logit - m) v.
    Empty subsets give m = -inf, l = 0, acc = 0."""
    q = np.asarray(q, dtype=np.float64)
    h, d = q.shape[0], V.shape[1]
    if K.shape[0] == 0:
        return np.full(h, -np.inf), np.zeros(h), np.zeros((h, d))
    logits = (q @ K.T) * np.float64(sm_scale)
    m = logits.max(axis=1)
    p = np.exp(logits - m[:, None])
    return m, p.sum(axis=1), p @ V


def merge_partials(parts) -> np.ndarray:
    """Online-softmax (log-sum-exp) merge of partials from disjoint token sets."""
    ms = np.stack([p[0] for p in parts])
    M = ms.max(axis=0)
    Msafe = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(ms), np.exp(ms - Msafe), 0.0)
    L = sum(wi * p[1] for wi, p in zip(w, parts))
    A = sum(wi[:, None] * p[2] for wi, p in zip(w, parts))
    with np.errstate(invalid="ignore", divide="ignore"):
        out = A / L[:, None]
    return np.where(L[:, None] > 0, out, 0.0)


def dequant_history(kind: str, codes_pool, sz_pool, table_row, hist_len: int, g: int, d: int,
                    n_pages: int | None = None, codebook: str = UNIFORM) -> np.ndarray:
    """Dequantised, still-rotated history vectors x_hat = zero + level(code) *
    scale (float64 [hist_len, d]) of KV head g, in history order; level(c) = c
    for the uniform codebook, LM_LEVELS[c] for the Lloyd-Max one; scale and
    zero are those of the channel's group (one group per head unless the
    scale/zero pool holds more).  History
    token t is in page table_row[t // 64] at offset t % 64."""
    t = np.arange(hist_len)
    pages = np.asarray(table_row, dtype=np.int64)[t // PAGE]
    n_pages = codes_pool.shape[0] if n_pages is None else n_pages
    if hist_len and (pages.min() < 0 or pages.max() >= n_pages):
        raise ValueError("block table entry outside the page pool")
    codes, s16, z16 = read_history_codes(kind, codes_pool, sz_pool, pages, t % PAGE, g, d)
    ng = sz_pool.shape[2] // PAGE
    z, s = f16_bits_to_f64(z16).reshape(hist_len, ng), f16_bits_to_f64(s16).reshape(hist_len, ng)
    # channel c belongs to group c // (d / ng)
    z, s = np.repeat(z, d // ng, axis=1), np.repeat(s, d // ng, axis=1)
    return z + code_levels(codebook)[codes] * s


def decode_attn_ref(cfg: dict, k_codes, v_codes, k_sz, v_sz, block_table=None, hist_len=None,
                    sink_len=None, recent_len=None, heads=None) -> np.ndarray:
    """Reference decode attention for every request and query head.

    cfg holds: q bf16 [B][Hq][d]; sink_k/sink_v bf16 [B][n_kv][sink_cap][d];
    recent_k/recent_v bf16 [B][n_kv][recent_cap][d]; sink_len, recent_len,
    hist_len int32 [B]; block_table int32 [B][max_pages]; r_k, r_v fp32
    [n_kv][d][d]; sm_scale; optionally codebook ("uniform" by default or
    "lloyd_max").  Optional overrides replace the cfg entries.
    ``heads`` restricts the work to a list of (b, h) pairs (others are NaN).

    Returns float32 [B][Hq][d]."""
    q = np.asarray(cfg["q"])
    B, Hq, d = q.shape
    n_kv = cfg["r_k"].shape[0]
    if Hq % n_kv:
        raise ValueError("n_q_heads must be a multiple of n_kv")
    G = Hq // n_kv
    table = cfg["block_table"] if block_table is None else block_table
    hl = cfg["hist_len"] if hist_len is None else hist_len
    sl = cfg["sink_len"] if sink_len is None else sink_len
    rl = cfg["recent_len"] if recent_len is None else recent_len
    sink_cap, recent_cap = cfg["sink_k"].shape[2], cfg["recent_k"].shape[2]
    sm = np.float64(np.float32(cfg["sm_scale"]))
    want = None if heads is None else {(int(b), int(h)) for b, h in heads}
    out = np.full((B, Hq, d), np.nan if want is not None else 0.0, dtype=np.float64)
    for b in range(B):
        if not (0 <= sl[b] <= sink_cap and 0 <= rl[b] <= recent_cap and 0 <= hl[b] <= table.shape[1] * PAGE):
            raise ValueError("segment length out of range")
        for g in range(n_kv):
            hs = [h for h in range(g * G, (g + 1) * G) if want is None or (b, h) in want]
            if not hs:
                continue
            Rk = np.asarray(cfg["r_k"][g], dtype=np.float32).astype(np.float64)
            Rv = np.asarray(cfg["r_v"][g], dtype=np.float32).astype(np.float64)
            cb = cfg.get("codebook", UNIFORM)
            xk = dequant_history("k", k_codes, k_sz, table[b], int(hl[b]), g, d, codebook=cb)
            xv = dequant_history("v", v_codes, v_sz, table[b], int(hl[b]), g, d, codebook=cb)
            K = np.concatenate([bf16_to_f64(cfg["sink_k"][b, g, : sl[b]]), xk @ Rk.T,
                                bf16_to_f64(cfg["recent_k"][b, g, : rl[b]])])
            V = np.concatenate([bf16_to_f64(cfg["sink_v"][b, g, : sl[b]]), xv @ Rv.T,
                                bf16_to_f64(cfg["recent_v"][b, g, : rl[b]])])
            out[b, hs] = attn_plain(bf16_to_f64(q[b, hs]), K, V, sm)
    return out.astype(np.float32)


def bf16_paged_attn_ref(q_bits, k_pages, v_pages, block_table, ctx_len, sm_scale,
                        heads=None) -> np.ndarray:
    """Plain decode attention over a context held entirely in BF16 pages
    (k_pages/v_pages bf16 [n_pages][n_kv][64][d]); the comparator's reference.
    Returns float32 [B][Hq][d]."""
    q_bits = np.asarray(q_bits)
    B, Hq, d = q_bits.shape
    n_kv = k_pages.shape[1]
    G = Hq // n_kv
    want = None if heads is None else {(int(b), int(h)) for b, h in heads}
    out = np.full((B, Hq, d), np.nan if want is not None else 0.0)
    sm = np.float64(np.float32(sm_scale))
    for b in range(B):
        t = np.arange(int(ctx_len[b]))
        pages = np.asarray(block_table[b], dtype=np.int64)[t // PAGE]
        for g in range(n_kv):
            hs = [h for h in range(g * G, (g + 1) * G) if want is None or (b, h) in want]
            if not hs:
                continue
            K = bf16_to_f64(k_pages[pages, g, t % PAGE])
            V = bf16_to_f64(v_pages[pages, g, t % PAGE])
            out[b, hs] = attn_plain(bf16_to_f64(q_bits[b, hs]), K, V, sm)
    return out.astype(np.float32)

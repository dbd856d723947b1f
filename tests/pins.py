"""Checks that pin the oracle to facts other than itself.

Each ``check_*`` function raises AssertionError on failure.  The oracle tests
call them on the real oracle; ``test_oracle_mutants.py`` calls them on oracle
copies with planted mistakes and expects a failure.  Nothing here imports the
HIP library.

What each check compares against:
* exact rational arithmetic (fractions.Fraction) and brute-force argmin over
  the four INT2 levels;
* hand-derived closed-form cases, written as literals;
* CPython's struct half-precision packing (round half to even) for fp16;
* torch.nn.functional.scaled_dot_product_attention in float64 on the CPU;
* algebraic invariants (orthogonal rotation, permutation invariance, LSE
  merge, q = 0 gives the mean of the values, a dominant key selects its value).
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np
import torch

import oracle
import synth

PAGE = 64


# --------------------------------------------------------------------------
# exact helpers
# --------------------------------------------------------------------------
def f32_round(fr: Fraction) -> float:
    """Correctly rounded (nearest, ties to even) float32 of a rational."""
    a = np.float32(float(fr))
    cands = [np.nextafter(a, np.float32(-np.inf)), a, np.nextafter(a, np.float32(np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        err = abs(Fraction(float(c)) - fr)
        key = (err, int(np.float32(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return float(best[1])


def f16_round(x: float) -> float:
    """fp16 round-to-nearest-even via CPython's struct packing."""
    return struct.unpack("<e", struct.pack("<e", x))[0]


def exact_rotate(x_bits: np.ndarray, rot: np.ndarray) -> np.ndarray:
    """y_j = sum_i x_i R[i, j] in exact rationals, rounded once to float32."""
    x = [Fraction(float(v)) for v in synth.bf16_bits_to_f32(x_bits)]
    d = len(x)
    out = np.empty(d, dtype=np.float32)
    for j in range(d):
        out[j] = f32_round(sum(x[i] * Fraction(float(rot[i, j])) for i in range(d)))
    return out


def random_orthogonal(d: int, rng) -> np.ndarray:
    q, r = np.linalg.qr(rng.standard_normal((d, d)))
    return (q * np.sign(np.diag(r))).astype(np.float32)


def signed_permutation(d: int, rng):
    perm = rng.permutation(d)
    while d > 2 and np.array_equal(perm[perm], np.arange(d)):   # want a non-involution
        perm = rng.permutation(d)
    sign = rng.choice([-1.0, 1.0], size=d)
    r = np.zeros((d, d), dtype=np.float32)
    r[np.arange(d), perm] = sign
    return r, perm, sign


# --------------------------------------------------------------------------
# quantiser pins
# --------------------------------------------------------------------------
def check_quant_closed_forms():
    """Hand-derived cases with R = I (values chosen exactly representable)."""
    def q(vals, tau):
        codes, s16, z16, _ = oracle.quantize_group(np.array([vals], np.float32), tau)
        return (codes[0].tolist(), float(np.array(s16).view(np.float16)[0]),
                float(np.array(z16).view(np.float16)[0]))
    # four evenly spaced levels reconstruct exactly: zero=-1.5, scale=1
    assert q([-1.5, -0.5, 0.5, 1.5], 8.0) == ([0, 1, 2, 3], 1.0, -1.5)
    # clipping to +-6: range 12, scale 4, zero -6; 0 sits at 1.5 steps -> ties to even -> 2
    assert q([-100.0, 0.0, 0.0, 100.0], 6.0) == ([0, 2, 2, 3], 4.0, -6.0)
    # half-way points round to even codes: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2
    assert q([0.0, 0.5, 1.5, 2.5, 3.0, 1.0, 2.0, 0.25], 8.0) == ([0, 0, 2, 2, 3, 1, 2, 0], 1.0, 0.0)
    # degenerate group: scale 0, all codes 0
    assert q([0.75, 0.75, 0.75, 0.75], 8.0) == ([0, 0, 0, 0], 0.0, 0.75)
    # asymmetric range: zero = fp16(min) = -1; fp32(5/3) = 1.6666666 lies nearer the
    # fp16 value 1707/1024 = 1.6669921875 than 1706/1024
    c, s, z = q([-1.0, 4.0, 0.0, 2.0], 8.0)
    assert (s, z) == (1.6669921875, -1.0) and c == [0, 3, 1, 2]


def check_quant_bruteforce(d: int = 16, n: int = 24, seed: int = 3):
    """Rotation, clip, min/max, fp16 rounding and code choice against exact
    arithmetic and an argmin over the four levels."""
    rng = np.random.default_rng(seed)
    rot = random_orthogonal(d, rng)
    x = synth.f32_to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32) * 3)
    x[0, 2] = synth.f32_to_bf16_bits(np.float32([60.0]))[0]          # a clipped outlier
    tau = np.float32(5.0)
    y = oracle.rotate_round_f32(x, rot)
    codes, s16, z16, info = oracle.quantize_group(y, tau)
    for r in range(n):
        ye = exact_rotate(x[r], rot)
        assert np.array_equal(ye, y[r]), "rotation y = x R (rounded once) mismatch"
        yc = [min(max(float(v), -5.0), 5.0) for v in ye]
        mn, mx = min(yc), max(yc)
        z = f16_round(mn)
        s = f16_round(f32_round(Fraction(f32_round(Fraction(mx) - Fraction(mn))) / 3))
        assert float(np.array(z16[r]).view(np.float16)) == z, "zero point"
        assert float(np.array(s16[r]).view(np.float16)) == s, "scale"
        for j in range(d):
            if s == 0:
                assert codes[r, j] == 0
                continue
            dist = [abs(Fraction(yc[j]) - (Fraction(z) + c * Fraction(s))) for c in range(4)]
            best = min(dist)
            winners = [c for c in range(4) if dist[c] == best]
            want = winners[0] if len(winners) == 1 else [c for c in winners if c % 2 == 0][0]
            if codes[r, j] != want:
                t = (Fraction(yc[j]) - Fraction(z)) / Fraction(s)
                edge = Fraction(min(codes[r, j], want)) + Fraction(1, 2)
                assert abs(t - edge) <= Fraction(1, 1 << 20) * max(1, abs(t)), \
                    f"code {codes[r, j]} vs argmin {want} away from a bin edge"
        # the extremes land on the end codes
        assert codes[r, int(np.argmin(yc))] == 0 and (s == 0 or codes[r, int(np.argmax(yc))] == 3)


def check_pack_literals():
    """Channel 4i+j sits in bits 2j of byte i (hand-computed bytes)."""
    row = oracle.pack_codes_row(np.array([1, 2, 3, 0, 3, 3, 3, 3], np.uint8))
    assert row.tolist() == [1 | 2 << 2 | 3 << 4, 255]
    assert row.tolist() == [57, 255]
    rng = np.random.default_rng(4)
    c = rng.integers(0, 4, size=(5, 64)).astype(np.uint8)
    assert np.array_equal(oracle.unpack_codes_row(oracle.pack_codes_row(c)), c)


def check_layout_literals():
    """In-page positions, written out by hand for d = 64 and d = 128."""
    # K, d=64: 4 planes of 4 bytes per token; plane p at p*256
    assert oracle.k_byte_offsets(0, 64).tolist() == [0, 1, 2, 3, 256, 257, 258, 259,
                                                     512, 513, 514, 515, 768, 769, 770, 771]
    assert oracle.k_byte_offsets(5, 64)[[0, 4, 15]].tolist() == [20, 276, 791]
    # K, d=128: 4 planes of 8 bytes per token; plane p at p*512
    assert oracle.k_byte_offsets(63, 128)[[0, 7, 8, 31]].tolist() == [504, 511, 1016, 2047]
    # V: byte-column-major, byte i of token o at i*64 + o
    assert oracle.v_byte_offsets(0, 128)[[0, 1, 31]].tolist() == [0, 64, 1984]
    assert oracle.v_byte_offsets(63, 64)[[0, 15]].tolist() == [63, 1023]
    for d in (64, 128):
        for fn in (oracle.k_byte_offsets, oracle.v_byte_offsets):
            allpos = np.concatenate([fn(o, d) for o in range(PAGE)])
            assert np.array_equal(np.sort(allpos), np.arange(PAGE * d // 4))


def check_column_permutation_invariance(seed: int = 5):
    """Permuting the columns of R permutes the codes and keeps scale/zero."""
    rng = np.random.default_rng(seed)
    d = 32
    rot = random_orthogonal(d, rng)
    perm = rng.permutation(d)
    x = synth.f32_to_bf16_bits(rng.standard_normal((40, d)).astype(np.float32))
    c1, s1, z1, _ = oracle.quantize_group(oracle.rotate_round_f32(x, rot), 2.5)
    c2, s2, z2, _ = oracle.quantize_group(oracle.rotate_round_f32(x, rot[:, perm]), 2.5)
    assert np.array_equal(s1, s2) and np.array_equal(z1, z2)
    assert np.array_equal(c1[:, perm], c2)


def check_grouped_quantize_pack(seed: int = 14):
    """32-channel groups: each group of a token is the whole-row quantiser
    applied to its 32 channels, and its (scale, zero) lands at group j,
    offset o of the group-planar pool: pair j*64 + o (hand layout)."""
    rng = np.random.default_rng(seed)
    d, nkv, n_pages, grp = 128, 2, 2, 32
    rot = np.stack([random_orthogonal(d, rng) for _ in range(nkv)])
    x = synth.f32_to_bf16_bits(rng.standard_normal((5, nkv, d)).astype(np.float32) * np.linspace(0.3, 3, d))
    kc = np.zeros((n_pages, nkv, PAGE * d // 4), np.uint8)
    ks = np.zeros((n_pages, nkv, PAGE * d // grp, 2), np.uint16)
    slots = np.array([70, 3, 127, 64, 9], np.int32)
    oracle.quantize_pack_ref("v", x, rot, 2.0, slots, kc, ks, group=grp)
    for r, s in enumerate(slots):
        p, o = divmod(int(s), PAGE)
        for g in range(nkv):
            y = oracle.rotate_round_f32(x[r, g][None], rot[g])[0]
            for j in range(d // grp):
                c, sc, ze, _ = oracle.quantize_group(np.ascontiguousarray(y[None, grp * j:grp * (j + 1)]), 2.0)
                assert ks[p, g, j * PAGE + o, 0] == sc[0] and ks[p, g, j * PAGE + o, 1] == ze[0]
                row = oracle.pack_codes_row(c[0])
                for i in range(grp // 4):   # V byte of channels 4(8j+i).. at (8j+i)*64 + o
                    assert kc[p, g, (grp // 4 * j + i) * PAGE + o] == row[i]


def check_quantize_pack_slots(seed: int = 6):
    """Scatter into (page, offset) = divmod(slot, 64); skip slots and source
    rows outside the pools; bytes land where the layout literals say."""
    rng = np.random.default_rng(seed)
    d, nkv, n_pages = 64, 2, 3
    rot = np.stack([np.eye(d, dtype=np.float32)] * nkv)
    x = synth.f32_to_bf16_bits(rng.standard_normal((6, nkv, d)).astype(np.float32))
    kc = np.zeros((n_pages, nkv, PAGE * d // 4), np.uint8)
    ks = np.zeros((n_pages, nkv, PAGE, 2), np.uint16)
    vc, vs = kc.copy(), ks.copy()
    slots = np.array([130, -1, 5, 192, 64, 7], np.int32)          # 192 = 3*64 is out of range
    src = np.array([0, 1, 2, 3, 9, 5], np.int32)                  # 9 is out of range
    oracle.quantize_pack_ref("k", x, rot, 9.0, slots, kc, ks, src_idx=src)
    oracle.quantize_pack_ref("v", x, rot, 9.0, slots, vc, vs, src_idx=src)
    for s, r in ((130, 0), (5, 2), (7, 5)):
        p, o = divmod(s, PAGE)
        for g in range(nkv):
            codes, sc, ze, _ = oracle.quantize_group(oracle.rotate_round_f32(x[r, g][None], rot[g]), 9.0)
            row = oracle.pack_codes_row(codes[0])
            # hand layout: K plane i//4 at (i//4)*256 + o*4 + i%4 ; V at i*64 + o
            for i in range(d // 4):
                assert kc[p, g, (i // 4) * 256 + o * 4 + i % 4] == row[i]
                assert vc[p, g, i * 64 + o] == row[i]
            assert ks[p, g, o, 0] == sc[0] and ks[p, g, o, 1] == ze[0]
    written = {(130 // 64, 130 % 64), (0, 5), (0, 7)}
    for p in range(n_pages):
        for o in range(PAGE):
            if (p, o) not in written:
                assert not ks[p, :, o].any()


# --------------------------------------------------------------------------
# decode pins
# --------------------------------------------------------------------------
def _write_pages_bruteforce(codes, scale, zero, slots, n_pages, d, nkv):
    """Place codes [n][nkv][d] into K and V pools bit by bit (pure loops).
    scale / zero are [n][nkv] (one group per head) or [n][nkv][ng] (group j
    of token o stored at j*64 + o)."""
    ng = 1 if scale[0].ndim == 2 else scale[0].shape[2]
    kc = np.zeros((n_pages, nkv, PAGE * d // 4), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.zeros((n_pages, nkv, PAGE * ng, 2), np.uint16)
    vs = np.zeros_like(ks)
    w = d // 16
    for t, slot in enumerate(slots):
        p, o = divmod(int(slot), PAGE)
        for g in range(nkv):
            for c in range(d):
                i, j = divmod(c, 4)
                kc[p, g, (i // w) * PAGE * w + o * w + i % w] |= np.uint8(int(codes[0][t, g, c]) << (2 * j))
                vc[p, g, i * PAGE + o] |= np.uint8(int(codes[1][t, g, c]) << (2 * j))
            for j in range(ng):
                pick = (lambda a: a[t, g]) if ng == 1 else (lambda a: a[t, g, j])
                ks[p, g, j * PAGE + o] = (pick(scale[0]), pick(zero[0]))
                vs[p, g, j * PAGE + o] = (pick(scale[1]), pick(zero[1]))
    return kc, vc, ks, vs


# Dequantised level of each 2-bit code, per codebook (the Lloyd-Max levels are
# +-0.4528 and +-1.5104 deviations of a Gaussian in the ratio 3 : 10)
CODE_LEVELS = {"uniform": (0.0, 1.0, 2.0, 3.0), "lloyd_max": (-10.0, -3.0, 3.0, 10.0)}


def make_small_cache(seed=7, B=2, Hq=6, nkv=3, d=32, sink=(5, 0), hist=(70, 9), recent=(3, 11),
                     sink_cap=6, recent_cap=12, rot="orth", codebook="uniform", groups=1):
    """A small three-segment cache with directly drawn codes and fp16
    scale/zero (no quantisation step).  Returns (cfg, pools, truth) where truth
    holds the materialised float64 K/V of every (b, g) in context order."""
    rng = np.random.default_rng(seed)
    max_pages = max(-(-h // PAGE) for h in hist) or 1
    n_hist = sum(hist)
    n_pages = sum(-(-h // PAGE) for h in hist) + 2
    perm = rng.permutation(n_pages)
    table = np.full((B, max_pages), -1, np.int32)
    k = 0
    slots = []
    for b in range(B):
        np_b = -(-hist[b] // PAGE)
        table[b, :np_b] = perm[k:k + np_b]
        k += np_b
        t = np.arange(hist[b])
        slots.append(table[b, t // PAGE] * PAGE + t % PAGE)
    slots = np.concatenate(slots)
    ck = rng.integers(0, 4, size=(n_hist, nkv, d)).astype(np.uint8)
    cv = rng.integers(0, 4, size=(n_hist, nkv, d)).astype(np.uint8)
    gshape = (n_hist, nkv) if groups == 1 else (n_hist, nkv, groups)   # one (scale, zero) per group
    sk = rng.uniform(0.2, 2.0, size=gshape).astype(np.float16)
    zk = rng.uniform(-3.0, -0.5, size=gshape).astype(np.float16)
    sv = rng.uniform(0.2, 2.0, size=gshape).astype(np.float16)
    zv = rng.uniform(-3.0, -0.5, size=gshape).astype(np.float16)
    kc, vc, ks, vs = _write_pages_bruteforce((ck, cv), (sk.view(np.uint16), sv.view(np.uint16)),
                                             (zk.view(np.uint16), zv.view(np.uint16)), slots, n_pages, d, nkv)
    if rot == "orth":
        rk = np.stack([random_orthogonal(d, rng) for _ in range(nkv)])
        rv = np.stack([random_orthogonal(d, rng) for _ in range(nkv)])
    elif rot == "signed_perm":
        rk = np.stack([signed_permutation(d, rng)[0] for _ in range(nkv)])
        rv = np.stack([signed_permutation(d, rng)[0] for _ in range(nkv)])
    else:
        rk = np.stack([np.eye(d, dtype=np.float32)] * nkv)
        rv = rk.copy()
    bf = lambda shape, s=1.0: synth.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * s)
    cfg = dict(q=bf((B, Hq, d)), sink_k=bf((B, nkv, sink_cap, d)), sink_v=bf((B, nkv, sink_cap, d), 2.0),
               recent_k=bf((B, nkv, recent_cap, d)), recent_v=bf((B, nkv, recent_cap, d), 2.0),
               sink_len=np.array(sink, np.int32), recent_len=np.array(recent, np.int32),
               hist_len=np.array(hist, np.int32), block_table=table, r_k=rk, r_v=rv,
               sm_scale=np.float32(1 / np.sqrt(d)))
    if codebook != "uniform":
        cfg["codebook"] = codebook
    lv = np.array(CODE_LEVELS[codebook])
    # truth: dequantised rotated history, inverse-rotated with R^T (row vectors)
    truth = {}
    off = 0
    for b in range(B):
        sl = slice(off, off + hist[b])
        off += hist[b]
        for g in range(nkv):
            # the (scale, zero) of each channel: its group's, channel c in group c // (d / groups)
            per_ch = lambda a: np.repeat(a[sl, g].astype(np.float64).reshape(hist[b], groups), d // groups, axis=1)
            xk = per_ch(zk) + lv[ck[sl, g]] * per_ch(sk)
            xv = per_ch(zv) + lv[cv[sl, g]] * per_ch(sv)
            K = np.concatenate([synth.bf16_bits_to_f32(cfg["sink_k"][b, g, :sink[b]]).astype(np.float64),
                                xk @ rk[g].astype(np.float64).T,
                                synth.bf16_bits_to_f32(cfg["recent_k"][b, g, :recent[b]]).astype(np.float64)])
            V = np.concatenate([synth.bf16_bits_to_f32(cfg["sink_v"][b, g, :sink[b]]).astype(np.float64),
                                xv @ rv[g].astype(np.float64).T,
                                synth.bf16_bits_to_f32(cfg["recent_v"][b, g, :recent[b]]).astype(np.float64)])
            truth[(b, g)] = (K, V, xk, xv)
    return cfg, (kc, vc, ks, vs), truth


def sdpa_reference(cfg, truth):
    """torch SDPA (float64, CPU, GQA) over the materialised cache."""
    q = synth.bf16_bits_to_f32(cfg["q"]).astype(np.float64)
    B, Hq, d = q.shape
    nkv = cfg["r_k"].shape[0]
    out = np.zeros((B, Hq, d))
    for b in range(B):
        n = truth[(b, 0)][0].shape[0]
        if n == 0:
            continue
        K = torch.from_numpy(np.stack([truth[(b, g)][0] for g in range(nkv)]))[None]
        V = torch.from_numpy(np.stack([truth[(b, g)][1] for g in range(nkv)]))[None]
        qq = torch.from_numpy(q[b])[None, :, None, :]
        o = torch.nn.functional.scaled_dot_product_attention(qq, K, V, scale=float(cfg["sm_scale"]),
                                                             enable_gqa=True)
        out[b] = o[0, :, 0, :].numpy()
    return out


def check_decode_vs_sdpa(seed=7, rot="orth"):
    cfg, pools, truth = make_small_cache(seed=seed, rot=rot)
    out = oracle.decode_attn_ref(cfg, *pools)
    ref = sdpa_reference(cfg, truth)
    assert np.abs(out - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max()), np.abs(out - ref).max()


def check_decode_vs_sdpa_grouped(seed=9):
    """Two (scale, zero) groups per head: the dequantisation must take each
    channel's own group."""
    cfg, pools, truth = make_small_cache(seed=seed, groups=2)
    out = oracle.decode_attn_ref(cfg, *pools)
    ref = sdpa_reference(cfg, truth)
    assert np.abs(out - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max()), np.abs(out - ref).max()


def check_inverse_rotation_direction(seed=8):
    """With R a non-involutive signed permutation, x_hat R^T is an index
    operation: (x_hat R^T)[i] = sign[i] * x_hat[perm[i]]."""
    rng = np.random.default_rng(seed)
    d = 32
    r, perm, sign = signed_permutation(d, rng)
    cfg, pools, _ = make_small_cache(seed=seed, B=1, Hq=2, nkv=1, d=d, sink=(0,), hist=(40,), recent=(0,),
                                     rot="identity")
    cfg["r_k"] = r[None].copy()
    cfg["r_v"] = r[None].copy()
    xk = oracle.dequant_history("k", pools[0], pools[2], cfg["block_table"][0], 40, 0, d)
    xv = oracle.dequant_history("v", pools[1], pools[3], cfg["block_table"][0], 40, 0, d)
    K = sign[None, :] * xk[:, perm]
    V = sign[None, :] * xv[:, perm]
    q = synth.bf16_bits_to_f32(cfg["q"][0]).astype(np.float64)
    lg = q @ K.T * float(cfg["sm_scale"])
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    ref = p @ V / p.sum(axis=1, keepdims=True)
    out = oracle.decode_attn_ref(cfg, *pools)[0]
    assert np.abs(out - ref).max() <= 1e-5 * np.abs(ref).max()


def check_rotated_space_identity(seed=9):
    """Scores (q R) . x_hat and (A R^T) equal the unrotated attention: the
    rotate-the-query-once form the kernel uses gives the same output."""
    cfg, pools, truth = make_small_cache(seed=seed, B=1, Hq=4, nkv=2, d=32, sink=(4,), hist=(100,), recent=(7,))
    out = oracle.decode_attn_ref(cfg, *pools)[0]
    q = synth.bf16_bits_to_f32(cfg["q"][0]).astype(np.float64)
    sm = float(cfg["sm_scale"])
    for h in range(4):
        g = h // 2
        K, V, xk, xv = truth[(0, g)]
        rk, rv = cfg["r_k"][g].astype(np.float64), cfg["r_v"][g].astype(np.float64)
        n_s = 4
        qr = q[h] @ rk
        lg = np.concatenate([K[:n_s] @ q[h], xk @ qr, K[n_s + 100:] @ q[h]]) * sm
        p = np.exp(lg - lg.max())
        acc_rot = p[n_s:n_s + 100] @ xv
        o = (p[:n_s] @ V[:n_s] + acc_rot @ rv.T + p[n_s + 100:] @ V[n_s + 100:]) / p.sum()
        assert np.abs(o - out[h]).max() <= 1e-5 * np.abs(o).max()


def check_decode_special_cases(seed=10):
    # q = 0: uniform weights, output = mean of every value in the context
    cfg, pools, truth = make_small_cache(seed=seed)
    cfg["q"] = np.zeros_like(cfg["q"])
    out = oracle.decode_attn_ref(cfg, *pools)
    for b in range(2):
        for h in range(6):
            V = truth[(b, h // 2)][1]
            assert np.abs(out[b, h] - V.mean(axis=0)).max() <= 1e-5 * np.abs(V).max()
    # a dominant recent key selects its own value
    cfg, pools, truth = make_small_cache(seed=seed + 1)
    qv = synth.bf16_bits_to_f32(cfg["q"][0, 0]).astype(np.float32)
    cfg["recent_k"][0, 0, 2] = synth.f32_to_bf16_bits(qv * 8)
    out = oracle.decode_attn_ref(cfg, *pools)
    want = synth.bf16_bits_to_f32(cfg["recent_v"][0, 0, 2]).astype(np.float64)
    assert np.abs(out[0, 0] - want).max() <= 1e-4 * np.abs(want).max()
    # no history: plain attention over the BF16 windows
    cfg, pools, truth = make_small_cache(seed=seed + 2, hist=(0, 0))
    out = oracle.decode_attn_ref(cfg, *pools)
    ref = sdpa_reference(cfg, truth)
    assert np.abs(out - ref).max() <= 1e-5 * np.abs(ref).max()
    # empty context: zero rows
    cfg, pools, truth = make_small_cache(seed=seed + 3, sink=(0, 2), hist=(0, 5), recent=(0, 1))
    out = oracle.decode_attn_ref(cfg, *pools)
    assert not out[0].any() and np.abs(out[1]).max() > 0


def check_decode_invariances(seed=11):
    cfg, pools, truth = make_small_cache(seed=seed, hist=(150, 64))
    base = oracle.decode_attn_ref(cfg, *pools)
    # physical page order: move every page and remap the table
    kc, vc, ks, vs = pools
    n_pages = kc.shape[0]
    perm = np.random.default_rng(seed).permutation(n_pages)    # new id of old page p = perm[p]
    inv = np.argsort(perm)
    t2 = cfg["block_table"].copy()
    t2[t2 >= 0] = perm[t2[t2 >= 0]]
    out = oracle.decode_attn_ref(cfg, kc[inv], vc[inv], ks[inv], vs[inv], block_table=t2)
    assert np.abs(out - base).max() <= 1e-6 * np.abs(base).max()
    # recent-window ring order
    cfg2 = dict(cfg)
    rp = np.random.default_rng(seed + 1).permutation(cfg["recent_len"][1])
    rk, rv = cfg["recent_k"].copy(), cfg["recent_v"].copy()
    rk[1, :, : len(rp)] = rk[1][:, rp]
    rv[1, :, : len(rp)] = rv[1][:, rp]
    cfg2["recent_k"], cfg2["recent_v"] = rk, rv
    out = oracle.decode_attn_ref(cfg2, *pools)
    assert np.abs(out - base).max() <= 1e-6 * np.abs(base).max()


def check_partition_merge(seed=12):
    """LSE-merging partials of any split of the tokens reproduces attention."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((3, 16))
    K = rng.standard_normal((97, 16)) * 2
    V = rng.standard_normal((97, 16))
    ref = oracle.attn_plain(q, K, V, 0.25)
    cuts = [0, 1, 1, 40, 41, 97]
    parts = [oracle.attn_partial(q, K[a:b], V[a:b], 0.25) for a, b in zip(cuts[:-1], cuts[1:])]
    assert np.abs(oracle.merge_partials(parts) - ref).max() <= 1e-12
    # against a library softmax too
    lg = torch.from_numpy(q @ K.T * 0.25)
    assert np.abs((torch.softmax(lg, dim=1).numpy() @ V) - ref).max() <= 1e-12


def check_bf16_paged_vs_sdpa(seed=13):
    rng = np.random.default_rng(seed)
    B, Hq, nkv, d = 2, 4, 2, 32
    ctx = np.array([130, 7], np.int32)
    n_pages = 5
    table = np.array([[3, 0, 4], [1, -1, -1]], np.int32)
    kp = synth.f32_to_bf16_bits(rng.standard_normal((n_pages, nkv, PAGE, d)).astype(np.float32))
    vp = synth.f32_to_bf16_bits(rng.standard_normal((n_pages, nkv, PAGE, d)).astype(np.float32))
    q = synth.f32_to_bf16_bits(rng.standard_normal((B, Hq, d)).astype(np.float32))
    out = oracle.bf16_paged_attn_ref(q, kp, vp, table, ctx, 0.2)
    for b in range(B):
        K = np.concatenate([kp[table[b, i]] for i in range(-(-ctx[b] // PAGE))], axis=1)[:, : ctx[b]]
        V = np.concatenate([vp[table[b, i]] for i in range(-(-ctx[b] // PAGE))], axis=1)[:, : ctx[b]]
        Kt = torch.from_numpy(synth.bf16_bits_to_f32(K).astype(np.float64))[None]
        Vt = torch.from_numpy(synth.bf16_bits_to_f32(V).astype(np.float64))[None]
        qq = torch.from_numpy(synth.bf16_bits_to_f32(q[b]).astype(np.float64))[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, Kt, Vt, scale=0.2, enable_gqa=True)[0, :, 0]
        assert np.abs(out[b] - ref.numpy()).max() <= 1e-5 * np.abs(ref.numpy()).max()

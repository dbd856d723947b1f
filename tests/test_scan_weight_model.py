"""CPU model of the INT2 history scan's softmax-weight arithmetic.

The scan accumulates, per head, sum_t p_t * (zero_t + scale_t * level(c_t))
over a wave's pages, with p_t = 2^(logit_t - m_ref) kept relative to a lazily
raised reference.  This file re-enacts that arithmetic on the CPU, token by
token, in the same floating-point precisions as the kernel, and compares the
normalised result with the exact fp64 value.  It is a model of the kernel
(its rounding steps), not of the method: the method's reference is the
oracle's exact attention.

Two weight representations are modelled:

* ``fixed30``: the earlier design.  p * scale becomes a 30-bit fixed-point
  integer with unit 2^-18 of the reference weight (2^12 of head-room for the
  lazy rescale), so a token lighter than 2^-19 of the reference rounds to
  zero in the value sum while its exact p still enters the weight sum: a
  one-sided bias that grows with the number of such tokens.
* ``f16x2``: the current design.  p * scale * kappa (kappa puts the largest
  possible weight at 2^14) is split into an fp16 high part and an fp16 low
  part that carries the remainder scaled by 2^11 (both rounded toward zero,
  as v_cvt_pkrtz_f16_f32 does); the products with the codes are summed in
  fp32.  A weight is then held to 2^-21 of itself, and the absolute floor is
  2^-35 of kappa's unit, far below any weight that matters.

The inputs are the long-context retrieval pattern: one dominant history token
and hundreds to thousands of background tokens 2^-17 .. 2^-30 lighter, with V
scales of 4..6, on waves of 7 pages (the 100k batch-1 split) and 56 pages
(the 28-request split).
"""
import numpy as np
import pytest

PAGE = 64
LAZY = 12.0          # lazy rescale threshold (log2 units)
SLACK = 1.75         # a V scale may exceed the running maximum by this factor before a rescale
MAX_ABS, REL_L2 = 2e-3, 1e-3


def rtz_f16(x):
    """float32 -> float16 rounded toward zero (v_cvt_pkrtz_f16_f32)."""
    x = np.asarray(x, np.float32)
    h = x.astype(np.float16)
    over = np.abs(h.astype(np.float32)) > np.abs(x)
    h[over] = np.nextafter(h[over], np.float16(0))
    return h


def lm_level(c):
    return np.array([-10.0, -3.0, 3.0, 10.0])[c]


def scan_wave(logit2, scale, zero, codes, scheme, codebook="uniform"):
    """One head's scan of a wave: logit2 [n] (log2 units), scale/zero [n]
    (fp16-valued), codes [n][d].  Returns the normalised fp64 output [d]
    (rotated space) as the kernel's arithmetic produces it.

    Summation structure as in the kernel: lane n of a head's 16 lanes holds
    tokens 4n..4n+3 of every page in its own fp32 weight and zero-point sums,
    added once at the end; the value sums take one fp32 rounding per 32-token
    half page (one matrix instruction's accumulate)."""
    n, d = codes.shape
    f32 = np.float32
    mref = f32(0.0)
    thr, smax, sthr, kap = -np.inf, f32(0.0), f32(0.0), f32(0.0)
    lsum = np.zeros(16, f32)
    zsum = np.zeros(16, f32)
    acc = np.zeros(d, np.float64)            # fixed30: exact integer sums; f16x2: fp32 sums
    facc = np.zeros(d, np.float32)           # fixed30: folded fp32 part
    if codebook == "uniform":
        level, zoff = codes.astype(np.float64), 0.0
    elif scheme == "fixed30":            # int8 operands held the levels themselves
        level, zoff = lm_level(codes), 0.0
    else:                                # 7c - (c >> 1) on the matrix cores, -10 with the zero point
        level, zoff = (7 * codes - (codes >> 1)).astype(np.float64), -10.0
    for p0 in range(0, n, PAGE):
        sl = slice(p0, min(n, p0 + PAGE))
        lg = (logit2[sl].astype(f32) - mref).astype(f32)
        sv = scale[sl].astype(f32)
        lmax = lg.max()
        if lmax > thr or sv.max() > sthr:
            first = not kap > 0
            s_new = max(smax, sv.max())
            delta = f32(lmax) if first else f32(max(lmax, 0.0))
            alpha = f32(2.0 ** -float(delta))
            if scheme == "fixed30":
                kw_old = kap
                if not first:
                    facc = ((facc + (acc / kw_old).astype(f32)) * alpha).astype(f32)
                    acc[:] = 0
                kap = f32(2.0 ** 30 / (2.0 ** LAZY * (s_new if s_new > 0 else 1.0)))
            else:
                kap_new = f32(2.0 ** 14 / (2.0 ** LAZY * SLACK * (s_new if s_new > 0 else 1.0)))
                if not first:
                    acc = (acc * np.float64(f32(alpha * (kap_new / kap)))).astype(f32).astype(np.float64)
                kap = kap_new
            if not first:
                lsum = (lsum * alpha).astype(f32)
                zsum = (zsum * alpha).astype(f32)
            mref = f32(mref + delta)
            lg = (lg - delta).astype(f32)
            thr, smax, sthr = LAZY, f32(s_new), f32(SLACK * s_new)
        pr = np.exp2(lg.astype(np.float64)).astype(f32)
        zz = (zero[sl] + zoff * scale[sl]).astype(f32)
        for t in range(len(pr)):
            ln = (t % PAGE) // 4
            lsum[ln] = f32(lsum[ln] + pr[t])
            zsum[ln] = f32(np.float64(pr[t]) * np.float64(zz[t]) + np.float64(zsum[ln]))
        if scheme == "fixed30":
            svk = (sv * kap).astype(f32)
            w = np.floor((pr.astype(np.float64) * svk + 0.5).astype(f32).astype(np.float64))
            acc += w @ level[sl]
        else:
            w = (pr * (sv * kap).astype(f32)).astype(f32)
            hi = rtz_f16(w)
            lo = rtz_f16((w * f32(2048.0) - hi.astype(f32) * f32(2048.0)).astype(f32))
            wq = hi.astype(np.float64) + lo.astype(np.float64) / 2048.0
            lv = level[sl]
            for h0 in range(0, len(wq), 32):
                acc = (acc + wq[h0:h0 + 32] @ lv[h0:h0 + 32]).astype(f32).astype(np.float64)
    if scheme == "fixed30":
        num = facc.astype(np.float64) + acc / np.float64(kap)
    else:
        num = acc / np.float64(kap)
    return (num + np.float64(zsum.astype(np.float64).sum())) / np.float64(lsum.astype(np.float64).sum())


def exact_wave(logit2, scale, zero, codes, codebook="uniform"):
    level = codes.astype(np.float64) if codebook == "uniform" else lm_level(codes)
    p = np.exp2(logit2 - logit2.max())
    x = zero[:, None].astype(np.float64) + scale[:, None].astype(np.float64) * level
    return (p @ x) / p.sum()


def needle_wave(seed, pages, lo, hi, where="first", d=128, codebook="uniform"):
    """One dominant token and a background lo..hi log2 units below it.  V
    scales are 4..6 for the uniform codebook (range / 3 of clipped rotated
    values) and a tenth of that for Lloyd-Max (0.151 standard deviations)."""
    rng = np.random.default_rng(seed)
    n = pages * PAGE
    logit2 = 3.0 - rng.uniform(lo, hi, size=n)
    pos = {"first": 0, "middle": n // 2 + 17, "last": n - 1}[where]
    logit2[pos] = 3.0
    unit = 1.0 if codebook == "uniform" else 0.1
    scale = (unit * rng.uniform(4.0, 6.0, size=n)).astype(np.float16).astype(np.float64)
    zero = (-1.5 * scale + rng.normal(0, 0.3, size=n)).astype(np.float16).astype(np.float64)
    codes = rng.integers(0, 4, size=(n, d))
    return logit2, scale, zero, codes


def err(got, want):
    e = np.abs(got - want)
    return e.max(), np.linalg.norm(e) / np.linalg.norm(want)


@pytest.mark.parametrize("pages", [7, 56])
def test_fixed_point_weights_fail_the_needle_pattern(pages):
    """The input reaches the earlier design's hole: background tokens
    2^-19..2^-22 below the needle are dropped from the value sum."""
    x = needle_wave(1, pages, 19, 22)
    ma, rl = err(scan_wave(*x, scheme="fixed30"), exact_wave(*x))
    assert ma > MAX_ABS, f"fixed-point model unexpectedly within tolerance ({ma:.2e})"


@pytest.mark.parametrize("codebook", ["uniform", "lloyd_max"])
@pytest.mark.parametrize("where", ["first", "middle", "last"])
@pytest.mark.parametrize("band", [(17, 21), (22, 26), (26, 30), (0, 12)])
@pytest.mark.parametrize("pages", [7, 56])
def test_fp16_pair_weights_meet_the_tolerance(pages, band, where, codebook):
    x = needle_wave(2 + pages, pages, *band, where=where, codebook=codebook)
    ma, rl = err(scan_wave(*x, scheme="f16x2", codebook=codebook), exact_wave(*x, codebook=codebook))
    assert ma <= MAX_ABS / 20 and rl <= REL_L2 / 20, f"max-abs {ma:.2e}, rel-L2 {rl:.2e}"


@pytest.mark.parametrize("pages", [7, 64])
def test_fp16_pair_weights_flat_and_rising_logits(pages):
    """No needle: logits of spread 2^5 (typical), then a steady rise that
    forces a rescale on most pages, with V scales that grow past the slack."""
    rng = np.random.default_rng(40 + pages)
    n = pages * PAGE
    for logit2 in (rng.normal(0, 4.6, size=n), np.linspace(0, 60, n) + rng.normal(0, 1, size=n)):
        scale = np.linspace(0.5, 7.0, n).astype(np.float16).astype(np.float64)
        zero = (-1.5 * scale).astype(np.float16).astype(np.float64)
        codes = rng.integers(0, 4, size=(n, 128))
        ma, rl = err(scan_wave(logit2, scale, zero, codes, scheme="f16x2"), exact_wave(logit2, scale, zero, codes))
        assert ma <= MAX_ABS / 20 and rl <= REL_L2 / 20, f"max-abs {ma:.2e}, rel-L2 {rl:.2e}"


def test_lloyd_max_levels_split_into_code_and_high_bit():
    """The Lloyd-Max level of a code is 7c - 10 - (c >> 1): the scan sums
    p*scale*c and p*scale*(c >> 1) on the matrix cores and moves the -10 into
    the zero-point sum."""
    c = np.arange(4)
    assert np.array_equal(7 * c - 10 - (c >> 1), lm_level(c))

"""Pins of the oracle's Lloyd-Max codebook variant against definitions written
out independently: nearest-level brute force, the group statistics by exact
summation, the mean-squared-error optimality of the 4-level Gaussian
quantiser (closed-form optimum 0.1175), the centroid condition, and decode
attention over a cache materialised with the Lloyd-Max levels."""
import math

import numpy as np
import pytest

import oracle
import pins


def test_codes_are_the_nearest_level():
    rng = np.random.default_rng(1)
    y = (rng.standard_normal((24, 64)) * rng.uniform(0.2, 3.0, size=(24, 1))).astype(np.float32)
    y[:, 5] *= 9                                                  # an outlier channel, clipped below
    codes, s16, z16, info = oracle.quantize_group_lloyd_max(y, 4.0)
    z = z16.view(np.float16).astype(np.float64)
    u = s16.view(np.float16).astype(np.float64)
    levels = (-10.0, -3.0, 3.0, 10.0)
    n_edge = 0
    for r in range(y.shape[0]):
        for c in range(y.shape[1]):
            v = float(info["yc"][r, c])
            dist = [abs(v - (z[r] + lv * u[r])) for lv in levels]
            best = int(np.argmin(dist))
            if codes[r, c] != best:                               # only on a midpoint, up to fp32 rounding
                mid = z[r] + 0.5 * (levels[best] + levels[codes[r, c]]) * u[r]
                assert abs(v - mid) <= 1e-6 * max(abs(mid), u[r]), (r, c)
                n_edge += 1
    assert n_edge <= 2


def test_group_statistics_by_exact_summation():
    rng = np.random.default_rng(2)
    y = (rng.standard_normal((16, 128)) * 2 + rng.standard_normal((16, 1))).astype(np.float32)
    _, s16, z16, _ = oracle.quantize_group_lloyd_max(y, 6.0)
    for r in range(16):
        yc = [min(max(float(v), -6.0), 6.0) for v in y[r]]
        mean = math.fsum(yc) / len(yc)
        dev = math.sqrt(math.fsum((v - mean) ** 2 for v in yc) / len(yc))
        assert z16[r] == np.float16(np.float32(mean)).view(np.uint16)
        assert s16[r] == np.float16(np.float32(0.15104 * dev)).view(np.uint16)


def test_gaussian_mse_is_the_lloyd_max_optimum():
    """For Gaussian groups the 4-level Lloyd-Max quantiser has normalised MSE
    0.1175; the uniform min-max INT2 of the same groups is several times worse."""
    rng = np.random.default_rng(3)
    y = rng.standard_normal((64, 4096)).astype(np.float32)
    lm = []
    un = []
    for cb, out in (("lloyd_max", lm), ("uniform", un)):
        q = oracle.quantize_group_lloyd_max if cb == "lloyd_max" else oracle.quantize_group
        codes, s16, z16, info = q(y, 1e4)
        xh = (z16.view(np.float16).astype(np.float64)[:, None]
              + oracle.code_levels(cb)[codes] * s16.view(np.float16).astype(np.float64)[:, None])
        out.append(np.mean((xh - info["yc"]) ** 2) / np.var(info["yc"].astype(np.float64)))
    assert abs(lm[0] - 0.1175) < 0.003
    assert un[0] > 3 * lm[0]


def test_centroid_condition():
    """Each level is (nearly) the mean of the values it receives."""
    rng = np.random.default_rng(4)
    y = rng.standard_normal((16, 8192)).astype(np.float32)
    codes, s16, z16, info = oracle.quantize_group_lloyd_max(y, 1e4)
    u = s16.view(np.float16).astype(np.float64)[:, None]
    z = z16.view(np.float16).astype(np.float64)[:, None]
    units = (info["yc"] - z) / u
    for c, lv in enumerate((-10.0, -3.0, 3.0, 10.0)):
        assert abs(units[codes == c].mean() - lv) < 0.05 * abs(lv)


@pytest.mark.parametrize("rot", ["orth", "eye"])
def test_decode_over_lloyd_max_cache_matches_materialised_attention(rot):
    cfg, pools, truth = pins.make_small_cache(seed=31, B=2, Hq=6, nkv=3, d=32, sink=(5, 0), hist=(70, 9),
                                              recent=(3, 11), rot=rot, codebook="lloyd_max")
    ref = pins.sdpa_reference(cfg, truth)
    got = oracle.decode_attn_ref(cfg, *pools)
    assert np.allclose(got, ref, atol=2e-6, rtol=1e-5)
    # the uniform reading of the same codes is a different cache
    plain = dict(cfg)
    plain.pop("codebook")
    assert not np.allclose(oracle.decode_attn_ref(plain, *pools), ref, atol=1e-3)


def test_quantize_pack_ref_lloyd_max_round_trip():
    """Packing and page placement are shared with the uniform codebook: the
    codes read back from the pages are the group codes."""
    rng = np.random.default_rng(5)
    d, n_kv = 64, 2
    x = pins.synth.f32_to_bf16_bits(rng.standard_normal((9, n_kv, d)).astype(np.float32))
    rot = np.stack([np.eye(d, dtype=np.float32)] * n_kv)
    slots = rng.permutation(3 * 64)[:9].astype(np.int32)
    kc = np.zeros((3, n_kv, 64 * d // 4), np.uint8)
    ks = np.zeros((3, n_kv, 64, 2), np.uint16)
    diag = oracle.quantize_pack_ref("k", x, rot, 3.0, slots, kc, ks, codebook="lloyd_max")
    for g in range(n_kv):
        codes, s16, z16 = oracle.read_history_codes("k", kc, ks, slots // 64, slots % 64, g, d)
        assert np.array_equal(codes, diag["codes"][:, g])
        assert np.array_equal(s16, diag["scale16"][:, g]) and np.array_equal(z16, diag["zero16"][:, g])

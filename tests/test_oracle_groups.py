"""Pins of the oracle's sub-head quantisation groups (64 and 32 channels at
head_dim 128): a grouped row equals its blocks quantised one by one, group =
head_dim reduces to the whole-head quantiser, each group's extremes map to
codes 0 and 3, the group-planar scale/zero pool round-trips, and decode
attention over a grouped cache matches the cache materialised channel by
channel with its group's scale and zero."""
import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("group", [64, 32])
@pytest.mark.parametrize("codebook", ["uniform", "lloyd_max"])
def test_grouped_rows_are_independent_blocks(codebook, group):
    rng = np.random.default_rng(1)
    q = oracle.quantize_group if codebook == "uniform" else oracle.quantize_group_lloyd_max
    y = (rng.standard_normal((9, 128)) * np.linspace(0.2, 4.0, 128)).astype(np.float32)
    codes, s16, z16, _ = oracle.quantize_rows_grouped(q, y, 5.0, group)
    assert s16.shape == (9, 128 // group)
    for j in range(128 // group):
        blk = slice(group * j, group * (j + 1))
        cj, sj, zj, _ = q(np.ascontiguousarray(y[:, blk]), 5.0)
        assert np.array_equal(codes[:, blk], cj)
        assert np.array_equal(s16[:, j], sj) and np.array_equal(z16[:, j], zj)
    c1, s1, z1, _ = oracle.quantize_rows_grouped(q, y, 5.0, 128)
    cw, sw, zw, _ = q(y, 5.0)
    assert np.array_equal(c1, cw) and np.array_equal(s1[:, 0], sw) and np.array_equal(z1[:, 0], zw)


@pytest.mark.parametrize("group", [64, 32])
def test_group_extremes_map_to_the_end_codes(group):
    rng = np.random.default_rng(2)
    y = rng.standard_normal((5, 128)).astype(np.float32)
    codes, _, _, info = oracle.quantize_rows_grouped(oracle.quantize_group, y, 100.0, group)
    for r in range(5):
        for j in range(128 // group):
            blk = slice(group * j, group * (j + 1))
            assert codes[r, blk][np.argmin(y[r, blk])] == 0 and codes[r, blk][np.argmax(y[r, blk])] == 3


@pytest.mark.parametrize("kind", ["k", "v"])
@pytest.mark.parametrize("group", [64, 32])
def test_group_planar_pool_round_trip(group, kind):
    rng = np.random.default_rng(3)
    d, n_kv = 128, 2
    ng = d // group
    x = pins.synth.f32_to_bf16_bits(rng.standard_normal((11, n_kv, d)).astype(np.float32))
    rot = np.stack([np.eye(d, dtype=np.float32)] * n_kv)
    slots = rng.permutation(3 * 64)[:11].astype(np.int32)
    kc = np.zeros((3, n_kv, 64 * d // 4), np.uint8)
    ks = np.zeros((3, n_kv, 64 * ng, 2), np.uint16)
    diag = oracle.quantize_pack_ref(kind, x, rot, 3.0, slots, kc, ks, group=group)
    for g in range(n_kv):
        codes, s16, z16 = oracle.read_history_codes(kind, kc, ks, slots // 64, slots % 64, g, d)
        assert np.array_equal(codes, diag["codes"][:, g])
        assert np.array_equal(s16, diag["scale16"][:, g]) and np.array_equal(z16, diag["zero16"][:, g])
        for j in range(ng):   # group j of token o at j*64 + o
            assert np.array_equal(ks[slots // 64, g, j * 64 + slots % 64, 0], diag["scale16"][:, g, j])
            assert np.array_equal(ks[slots // 64, g, j * 64 + slots % 64, 1], diag["zero16"][:, g, j])
    with pytest.raises(ValueError):
        oracle.quantize_pack_ref(kind, x, rot, 3.0, slots, kc, np.zeros((3, n_kv, 64, 2), np.uint16), group=group)


@pytest.mark.parametrize("d,groups", [(32, 2), (32, 4), (128, 4)])
@pytest.mark.parametrize("codebook", ["uniform", "lloyd_max"])
def test_decode_over_grouped_cache_matches_materialised_attention(codebook, d, groups):
    cfg, pools, truth = pins.make_small_cache(seed=41, B=2, Hq=6, nkv=3, d=d, sink=(5, 0), hist=(70, 9),
                                              recent=(3, 11), codebook=codebook, groups=groups)
    assert pools[2].shape[2] == 64 * groups
    ref = pins.sdpa_reference(cfg, truth)
    assert np.allclose(oracle.decode_attn_ref(cfg, *pools), ref, atol=2e-6, rtol=1e-5)

"""GPU parity of sub-head quantisation groups (oscar.h OSCAR_GROUPS_64 and
OSCAR_GROUPS_32) against the oracle: the demotion on every kernel path (one
block per token, the matrix-core tiles with their exact pass at head_dim 128,
the fp64 tiles at head_dim 64), both codebooks; the decode over grouped pools
for every group size, with ragged segments, a demoted layer, shared-prefix
pairs; head_dim 64, where a 64-channel group is the whole head and a
32-channel group is half of it."""
import numpy as np
import pytest

import oracle
import pins
import synth
from gpu_util import compare_out, compare_quant, gpu_decode, gpu_quantize, oracle_pools

pytestmark = pytest.mark.gpu
CODEBOOKS = ["uniform", "lloyd_max"]
GROUPS = [64, 32]


def _oracle(kind, x, rot, clip, slots, n_pages, codebook, group):
    n_kv, d = rot.shape[0], rot.shape[-1]
    c = np.zeros((n_pages, n_kv, 64 * d // 4), np.uint8)
    s = np.zeros((n_pages, n_kv, 64 * (d // group), 2), np.uint16)
    diag = oracle.quantize_pack_ref(kind, x, rot, clip, slots, c, s, codebook=codebook, group=group)
    return c, s, diag


def _tokens(seed, n_tok, n_kv, d, n_pages):
    rng = np.random.default_rng(seed)
    x = synth.kv_tokens(rng, (n_tok,), n_kv, d, synth.outlier_channels(rng, n_kv, d, 3))
    return rng, x, rng.permutation(n_pages * 64)[:n_tok].astype(np.int32)


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("n_tok", [7, 300])          # one block per token / 32-token tiles
@pytest.mark.parametrize("codebook", CODEBOOKS)
@pytest.mark.parametrize("kind", ["k", "v"])
def test_demotion_signed_permutation_bit_exact(kind, codebook, n_tok, group):
    rng, x, slots = _tokens(21, n_tok, 3, 128, 6)
    rot = np.stack([pins.signed_permutation(128, rng)[0] for _ in range(3)])
    ref = _oracle(kind, x, rot, 9.5, slots, 6, codebook, group)
    got = gpu_quantize(kind, x, rot, 9.5, slots, 6, codebook=codebook, group_channels=group)
    compare_quant(kind, got[0], got[1], ref[0], ref[1], ref[2], 128, exact=True, codebook=codebook)


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("codebook", CODEBOOKS)
@pytest.mark.parametrize("kind", ["k", "v"])
def test_demotion_real_rotation(kind, codebook, group):
    rng, x, slots = _tokens(22, 500, 2, 128, 9)
    rot = np.stack([synth.make_rotation(128, rng) for _ in range(2)])
    tau = synth.clip_threshold(x, rot)
    ref = _oracle(kind, x, rot, tau, slots, 9, codebook, group)
    got = gpu_quantize(kind, x, rot, tau, slots, 9, codebook=codebook, group_channels=group)
    compare_quant(kind, got[0], got[1], ref[0], ref[1], ref[2], 128, codebook=codebook)


def test_demotion_32_channel_groups_many_tiles():
    """The matrix-core tiles and their exact pass over several blocks and a
    ragged last tile, every group on its own scale."""
    rng, x, slots = _tokens(24, 64 * 40 + 13, 2, 128, 48)
    rot = np.stack([synth.make_rotation(128, rng) for _ in range(2)])
    tau = synth.clip_threshold(x, rot)
    for kind in ("k", "v"):
        ref = _oracle(kind, x, rot, tau, slots, 48, "uniform", 32)
        got = gpu_quantize(kind, x, rot, tau, slots, 48, group_channels=32)
        compare_quant(kind, got[0], got[1], ref[0], ref[1], ref[2], 128)


def test_head_dim_64_group_is_the_whole_head():
    rng, x, slots = _tokens(23, 40, 2, 64, 2)
    rot = np.stack([synth.make_rotation(64, rng) for _ in range(2)])
    a = gpu_quantize("k", x, rot, 9.0, slots, 2)
    b = gpu_quantize("k", x, rot, 9.0, slots, 2, group_channels=64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("n_tok", [7, 300])          # one block per token / fp64 tiles
@pytest.mark.parametrize("codebook", CODEBOOKS)
@pytest.mark.parametrize("kind", ["k", "v"])
def test_head_dim_64_with_32_channel_groups(kind, codebook, n_tok):
    rng, x, slots = _tokens(25, n_tok, 2, 64, 6)
    rot = np.stack([synth.make_rotation(64, rng) for _ in range(2)])
    tau = synth.clip_threshold(x, rot)
    ref = _oracle(kind, x, rot, tau, slots, 6, codebook, 32)
    got = gpu_quantize(kind, x, rot, tau, slots, 6, codebook=codebook, group_channels=32)
    compare_quant(kind, got[0], got[1], ref[0], ref[1], ref[2], 64, codebook=codebook)


@pytest.mark.parametrize("d,group", [(128, 64), (128, 32), (64, 32)])
@pytest.mark.parametrize("codebook", CODEBOOKS)
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_decode_ragged_segments(G, codebook, d, group):
    cfg, pools, _ = pins.make_small_cache(seed=60 + G + group, B=3, Hq=2 * G, nkv=2, d=d, sink=(64, 5, 0),
                                          hist=(0, 37, 200), recent=(256, 1, 100), sink_cap=64, recent_cap=256,
                                          codebook=codebook, groups=d // group)
    cfg["group_channels"] = group
    ref = oracle.decode_attn_ref(cfg, *pools)
    compare_out(gpu_decode(cfg, pools), ref, what=f"{group}-channel groups d={d} G={G} {codebook}")


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("codebook", CODEBOOKS)
def test_decode_demoted_layer(codebook, group):
    shape = synth.DecodeShape("groups-b2-h16kv2-d128", 2, 16, 2, 128, 64 + 256 + 64 * 30 + 17)
    cfg = dict(synth.make_decode_config(0, shape=shape, seed_index=71), codebook=codebook, group_channels=group)
    pools = oracle_pools(cfg)
    compare_out(gpu_decode(cfg, pools), oracle.decode_attn_ref(cfg, *pools),
                what=f"demoted {group}-channel grouped layer {codebook}")


@pytest.mark.parametrize("group", GROUPS)
def test_decode_shared_prefix_pairs(group):
    shape = synth.DecodeShape("groups-prefix", 3, 8, 2, 128, 64 + 256 + 64 * 21, shared_hist_pages=13)
    cfg = dict(synth.make_decode_config(0, shape=shape, seed_index=72), group_channels=group)
    pools = oracle_pools(cfg)
    ref = oracle.decode_attn_ref(cfg, *pools)
    compare_out(gpu_decode(cfg, pools, shared_pages=13), ref, what=f"{group}-channel grouped shared prefix")

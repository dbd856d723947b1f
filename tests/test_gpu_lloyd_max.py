"""GPU parity of the Lloyd-Max codebook variant (oscar.h
OSCAR_CODEBOOK_LLOYD_MAX) against the oracle: the demotion on both of its
paths (one block per token, 32-token tiles), bit-exact with a signed
permutation and under the bin-edge rule with real rotations; and the decode
over Lloyd-Max pools for every group size, head dim and segment shape."""
import numpy as np
import pytest

import oracle
import pins
import synth
from gpu_util import compare_out, compare_quant, gpu_decode, gpu_quantize, oracle_pools

pytestmark = pytest.mark.gpu
LM = "lloyd_max"


def _oracle(kind, x, rot, clip, slots, n_pages):
    n_kv, d = rot.shape[0], rot.shape[-1]
    c = np.zeros((n_pages, n_kv, 64 * d // 4), np.uint8)
    s = np.zeros((n_pages, n_kv, 64, 2), np.uint16)
    diag = oracle.quantize_pack_ref(kind, x, rot, clip, slots, c, s, codebook=LM)
    return c, s, diag


@pytest.mark.parametrize("n_tok", [7, 300])          # one block per token / 32-token tiles
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", ["k", "v"])
def test_demotion_signed_permutation_bit_exact(kind, d, n_tok):
    rng = np.random.default_rng(11 + d)
    outl = synth.outlier_channels(rng, 3, d, 3)
    x = synth.kv_tokens(rng, (n_tok,), 3, d, outl)
    slots = rng.permutation(6 * 64)[:n_tok].astype(np.int32)
    rot = np.stack([pins.signed_permutation(d, rng)[0] for _ in range(3)])
    ref = _oracle(kind, x, rot, 9.5, slots, 6)
    got = gpu_quantize(kind, x, rot, 9.5, slots, 6, codebook=LM)
    compare_quant(kind, got[0], got[1], ref[0], ref[1], ref[2], d, exact=True, codebook=LM)


@pytest.mark.parametrize("kind", ["k", "v"])
def test_demotion_tiny_history(kind):
    cfg = synth.make_decode_config(0)
    x, rot, tau = cfg["hist_" + kind], cfg["r_" + kind], cfg["tau_" + kind]
    ref = _oracle(kind, x, rot, tau, cfg["hist_slot"], cfg["n_pages"])
    got = gpu_quantize(kind, x, rot, tau, cfg["hist_slot"], cfg["n_pages"], codebook=LM)
    compare_quant(kind, got[0], got[1], ref[0], ref[1], ref[2], cfg["head_dim"], codebook=LM)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_ragged_segments(G, d):
    cfg, pools, _ = pins.make_small_cache(seed=50 + G + d, B=3, Hq=2 * G, nkv=2, d=d, sink=(64, 5, 0),
                                          hist=(0, 37, 200), recent=(256, 1, 100), sink_cap=64, recent_cap=256,
                                          codebook=LM)
    ref = oracle.decode_attn_ref(cfg, *pools)
    compare_out(gpu_decode(cfg, pools), ref, what=f"Lloyd-Max ragged G={G} d={d}")


def test_decode_tiny_config_demoted_history():
    cfg = dict(synth.make_decode_config(0), codebook=LM)
    pools = oracle_pools(cfg)
    compare_out(gpu_decode(cfg, pools), oracle.decode_attn_ref(cfg, *pools), what="Lloyd-Max tiny config")


def test_decode_shared_prefix_pairs():
    shape = synth.DecodeShape("lm-prefix", 3, 8, 2, 128, 64 + 256 + 64 * 21, shared_hist_pages=13)
    cfg = dict(synth.make_decode_config(0, shape=shape, seed_index=61), codebook=LM)
    pools = oracle_pools(cfg)
    ref = oracle.decode_attn_ref(cfg, *pools)
    compare_out(gpu_decode(cfg, pools, shared_pages=13), ref, what="Lloyd-Max shared prefix")

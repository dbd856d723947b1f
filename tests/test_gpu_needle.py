"""Long-context retrieval pattern: one dominant history token over a flat
background 2^-17 .. 2^-30 lighter, on waves of the two lengths the split
policy produces for the 100k workloads (7 pages per wave at batch 1, 56 at
28 requests).  Every background token is light enough that a fixed-point
weight with 2^18 units at the reference would drop it from the value sum
while its weight still counts; the oracle's fp64 attention over the same
cache is the reference.

Construction: R_K = R_V = I, q = 0.25 in every channel and all K codes 0, so
a history token's log2 logit is sm * log2(e) * 32 * zero_K: the K zero
points set the logits exactly.  V codes are random, V scales 4..6 (the range
of clipped rotated values / 3) and V zeros near -1.5 scale.  Sink and recent
windows are empty, so history decides the output."""
import numpy as np
import pytest

import oracle
from gpu_util import PAGE, compare_out, gpu_decode

pytestmark = pytest.mark.gpu


def needle_cache(seed, B, n_kv, G, pages, band, where, codebook="uniform"):
    rng = np.random.default_rng(seed)
    d = 128
    Hq = n_kv * G
    hl = pages * PAGE
    sm = np.float32(1 / np.sqrt(d))
    q = np.full((B, Hq, d), 0x3E80, np.uint16)                  # bf16 0.25
    per_z = float(sm) * 1.4426950408889634 * 32.0               # log2 logit per unit of zero_K
    lg = -rng.uniform(*band, size=hl)
    pos = {"first": 0, "middle": hl // 2 + 37, "last": hl - 1}[where]
    lg[pos] = 0.0
    zk = (lg / per_z).astype(np.float16)
    kc = np.zeros((pages, n_kv, PAGE * d // 4), np.uint8)
    ks = np.zeros((pages, n_kv, PAGE, 2), np.uint16)
    ks[..., 0] = np.float16(1.0).view(np.uint16)
    ks[..., 1] = zk.reshape(pages, PAGE).view(np.uint16)[:, None, :]
    vc = rng.integers(0, 256, size=(pages, n_kv, PAGE * d // 4), dtype=np.uint8)
    unit = 1.0 if codebook == "uniform" else 0.1                # Lloyd-Max scales are ~0.15 sigma
    sv = (unit * rng.uniform(4.0, 6.0, size=(pages, n_kv, PAGE))).astype(np.float16)
    zv = (-1.5 * sv.astype(np.float32) + rng.normal(0, 0.3, size=sv.shape)).astype(np.float16)
    vs = np.stack([sv.view(np.uint16), zv.view(np.uint16)], axis=-1)
    table = np.tile(rng.permutation(pages).astype(np.int32), (B, 1))
    eye = np.stack([np.eye(d, dtype=np.float32)] * n_kv)
    cfg = dict(q=q, sink_k=np.zeros((B, n_kv, 64, d), np.uint16), sink_v=np.zeros((B, n_kv, 64, d), np.uint16),
               recent_k=np.zeros((B, n_kv, 256, d), np.uint16), recent_v=np.zeros((B, n_kv, 256, d), np.uint16),
               sink_len=np.zeros(B, np.int32), recent_len=np.zeros(B, np.int32),
               hist_len=np.full(B, hl, np.int32), block_table=table, r_k=eye, r_v=eye, sm_scale=sm)
    if codebook != "uniform":
        cfg["codebook"] = codebook
    return cfg, (kc, vc, ks, vs)


# (B, n_kv, G, pages): the split policy gives 27 pages per split, 7 per wave,
# for 64 units of 80 pages; one split of 224 pages, 56 per wave, for 88 units
WAVES = {7: (8, 8, 8, 80), 56: (11, 8, 4, 224)}


@pytest.mark.parametrize("codebook", ["uniform", "lloyd_max"])
@pytest.mark.parametrize("where", ["first", "middle", "last"])
@pytest.mark.parametrize("band", [(17, 22), (22, 30)])
@pytest.mark.parametrize("wave_pages", [7, 56])
def test_needle_over_flat_background(wave_pages, band, where, codebook):
    B, n_kv, G, pages = WAVES[wave_pages]
    cfg, pools = needle_cache(100 + wave_pages, B, n_kv, G, pages, band, where, codebook)
    Hq = n_kv * G
    got = gpu_decode(cfg, pools)
    ref = oracle.decode_attn_ref(cfg, *pools, heads=[(0, h) for h in range(Hq)])
    compare_out(got[:1], ref[:1], what=f"needle over 2^-{band[0]}..2^-{band[1]}, {wave_pages}-page waves, {where}")
    # every request holds the same pages and query: the same result, bit for bit
    assert np.array_equal(got, np.broadcast_to(got[:1], got.shape))


def test_needle_with_shared_prefix_pairs():
    """The 56-page waves of request pairs reading a declared shared prefix."""
    B, n_kv, G, pages = WAVES[56]
    cfg, pools = needle_cache(7, B, n_kv, G, pages, (17, 24), "middle")
    got = gpu_decode(cfg, pools, shared_pages=pages)
    ref = oracle.decode_attn_ref(cfg, *pools, heads=[(0, h) for h in range(n_kv * G)])
    compare_out(got[:1], ref[:1], what="needle, shared-prefix pairs")
    assert np.array_equal(got, np.broadcast_to(got[:1], got.shape))

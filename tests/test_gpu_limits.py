"""The history path at its design limits.

With 88 (request, KV head) units and 256 history pages, the split policy
gives one split of 256 pages per unit, so every history wave scans the
maximum of 64 pages.  The cache is built so that no rescale ever fires and
the PV operands and sums grow as large as the design allows: every V code is
2 or 3 (the largest operands), the V scales are equal (no scale-driven
rescale), and from the second page on every logit sits 11.5 log2-units above
the first page's maximum, just under the lazy-rescale threshold of 12, so
every weight p*scale_V*kap is near the 2^14 top of its fp16 pair and the
fp32 sums run over 4096 such tokens unscaled.  The oracle's fp64 attention
over the same cache is the reference."""
import numpy as np
import pytest

import oracle
from gpu_util import PAGE, compare_out, gpu_decode

pytestmark = pytest.mark.gpu


def _limit_cache(codebook, groups=1):
    rng = np.random.default_rng(404)
    B, n_kv, G, d, hp = 11, 8, 1, 128, 256
    Hq = n_kv * G
    hl = hp * PAGE
    sm = np.float32(1 / np.sqrt(d))
    # q = 0.25 everywhere: sum(q_rot) = 32 with R = I, so a K row of all-zero codes and zero z gives
    # the log2 logit sm * log2(e) * 32 * z
    q = np.full((B, Hq, d), 0x3E80, np.uint16)                  # bf16 0.25
    per_z = float(sm) * 1.4426950408889634 * 32.0
    z_first = rng.uniform(0.0, 0.05, size=(PAGE,)) / per_z        # page 0: logits in [0, 0.05]
    z_rest = (11.5 - rng.uniform(0.0, 0.4, size=(hp - 1, PAGE))) / per_z
    zk = np.concatenate([z_first[None], z_rest]).astype(np.float16)          # [page][token]
    kc = np.zeros((hp, n_kv, PAGE * d // 4), np.uint8)
    fields = rng.integers(2, 4, size=(hp, n_kv, PAGE * d // 4, 4)).astype(np.uint8)   # codes 2 or 3
    vc = (fields[..., 0] | (fields[..., 1] << 2) | (fields[..., 2] << 4) | (fields[..., 3] << 6)).astype(np.uint8)
    ks = np.zeros((hp, n_kv, PAGE, 2), np.uint16)
    ks[..., 0] = np.float16(1.0).view(np.uint16)
    ks[..., 1] = zk.view(np.uint16)[:, None, :]
    vs = np.zeros((hp, n_kv, PAGE, 2), np.uint16)
    vs[..., 0] = np.float16(0.75).view(np.uint16)
    vs[..., 1] = np.float16(-1.0).view(np.uint16)
    if groups > 1:   # the same K pairs for every group, V groups past the first at a smaller scale
        ks = np.concatenate([ks] * groups, axis=2)
        vs2 = vs.copy()
        vs2[..., 0] = np.float16(0.5).view(np.uint16)
        vs = np.concatenate([vs] + [vs2] * (groups - 1), axis=2)
    table = np.tile(rng.permutation(hp).astype(np.int32), (B, 1))
    eye = np.stack([np.eye(d, dtype=np.float32)] * n_kv)
    cfg = dict(q=q, sink_k=np.zeros((B, n_kv, 64, d), np.uint16), sink_v=np.zeros((B, n_kv, 64, d), np.uint16),
               recent_k=np.zeros((B, n_kv, 256, d), np.uint16), recent_v=np.zeros((B, n_kv, 256, d), np.uint16),
               sink_len=np.zeros(B, np.int32), recent_len=np.zeros(B, np.int32),
               hist_len=np.full(B, hl, np.int32), block_table=table, r_k=eye, r_v=eye, sm_scale=sm)
    if codebook != "uniform":
        cfg["codebook"] = codebook
    if groups > 1:
        cfg["group_channels"] = d // groups
    return cfg, (kc, vc, ks, vs)


@pytest.mark.parametrize("groups", [1, 2, 4])
@pytest.mark.parametrize("codebook", ["uniform", "lloyd_max"])
def test_longest_wave_range_at_the_integer_bound(codebook, groups):
    cfg, pools = _limit_cache(codebook, groups)
    B, Hq, d = cfg["q"].shape
    got = gpu_decode(cfg, pools)
    ref = oracle.decode_attn_ref(cfg, *pools, heads=[(0, h) for h in range(Hq)])
    compare_out(got[:1], ref[:1], what=f"64-page waves at the integer bound ({codebook}, {groups} groups)")
    # every request holds the same pages and query: the same partials, bit for bit
    assert np.array_equal(got, np.broadcast_to(got[:1], got.shape))

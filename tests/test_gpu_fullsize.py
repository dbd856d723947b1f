"""Full-size parity in the launch configurations the benchmark times.

* The GPU demotion of the whole history of the 32k and 100k layers (the
  benchmark fills its cache replicas with exactly these launches) and of the
  whole bulk-demotion workload (131072 tokens x 8 heads, K and V), compared
  with the oracle quantiser slot by slot: scale/zero bit-exact, codes
  bit-exact except the bin-edge rule.
* The same with 64- and 32-channel quantisation groups (the 100k layer's
  history and the bulk workload), and the 100k layer's decode over
  oracle-quantised grouped pools, every head.
* The 28-request, 100k-context layer with its 1406-page shared prefix
  declared to the scan (packs of four requests read each shared split once),
  and the same with the prefix in cascade blocks (groups of 16 requests): all
  32 query heads of four requests (the first and the last, and two members of
  one pack) against the oracle over oracle-quantised pages.  The private
  pages of the other requests hold random codes; their rows are checked to
  be finite."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import PAGE, compare_out, compare_quant, gpu_decode, gpu_quantize, oracle_pools

pytestmark = pytest.mark.gpu


def _oracle_pools(kind, x, rot, tau, slots, n_pages, src_idx=None, group=None):
    n_kv, d = rot.shape[0], rot.shape[-1]
    ng = 1 if group is None else d // group
    c = np.zeros((n_pages, n_kv, PAGE * d // 4), np.uint8)
    s = np.zeros((n_pages, n_kv, PAGE * ng, 2), np.uint16)
    diag = oracle.quantize_pack_ref(kind, x, rot, tau, slots, c, s, src_idx=src_idx, group=group)
    return c, s, diag


@pytest.mark.parametrize("cfg_index", [1, 3])
def test_history_demotion_of_decode_layers(cfg_index):
    cfg = synth.make_decode_config(cfg_index)
    for kind in ("k", "v"):
        x, rot, tau = cfg["hist_" + kind], cfg["r_" + kind], cfg["tau_" + kind]
        gc, gs = gpu_quantize(kind, x, rot, tau, cfg["hist_slot"], cfg["n_pages"])
        rc, rs, diag = _oracle_pools(kind, x, rot, tau, cfg["hist_slot"], cfg["n_pages"])
        compare_quant(kind, gc, gs, rc, rs, diag, cfg["head_dim"])


def test_bulk_demotion_whole_workload():
    cfg = synth.make_bulk_demotion_config()
    for kind in ("k", "v"):
        x, rot, tau = cfg["x_" + kind], cfg["r_" + kind], cfg["tau_" + kind]
        gc, gs = gpu_quantize(kind, x, rot, tau, cfg["dst_slot"], cfg["n_pages"])
        rc, rs, diag = _oracle_pools(kind, x, rot, tau, cfg["dst_slot"], cfg["n_pages"])
        compare_quant(kind, gc, gs, rc, rs, diag, cfg["head_dim"])
        assert np.count_nonzero(gs[..., 0]) == gs[..., 0].size   # every slot written, no degenerate group


@pytest.mark.parametrize("group", [64, 32])
def test_history_demotion_of_the_100k_layer_grouped(group):
    cfg = synth.make_decode_config(3)
    for kind in ("k", "v"):
        x, rot, tau = cfg["hist_" + kind], cfg["r_" + kind], cfg["tau_" + kind]
        gc, gs = gpu_quantize(kind, x, rot, tau, cfg["hist_slot"], cfg["n_pages"], group_channels=group)
        rc, rs, diag = _oracle_pools(kind, x, rot, tau, cfg["hist_slot"], cfg["n_pages"], group=group)
        compare_quant(kind, gc, gs, rc, rs, diag, cfg["head_dim"])


def test_bulk_demotion_whole_workload_32_channel_groups():
    cfg = synth.make_bulk_demotion_config()
    for kind in ("k", "v"):
        x, rot, tau = cfg["x_" + kind], cfg["r_" + kind], cfg["tau_" + kind]
        gc, gs = gpu_quantize(kind, x, rot, tau, cfg["dst_slot"], cfg["n_pages"], group_channels=32)
        rc, rs, diag = _oracle_pools(kind, x, rot, tau, cfg["dst_slot"], cfg["n_pages"], group=32)
        compare_quant(kind, gc, gs, rc, rs, diag, cfg["head_dim"])


@pytest.mark.parametrize("group", [64, 32])
def test_qwen3_32b_layer_100k_grouped(group):
    cfg = dict(synth.make_decode_config(3), group_channels=group)
    pools = oracle_pools(cfg)
    ref = oracle.decode_attn_ref(cfg, *pools)
    got = gpu_decode(cfg, pools)
    compare_out(got, ref, what=f"Qwen3-32B layer, 100k, {group}-channel groups")


def test_batch28_shared_prefix_four_requests_all_heads():
    cfg = synth.make_decode_config(4)
    shape = cfg["shape"]
    B, n_kv, d, P = cfg["batch"], cfg["n_kv"], cfg["head_dim"], cfg["n_pages"]
    hl = shape.hist_len
    shared = shape.shared_hist_pages
    private = hl - shared * PAGE
    check = [0, 13, 14, 27]
    # tokens of hist_slot order: request 0's whole history, then each later request's private part
    rows = [np.arange(hl)] + [hl + (b - 1) * private + np.arange(private) for b in check if b > 0]
    sel = np.concatenate(rows)
    rng = np.random.default_rng(28)
    sigma = float(np.sqrt((d - 3 + 3 * 400) / d))
    pools = []
    for kind in ("k", "v"):
        c, s = synth.random_pages(rng, P, n_kv, d, sigma)
        oracle.quantize_pack_ref(kind, cfg["hist_" + kind], cfg["r_" + kind], cfg["tau_" + kind],
                                 cfg["hist_slot"][sel], c, s, src_idx=sel)
        pools.append((c, s))
    pools = (pools[0][0], pools[1][0], pools[0][1], pools[1][1])
    got = gpu_decode(cfg, pools, shared_pages=shared)
    casc = gpu_decode(cfg, pools, shared_pages=shared, prefix_cascade=True)
    ref = oracle.decode_attn_ref(cfg, *pools, heads=[(b, h) for b in check for h in range(cfg["n_q_heads"])])
    compare_out(got[check], ref[check], what="28 x 100k, four requests, all heads")
    compare_out(casc[check], ref[check], what="28 x 100k in cascade blocks, four requests, all heads")
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(casc))

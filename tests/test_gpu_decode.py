"""GPU parity of oscar_decode_attn (and the BF16 comparator) against the oracle.

Decode inputs never come from the HIP path: history pages are written by the
oracle quantiser or by the brute-force page writer of tests/pins.py.  The
100k and 28-request layers in the benchmark's launch configuration are in
tests/test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_attn_amd as hip
import oracle
import pins
import synth
from gpu_util import compare_out, dev, gpu_decode, host, oracle_pools

pytestmark = pytest.mark.gpu
PAGE = 64


def ragged_cache(seed, B, n_kv, G, d, sink, hist, recent, sink_cap=64, recent_cap=256):
    rng = np.random.default_rng(seed)
    cfg, pools, _ = pins.make_small_cache(seed=seed, B=B, Hq=n_kv * G, nkv=n_kv, d=d, sink=sink,
                                          hist=hist, recent=recent, sink_cap=sink_cap,
                                          recent_cap=recent_cap)
    return cfg, pools


def test_tiny_config():
    cfg = synth.make_decode_config(0)
    pools = oracle_pools(cfg)
    ref = oracle.decode_attn_ref(cfg, *pools)
    got = gpu_decode(cfg, pools)
    compare_out(got, ref, what="tiny config")


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_segments(G, d):
    """Partial pages, partial windows, empty history, empty windows."""
    cfg, pools = ragged_cache(10 + G, B=3, n_kv=2, G=G, d=d, sink=(64, 5, 0), hist=(0, 37, 200),
                              recent=(256, 1, 100))
    ref = oracle.decode_attn_ref(cfg, *pools)
    got = gpu_decode(cfg, pools)
    compare_out(got, ref, what=f"ragged G={G} d={d}")


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_large_batch_merge(G, d):
    """16 requests x 2 KV heads: at most 11 history splits per head, so every
    head's partials fit one round and the merge runs one block per (request,
    KV head) (per head when G*d/4 exceeds a block).  Ragged segments, an empty
    history and an empty context among them."""
    rng = np.random.default_rng(70 + G + d)
    B = 16
    hist = [int(x) for x in rng.integers(1, 700, size=B)]
    sink = [int(x) for x in rng.integers(0, 65, size=B)]
    recent = [int(x) for x in rng.integers(0, 257, size=B)]
    hist[3] = 0
    sink[5], hist[5], recent[5] = 0, 0, 0
    cfg, pools = ragged_cache(80 + G + d, B=B, n_kv=2, G=G, d=d, sink=tuple(sink), hist=tuple(hist),
                              recent=tuple(recent))
    ref = oracle.decode_attn_ref(cfg, *pools)
    got = gpu_decode(cfg, pools)
    assert not got[5].any()
    compare_out(got, ref, what=f"large batch G={G} d={d}")


@pytest.mark.parametrize("G", [1, 4, 8])
def test_merge_in_rounds(G):
    """16 requests x 8 KV heads (128 merge units) with a 1024-token recent
    window: 16 BF16 chunks, one sink chunk and the history splits give every
    head more partials than one round of the per-unit merge takes, so they are
    combined in two rounds online (rotated history partials in the first,
    plain chunk partials in both).  Ragged segments, an empty history and an
    empty context among them."""
    rng = np.random.default_rng(95 + G)
    B = 16
    hist = [int(x) for x in rng.integers(1, 900, size=B)]
    sink = [int(x) for x in rng.integers(0, 65, size=B)]
    recent = [int(x) for x in rng.integers(0, 1025, size=B)]
    hist[2] = 0
    sink[7], hist[7], recent[7] = 0, 0, 0
    cfg, pools = ragged_cache(110 + G, B=B, n_kv=8, G=G, d=128, sink=tuple(sink), hist=tuple(hist),
                              recent=tuple(recent), recent_cap=1024)
    ref = oracle.decode_attn_ref(cfg, *pools)
    got = gpu_decode(cfg, pools)
    assert not got[7].any()
    compare_out(got, ref, what=f"merge in rounds G={G}")


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_many_units_every_group_size(G, d):
    """16 requests x 8 KV heads (128 units, the per-unit merge where its
    block holds the unit's heads) for every group size and both head dims.
    Ragged segments, an empty history and an empty context."""
    rng = np.random.default_rng(130 + G + d)
    B = 16
    hist = [int(x) for x in rng.integers(1, 400, size=B)]
    sink = [int(x) for x in rng.integers(0, 65, size=B)]
    recent = [int(x) for x in rng.integers(0, 257, size=B)]
    hist[4] = 0
    sink[9], hist[9], recent[9] = 0, 0, 0
    cfg, pools = ragged_cache(140 + G + d, B=B, n_kv=8, G=G, d=d, sink=tuple(sink), hist=tuple(hist),
                              recent=tuple(recent))
    ref = oracle.decode_attn_ref(cfg, *pools)
    got = gpu_decode(cfg, pools)
    assert not got[9].any()
    compare_out(got, ref, what=f"128 units G={G} d={d}")


@pytest.mark.parametrize("log2_scale", [-100, 0, 64])
def test_query_scale_extremes(log2_scale):
    """q scaled by a power of two far from 1 (exact in bf16): the fixed-point
    scale of the rotated query is taken from the query's norm, which must
    neither overflow (|q| near 2^64: |q|^2 is past the fp32 range) nor
    underflow (|q| near 2^-100).  At 2^64 the softmax is one-hot."""
    cfg, pools = ragged_cache(5, B=2, n_kv=2, G=4, d=128, sink=(64, 3), hist=(300, 130), recent=(256, 7))
    q = (cfg["q"].astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** log2_scale)
    cfg["q"] = (q.view(np.uint32) >> 16).astype(np.uint16)
    assert np.isfinite(q).all() and (q[q != 0] != 0).all()
    ref = oracle.decode_attn_ref(cfg, *pools)
    got = gpu_decode(cfg, pools)
    compare_out(got, ref, what=f"q scaled by 2^{log2_scale}")


def test_empty_context_rows_are_zero():
    cfg, pools = ragged_cache(3, B=2, n_kv=1, G=4, d=64, sink=(0, 3), hist=(0, 70), recent=(0, 2))
    got = gpu_decode(cfg, pools)
    assert not got[0].any()
    compare_out(got, oracle.decode_attn_ref(cfg, *pools), what="empty context")


def test_bad_inputs_poison_only_their_request():
    cfg, pools = ragged_cache(4, B=3, n_kv=2, G=4, d=128, sink=(64, 64, 64), hist=(130, 130, 130),
                              recent=(256, 256, 256))
    ref = oracle.decode_attn_ref(cfg, *pools)
    table = cfg["block_table"].copy()
    table[1, 1] = pools[0].shape[0] + 5          # outside the pool
    hl = cfg["hist_len"].copy()
    hl[2] = 10_000                               # above max_hist_len
    got = gpu_decode(cfg, pools, block_table=table, hist_len=hl, max_hist_len=130)
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2]))
    compare_out(got[:1], ref[:1], what="unaffected request")
    sl = cfg["sink_len"].copy()
    sl[0] = 65                                   # above sink_cap
    got = gpu_decode(cfg, pools, sink_len=sl)
    assert np.all(np.isnan(got[0]))
    compare_out(got[1:], ref[1:], what="unaffected requests")


def test_split_partition_and_page_order_invariance():
    cfg, pools = ragged_cache(6, B=2, n_kv=2, G=8, d=128, sink=(64, 64), hist=(1000, 999),
                              recent=(256, 256))
    ref = oracle.decode_attn_ref(cfg, *pools)
    base = gpu_decode(cfg, pools)
    compare_out(base, ref, what="base")
    # a larger max_hist_len changes pages per split (a different partition)
    wide = np.full((2, 125), -1, np.int32)
    wide[:, : cfg["block_table"].shape[1]] = cfg["block_table"]
    other = gpu_decode(cfg, pools, block_table=wide, max_hist_len=8000)
    compare_out(other, ref, what="other split count")
    # physical page order: same logical pages -> bit-identical
    n_pages = pools[0].shape[0]
    perm = np.random.default_rng(1).permutation(n_pages)
    inv = np.argsort(perm)
    t2 = cfg["block_table"].copy()
    t2[t2 >= 0] = perm[t2[t2 >= 0]]
    moved = gpu_decode(cfg, tuple(p[inv] for p in pools), block_table=t2)
    assert np.array_equal(moved, base)


def test_deterministic():
    cfg = synth.make_decode_config(0)
    pools = oracle_pools(cfg)
    a = gpu_decode(cfg, pools)
    b = gpu_decode(cfg, pools, reps=3)
    assert np.array_equal(a, b)


def test_qwen3_8b_layer_32k():
    cfg = synth.make_decode_config(1)
    pools = oracle_pools(cfg)
    ref = oracle.decode_attn_ref(cfg, *pools)
    got = gpu_decode(cfg, pools)
    compare_out(got, ref, what="Qwen3-8B layer, 32k")


def test_qwen3_32b_layer_100k():
    cfg = synth.make_decode_config(3)
    pools = oracle_pools(cfg)
    ref = oracle.decode_attn_ref(cfg, *pools)
    got = gpu_decode(cfg, pools)
    compare_out(got, ref, what="Qwen3-32B layer, 100k")


# ---- BF16 comparator ------------------------------------------------------
def _gpu_bf16(q, kp, vp, table, ctx, sm):
    B, Hq, d = q.shape
    ws = torch.empty(max(1, hip.oscar_decode_bf16_workspace_bytes(B, Hq, kp.shape[1], d, int(ctx.max()))),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    hip.oscar_decode_attn_bf16(q=dev(q), k_pages=dev(kp), v_pages=dev(vp), block_table=dev(table),
                               ctx_len=dev(ctx), max_ctx_len=int(ctx.max()), out=out, workspace=ws,
                               sm_scale=float(sm))
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("cfg_index", [0, 1])
def test_bf16_comparator(cfg_index):
    cfg = synth.make_decode_config(cfg_index)
    bf = synth.bf16_context_pages(cfg)
    ref = oracle.bf16_paged_attn_ref(cfg["q"], bf["k_pages"], bf["v_pages"], bf["block_table"], bf["ctx_len"],
                                     cfg["sm_scale"])
    got = _gpu_bf16(cfg["q"], bf["k_pages"], bf["v_pages"], bf["block_table"], bf["ctx_len"], cfg["sm_scale"])
    compare_out(got, ref, what=f"bf16 comparator config {cfg_index}")


def test_bf16_comparator_ragged():
    rng = np.random.default_rng(9)
    B, Hq, nkv, d = 3, 16, 2, 128
    ctx = np.array([0, 65, 700], np.int32)
    n_pages = 14
    table = np.full((B, 11), -1, np.int32)
    perm = rng.permutation(n_pages)
    table[1, :2] = perm[:2]
    table[2, :11] = perm[2:13]
    kp = synth.f32_to_bf16_bits(rng.standard_normal((n_pages, nkv, PAGE, d)).astype(np.float32) * 2)
    vp = synth.f32_to_bf16_bits(rng.standard_normal((n_pages, nkv, PAGE, d)).astype(np.float32))
    q = synth.f32_to_bf16_bits(rng.standard_normal((B, Hq, d)).astype(np.float32))
    ref = oracle.bf16_paged_attn_ref(q, kp, vp, table, ctx, 1 / np.sqrt(d))
    got = _gpu_bf16(q, kp, vp, table, ctx, 1 / np.sqrt(d))
    compare_out(got, ref, what="bf16 ragged")


def test_writes_stay_inside_workspace_and_output():
    """Canary bytes around the workspace and the output must survive a call."""
    cfg, pools = ragged_cache(21, B=2, n_kv=2, G=8, d=128, sink=(64, 3), hist=(300, 65), recent=(256, 9))
    B, Hq, d = cfg["q"].shape
    mh = int(cfg["hist_len"].max())
    need = hip.oscar_decode_workspace_bytes(B, Hq, 2, d, mh, 64, 256)
    guard = 1 << 16
    ws_full = torch.full((need + 2 * guard,), 0xAB, dtype=torch.uint8, device="cuda")
    ws = ws_full[guard:guard + need]
    out_full = torch.full((B * Hq * d + 2 * 4096,), 12345.0, dtype=torch.float32, device="cuda")
    out = out_full[4096:4096 + B * Hq * d].view(B, Hq, d)
    kc, vc, ks, vs = (dev(p) for p in pools)
    hip.oscar_decode_attn(q=dev(cfg["q"]), sink_k=dev(cfg["sink_k"]), sink_v=dev(cfg["sink_v"]),
                          recent_k=dev(cfg["recent_k"]), recent_v=dev(cfg["recent_v"]),
                          sink_len=dev(cfg["sink_len"]), recent_len=dev(cfg["recent_len"]),
                          hist_len=dev(cfg["hist_len"]), max_hist_len=mh, k_codes=kc, v_codes=vc, k_sz=ks, v_sz=vs,
                          block_table=dev(cfg["block_table"]), r_k=dev(cfg["r_k"]), r_v=dev(cfg["r_v"]), out=out,
                          workspace=ws, sm_scale=float(cfg["sm_scale"]))
    torch.cuda.synchronize()
    wsh = host(ws_full)
    assert np.all(wsh[:guard] == 0xAB) and np.all(wsh[guard + need:] == 0xAB), "write outside the workspace"
    oh = host(out_full)
    assert np.all(oh[:4096] == 12345.0) and np.all(oh[4096 + B * Hq * d:] == 12345.0), "write outside out"
    compare_out(host(out), oracle.decode_attn_ref(cfg, *pools), what="canary run")

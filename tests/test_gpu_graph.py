"""GPU: oscar_decode_step captured in a HIP graph (as bench.py times it) and
replayed several times, with eager work between the replays, must reproduce
the eager call bit for bit on every replay: the decode output and the pools
the step's demotions write.  The output is filled with NaN before each
replay, so a replay that skipped a write would show."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_attn_amd as hip
import synth
from gpu_util import PAGE, dev, host, oracle_pools

pytestmark = pytest.mark.gpu


def _step_inputs():
    shape = synth.DecodeShape("graph-b3-h16kv2-d128-L1000", 3, 16, 2, 128, 1000)
    cfg = synth.make_decode_config(0, shape=shape, seed_index=9)
    B, Hq, d = cfg["q"].shape
    n_kv, cap = cfg["n_kv"], cfg["recent_k"].shape[2]
    # one free page per request so that slot hist_len exists
    extra = (cfg["n_pages"] + np.arange(B)).astype(np.int32)[:, None]
    cfg = dict(cfg, block_table=np.concatenate([cfg["block_table"], extra], axis=1), n_pages=cfg["n_pages"] + B)
    hl = cfg["hist_len"]
    slot = (cfg["block_table"][np.arange(B), hl // PAGE] * PAGE + hl % PAGE).astype(np.int32)
    src = (np.arange(B) * n_kv * cap + 5).astype(np.int32)
    return cfg, slot, src


def test_decode_step_graph_replays_match_eager():
    cfg, slot, src = _step_inputs()
    B, Hq, d = cfg["q"].shape
    n_kv, cap = cfg["n_kv"], cfg["recent_k"].shape[2]
    pools0 = oracle_pools(cfg)
    pools = [dev(p) for p in pools0]
    t = {k: dev(cfg[k]) for k in ("q", "sink_k", "sink_v", "recent_k", "recent_v", "sink_len", "recent_len",
                                  "hist_len", "block_table", "r_k", "r_v")}
    src_t, slot_t = dev(src), dev(slot)
    ws = torch.empty(hip.oscar_decode_workspace_bytes(B, Hq, n_kv, d, int(cfg["hist_len"].max()), 64, cap),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    # the marshalled arguments keep raw pointers: every tensor above stays referenced
    args = hip.decode_args(q=t["q"], sink_k=t["sink_k"], sink_v=t["sink_v"], recent_k=t["recent_k"],
                           recent_v=t["recent_v"], sink_len=t["sink_len"], recent_len=t["recent_len"],
                           hist_len=t["hist_len"], max_hist_len=int(cfg["hist_len"].max()), k_codes=pools[0],
                           v_codes=pools[1], k_sz=pools[2], v_sz=pools[3], block_table=t["block_table"],
                           r_k=t["r_k"], r_v=t["r_v"], out=out, workspace=ws, sm_scale=float(cfg["sm_scale"]))
    common = dict(src_idx=src_t, n_src=B * n_kv * cap, x_tok_stride=d, x_head_stride=cap * d)
    dk = hip.demote_args(x=t["recent_k"], rot=t["r_k"], clip=float(cfg["tau_k"]), dst_slot=slot_t,
                         codes=pools[0], scale_zero=pools[2], **common)
    dv = hip.demote_args(x=t["recent_v"], rot=t["r_v"], clip=float(cfg["tau_v"]), dst_slot=slot_t,
                         codes=pools[1], scale_zero=pools[3], **common)

    def step():
        hip.oscar_decode_step(args=args, demote_k=dk, demote_v=dv)

    def reset_pools():
        for p, p0 in zip(pools, pools0):
            p.copy_(dev(p0))

    step()
    torch.cuda.synchronize()
    want_out = host(out).copy()
    want_pools = [host(p).copy() for p in pools]
    assert np.isfinite(want_out).all()

    reset_pools()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()

    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        reset_pools()
        out.fill_(float("nan"))
        ws.fill_(rep * 37 % 256)          # the workspace contents on entry must not matter
        scratch.mul_(1.5).add_(1.0)       # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), want_out), f"replay {rep}: output differs from the eager call"
        for k, (p, w) in enumerate(zip(pools, want_pools)):
            assert np.array_equal(host(p), w), f"replay {rep}: pool {k} differs from the eager call"

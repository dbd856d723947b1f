"""oscar_decode_step_static (the entry point that allocates nothing) against
oscar_decode_step with a caller workspace, through the C ABI: two calls in
a row, the second with a smaller input (fewer requests, a shorter history, a
smaller head dim), each bit-identical to the workspace call (the same
kernels read and write the same layout) and within the decode tolerance of
the oracle; the demoted slots equal the oracle quantiser's.  The scratch
buffer keeps the previous call's contents, which the second call must not
depend on."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_attn_amd as hip
import oracle
import synth
from gpu_util import PAGE, compare_out, compare_quant, dev, host, oracle_pools

pytestmark = pytest.mark.gpu


def _case(shape, seed):
    cfg = synth.make_decode_config(0, shape=shape, seed_index=seed)
    B = cfg["q"].shape[0]
    extra = (cfg["n_pages"] + np.arange(B)).astype(np.int32)[:, None]
    cfg = dict(cfg, block_table=np.concatenate([cfg["block_table"], extra], axis=1), n_pages=cfg["n_pages"] + B)
    hl = cfg["hist_len"]
    slot = (cfg["block_table"][np.arange(B), hl // PAGE] * PAGE + hl % PAGE).astype(np.int32)
    return cfg, slot


def _run(cfg, slot, pools_np, static):
    B, Hq, d = cfg["q"].shape
    n_kv, cap = cfg["n_kv"], cfg["recent_k"].shape[2]
    pools = [dev(p) for p in pools_np]
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    hl = int(cfg["hist_len"].max())
    ws = None if static else torch.empty(hip.oscar_decode_workspace_bytes(B, Hq, n_kv, d, hl, 64, cap),
                                         dtype=torch.uint8, device="cuda")
    args = hip.decode_args(q=dev(cfg["q"]), sink_k=dev(cfg["sink_k"]), sink_v=dev(cfg["sink_v"]),
                           recent_k=dev(cfg["recent_k"]), recent_v=dev(cfg["recent_v"]),
                           sink_len=dev(cfg["sink_len"]), recent_len=dev(cfg["recent_len"]),
                           hist_len=dev(cfg["hist_len"]), max_hist_len=hl, k_codes=pools[0], v_codes=pools[1],
                           k_sz=pools[2], v_sz=pools[3], block_table=dev(cfg["block_table"]), r_k=dev(cfg["r_k"]),
                           r_v=dev(cfg["r_v"]), out=out, workspace=ws, sm_scale=float(cfg["sm_scale"]))
    ring = 2
    src = dev((np.arange(B) * n_kv * cap + ring).astype(np.int32))
    common = dict(src_idx=src, n_src=B * n_kv * cap, x_tok_stride=d, x_head_stride=cap * d)
    dk = hip.demote_args(x=dev(cfg["recent_k"]), rot=dev(cfg["r_k"]), clip=float(cfg["tau_k"]), dst_slot=dev(slot),
                         codes=pools[0], scale_zero=pools[2], **common)
    dv = hip.demote_args(x=dev(cfg["recent_v"]), rot=dev(cfg["r_v"]), clip=float(cfg["tau_v"]), dst_slot=dev(slot),
                         codes=pools[1], scale_zero=pools[3], **common)
    if static:
        hip.oscar_decode_step_static(args=args, demote_k=dk, demote_v=dv)
    else:
        hip.oscar_decode_step(args=args, demote_k=dk, demote_v=dv)
    torch.cuda.synchronize()
    return host(out), [host(pools[0]), host(pools[1]), host(pools[2], np.uint16), host(pools[3], np.uint16)]


CASES = [
    synth.DecodeShape("noalloc-b3-h16kv2-d128-L2100", 3, 16, 2, 128, 2100),   # then the smaller call:
    synth.DecodeShape("noalloc-b1-h4kv2-d64-L700", 1, 4, 2, 64, 700),
]


def test_static_scratch_step_matches_workspace_step_twice():
    for i, shape in enumerate(CASES):
        cfg, slot = _case(shape, 30 + i)
        pools = oracle_pools(cfg)
        ref_out = oracle.decode_attn_ref(cfg, *pools)
        ring = 2
        ref_pools = [p.copy() for p in pools]
        dk_ref = oracle.quantize_pack_ref("k", cfg["recent_k"][:, :, ring, :], cfg["r_k"], cfg["tau_k"], slot,
                                          ref_pools[0], ref_pools[2])
        dv_ref = oracle.quantize_pack_ref("v", cfg["recent_v"][:, :, ring, :], cfg["r_v"], cfg["tau_v"], slot,
                                          ref_pools[1], ref_pools[3])
        got_ws, pools_ws = _run(cfg, slot, pools, static=False)
        got_st, pools_st = _run(cfg, slot, pools, static=True)
        assert np.array_equal(got_st, got_ws, equal_nan=True), f"call {i}: output differs from the workspace call"
        for a, b in zip(pools_st, pools_ws):
            assert np.array_equal(a, b), f"call {i}: demoted pools differ from the workspace call"
        compare_out(got_st, ref_out, what=f"static scratch call {i} ({shape.name})")
        d = shape.head_dim
        compare_quant("k", pools_st[0], pools_st[2], ref_pools[0], ref_pools[2], dk_ref, d)
        compare_quant("v", pools_st[1], pools_st[3], ref_pools[1], ref_pools[3], dv_ref, d)

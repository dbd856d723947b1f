"""The binding's marshalled arguments keep their tensors alive.

decode_args and demote_args hand raw device pointers to the C ABI.  Here
every input tensor is created inline in the call (nothing else refers to
it), the caching allocator is then given freed-memory-sized work that would
reuse any block the arguments let go, and the step must still match the
oracle: the decode over the cache as given, and the demoted slots."""
import gc

import numpy as np
import pytest
import torch

import bit_rotated_kv_attn_amd as hip
import oracle
import synth
from gpu_util import PAGE, compare_out, compare_quant, dev, host, oracle_pools

pytestmark = pytest.mark.gpu


def _churn():
    # allocate and fill blocks of many sizes, so that any tensor freed behind the
    # arguments' back is reused and overwritten before the launch
    gc.collect()
    junk = [torch.full((n,), 7, dtype=torch.uint8, device="cuda") for n in (1 << k for k in range(8, 24))]
    junk += [torch.full((n,), 7, dtype=torch.uint8, device="cuda") for n in (3 << k for k in range(6, 20))]
    torch.cuda.synchronize()
    return junk


def test_inline_tensors_stay_alive_through_a_decode_step():
    shape = synth.DecodeShape("lifetime-b2-h8kv2-d128-L900", 2, 8, 2, 128, 900)
    cfg = synth.make_decode_config(0, shape=shape, seed_index=11)
    B, Hq, d = cfg["q"].shape
    n_kv, cap = cfg["n_kv"], cfg["recent_k"].shape[2]
    # one free history slot per request for the step's demotion
    extra = (cfg["n_pages"] + np.arange(B)).astype(np.int32)[:, None]
    cfg = dict(cfg, block_table=np.concatenate([cfg["block_table"], extra], axis=1), n_pages=cfg["n_pages"] + B)
    hl = cfg["hist_len"]
    slot = (cfg["block_table"][np.arange(B), hl // PAGE] * PAGE + hl % PAGE).astype(np.int32)
    kc, vc, ks, vs = oracle_pools(cfg)
    ref_out = oracle.decode_attn_ref(cfg, kc, vc, ks, vs)
    ring = 5
    src = (np.arange(B) * n_kv * cap + ring).astype(np.int32)
    kc_ref, vc_ref, ks_ref, vs_ref = kc.copy(), vc.copy(), ks.copy(), vs.copy()
    dk_ref = oracle.quantize_pack_ref("k", cfg["recent_k"][:, :, ring, :], cfg["r_k"], cfg["tau_k"], slot,
                                      kc_ref, ks_ref)
    dv_ref = oracle.quantize_pack_ref("v", cfg["recent_v"][:, :, ring, :], cfg["r_v"], cfg["tau_v"], slot,
                                      vc_ref, vs_ref)

    # outputs and pools are kept here to read them back; everything else exists only in the args
    pools = [dev(p) for p in (kc, vc, ks, vs)]
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    args = hip.decode_args(q=dev(cfg["q"]), sink_k=dev(cfg["sink_k"]), sink_v=dev(cfg["sink_v"]),
                           recent_k=dev(cfg["recent_k"]), recent_v=dev(cfg["recent_v"]),
                           sink_len=dev(cfg["sink_len"]), recent_len=dev(cfg["recent_len"]),
                           hist_len=dev(cfg["hist_len"]), max_hist_len=int(hl.max()), k_codes=pools[0],
                           v_codes=pools[1], k_sz=pools[2], v_sz=pools[3], block_table=dev(cfg["block_table"]),
                           r_k=dev(cfg["r_k"]), r_v=dev(cfg["r_v"]), out=out,
                           workspace=torch.zeros(hip.oscar_decode_workspace_bytes(B, Hq, n_kv, d, int(hl.max())),
                                                 dtype=torch.uint8, device="cuda"),
                           sm_scale=float(cfg["sm_scale"]))
    common = dict(n_src=B * n_kv * cap, x_tok_stride=d, x_head_stride=cap * d)
    dk = hip.demote_args(x=dev(cfg["recent_k"]), rot=dev(cfg["r_k"]), clip=float(cfg["tau_k"]),
                         dst_slot=dev(slot), codes=pools[0], scale_zero=pools[2], src_idx=dev(src), **common)
    dv = hip.demote_args(x=dev(cfg["recent_v"]), rot=dev(cfg["r_v"]), clip=float(cfg["tau_v"]),
                         dst_slot=dev(slot), codes=pools[1], scale_zero=pools[3], src_idx=dev(src), **common)
    junk = _churn()
    hip.oscar_decode_step(args=args, demote_k=dk, demote_v=dv)
    torch.cuda.synchronize()
    del junk
    compare_out(host(out), ref_out, what="decode with inline tensors")
    compare_quant("k", host(pools[0]), host(pools[2], np.uint16), kc_ref, ks_ref, dk_ref, d)
    compare_quant("v", host(pools[1]), host(pools[3], np.uint16), vc_ref, vs_ref, dv_ref, d)

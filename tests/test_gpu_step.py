"""GPU parity of oscar_decode_step: the step's K and V demotions run in the
decode's last launch.  The decode must equal the oracle decode of the cache
as given (the demoted slots lie past hist_len), and the demoted slots must
equal the oracle quantiser's output for the demoted tokens, also in batches
whose merge and demotion blocks take more than one round of resident blocks."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_attn_amd as hip
import oracle
import synth
from gpu_util import CODEBOOK_FLAG, PAGE, compare_out, compare_quant, dev, host, oracle_pools

pytestmark = pytest.mark.gpu

SHAPES = [
    synth.DecodeShape("step-b1-h4kv2-d64-L1024", 1, 4, 2, 64, 1024),          # history ends on a page boundary
    synth.DecodeShape("step-b3-h16kv2-d128-L1000", 3, 16, 2, 128, 1000),       # partial last page, 3 requests
]


def _with_free_slots(cfg):
    """Append one page per request to the pool and the table so that slot
    hist_len of every request exists; return the widened config and the
    step's destination slots."""
    B = cfg["q"].shape[0]
    table = cfg["block_table"]
    extra = (cfg["n_pages"] + np.arange(B)).astype(np.int32)[:, None]
    cfg = dict(cfg, block_table=np.concatenate([table, extra], axis=1), n_pages=cfg["n_pages"] + B)
    hl = cfg["hist_len"]
    slot = cfg["block_table"][np.arange(B), hl // PAGE] * PAGE + hl % PAGE
    return cfg, slot.astype(np.int32)


def _pools_with_room(cfg):
    kc, vc, ks, vs = oracle_pools(cfg)
    return kc, vc, ks, vs


# large batches: 29 x 8 and 41 x 8 (request, KV head) units (the per-unit
# merge, 464 and 656 demotion blocks), and group size 16 (the per-head merge)
MANY = [
    synth.DecodeShape("step-b29-h32kv8-d128-L700", 29, 32, 8, 128, 700),
    synth.DecodeShape("step-b41-h32kv8-d128-L520", 41, 32, 8, 128, 520),
    synth.DecodeShape("step-b9-h128kv8-d128-L600", 9, 128, 8, 128, 600),
]


@pytest.mark.parametrize("groups", [0, 64, 32])
@pytest.mark.parametrize("codebook", ["uniform", "lloyd_max"])
@pytest.mark.parametrize("shape", SHAPES, ids=[s.name for s in SHAPES])
def test_decode_step_matches_separate_oracle_steps(shape, codebook, groups):
    _check_step(shape, codebook, groups)


@pytest.mark.parametrize("codebook,groups", [("uniform", 0), ("lloyd_max", 32)])
@pytest.mark.parametrize("shape", MANY, ids=[s.name for s in MANY])
def test_decode_step_large_batches(shape, codebook, groups):
    _check_step(shape, codebook, groups)


def _check_step(shape, codebook, groups):
    cfg, slot = _with_free_slots(synth.make_decode_config(0, shape=shape, seed_index=7))
    cfg["codebook"] = codebook
    cfg["group_channels"] = groups
    B, Hq, d = cfg["q"].shape
    n_kv, cap = cfg["n_kv"], cfg["recent_k"].shape[2]
    kc, vc, ks, vs = _pools_with_room(cfg)
    ref_out = oracle.decode_attn_ref(cfg, kc, vc, ks, vs)
    # the step demotes ring slot 3 of every request's recent window
    ring = 3
    src = (np.arange(B) * n_kv * cap + ring).astype(np.int32)
    kc_ref, vc_ref, ks_ref, vs_ref = kc.copy(), vc.copy(), ks.copy(), vs.copy()
    dk_ref = oracle.quantize_pack_ref("k", cfg["recent_k"][:, :, ring, :], cfg["r_k"], cfg["tau_k"], slot,
                                      kc_ref, ks_ref, codebook=codebook, group=groups or None)
    dv_ref = oracle.quantize_pack_ref("v", cfg["recent_v"][:, :, ring, :], cfg["r_v"], cfg["tau_v"], slot,
                                      vc_ref, vs_ref, codebook=codebook, group=groups or None)

    pools = [dev(p) for p in (kc, vc, ks, vs)]
    ws = torch.zeros(hip.oscar_decode_workspace_bytes(B, Hq, n_kv, d, int(cfg["hist_len"].max()), 64, cap),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    rk, rv, rec_k, rec_v = dev(cfg["r_k"]), dev(cfg["r_v"]), dev(cfg["recent_k"]), dev(cfg["recent_v"])
    src_t, slot_t = dev(src), dev(slot)
    # decode_args and demote_args keep raw pointers: every tensor stays referenced until the step ran
    t = {k: dev(cfg[k]) for k in ("q", "sink_k", "sink_v", "sink_len", "recent_len", "hist_len", "block_table")}
    args = hip.decode_args(q=t["q"], sink_k=t["sink_k"], sink_v=t["sink_v"], recent_k=rec_k, recent_v=rec_v,
                           sink_len=t["sink_len"], recent_len=t["recent_len"], hist_len=t["hist_len"],
                           max_hist_len=int(cfg["hist_len"].max()), k_codes=pools[0], v_codes=pools[1],
                           k_sz=pools[2], v_sz=pools[3], block_table=t["block_table"], r_k=rk, r_v=rv, out=out,
                           workspace=ws, sm_scale=float(cfg["sm_scale"]), codebook=CODEBOOK_FLAG[codebook],
                           group_channels=groups)
    common = dict(src_idx=src_t, n_src=B * n_kv * cap, x_tok_stride=d, x_head_stride=cap * d)
    dk = hip.demote_args(x=rec_k, rot=rk, clip=float(cfg["tau_k"]), dst_slot=slot_t, codes=pools[0],
                         scale_zero=pools[2], **common)
    dv = hip.demote_args(x=rec_v, rot=rv, clip=float(cfg["tau_v"]), dst_slot=slot_t, codes=pools[1],
                         scale_zero=pools[3], **common)
    hip.oscar_decode_step(args=args, demote_k=dk, demote_v=dv)
    torch.cuda.synchronize()
    compare_out(host(out), ref_out, what=f"step decode {shape.name}")
    compare_quant("k", host(pools[0]), host(pools[2], np.uint16), kc_ref, ks_ref, dk_ref, d, codebook=codebook)
    compare_quant("v", host(pools[1]), host(pools[3], np.uint16), vc_ref, vs_ref, dv_ref, d, codebook=codebook)


def test_decode_step_without_demotion_equals_decode():
    cfg = synth.make_decode_config(0)
    B, Hq, d = cfg["q"].shape
    pools = [dev(p) for p in oracle_pools(cfg)]
    cap = cfg["recent_k"].shape[2]
    ws = torch.zeros(hip.oscar_decode_workspace_bytes(B, Hq, cfg["n_kv"], d, int(cfg["hist_len"].max()), 64, cap),
                     dtype=torch.uint8, device="cuda")
    outs = []
    # decode_args keeps raw pointers: the tensors stay referenced until the calls ran
    t = {k: dev(cfg[k]) for k in ("q", "sink_k", "sink_v", "recent_k", "recent_v", "sink_len", "recent_len",
                                  "hist_len", "block_table", "r_k", "r_v")}
    for use_step in (False, True):
        out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
        args = hip.decode_args(q=t["q"], sink_k=t["sink_k"], sink_v=t["sink_v"], recent_k=t["recent_k"],
                               recent_v=t["recent_v"], sink_len=t["sink_len"], recent_len=t["recent_len"],
                               hist_len=t["hist_len"], max_hist_len=int(cfg["hist_len"].max()),
                               k_codes=pools[0], v_codes=pools[1], k_sz=pools[2], v_sz=pools[3],
                               block_table=t["block_table"], r_k=t["r_k"], r_v=t["r_v"], out=out, workspace=ws,
                               sm_scale=float(cfg["sm_scale"]))
        if use_step:
            hip.oscar_decode_step(args=args)
        else:
            hip.oscar_decode_attn(args=args)
        torch.cuda.synchronize()
        outs.append(host(out))
    assert np.array_equal(outs[0], outs[1])


def test_decode_step_with_no_requests_only_demotes():
    """Batch 0: the q-rotation and scan launches have no blocks, and the merge
    launch holds only the demotion blocks.  The pools must equal the oracle
    quantiser's output for the demoted tokens."""
    cfg = synth.make_decode_config(0)
    n_kv, d, P = cfg["n_kv"], cfg["head_dim"], cfg["n_pages"]
    Hq = cfg["q"].shape[1]
    n_tok = 7
    pick = np.array([0, 5, 64, 65, 130, 300, 703], dtype=np.int32)[:n_tok]
    slot = cfg["hist_slot"][pick].astype(np.int32)
    kc_ref = np.zeros((P, n_kv, PAGE * d // 4), np.uint8)
    vc_ref = np.zeros_like(kc_ref)
    ks_ref = np.zeros((P, n_kv, PAGE, 2), np.uint16)
    vs_ref = np.zeros_like(ks_ref)
    dk_ref = oracle.quantize_pack_ref("k", cfg["hist_k"][pick], cfg["r_k"], cfg["tau_k"], slot, kc_ref, ks_ref)
    dv_ref = oracle.quantize_pack_ref("v", cfg["hist_v"][pick], cfg["r_v"], cfg["tau_v"], slot, vc_ref, vs_ref)

    pools = [dev(np.zeros_like(a)) for a in (kc_ref, vc_ref, ks_ref, vs_ref)]
    rk, rv = dev(cfg["r_k"]), dev(cfg["r_v"])
    e16 = lambda *s: torch.zeros(s, dtype=torch.int16, device="cuda")
    e32 = lambda *s: torch.zeros(s, dtype=torch.int32, device="cuda")
    out = torch.zeros((0, Hq, d), dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(1, hip.oscar_decode_workspace_bytes(0, Hq, n_kv, d, 0, 64, 256)), dtype=torch.uint8,
                     device="cuda")
    args = hip.decode_args(q=e16(0, Hq, d), sink_k=e16(0, n_kv, 64, d), sink_v=e16(0, n_kv, 64, d),
                           recent_k=e16(0, n_kv, 256, d), recent_v=e16(0, n_kv, 256, d), sink_len=e32(0),
                           recent_len=e32(0), hist_len=e32(0), max_hist_len=0, k_codes=pools[0],
                           v_codes=pools[1], k_sz=pools[2], v_sz=pools[3], block_table=e32(0, 1), r_k=rk,
                           r_v=rv, out=out, workspace=ws)
    # demote_args keeps raw pointers: the tensors must outlive the call
    xk, xv, slot_t = dev(cfg["hist_k"][pick]), dev(cfg["hist_v"][pick]), dev(slot)
    dk = hip.demote_args(x=xk, rot=rk, clip=float(cfg["tau_k"]), dst_slot=slot_t, codes=pools[0],
                         scale_zero=pools[2])
    dv = hip.demote_args(x=xv, rot=rv, clip=float(cfg["tau_v"]), dst_slot=slot_t, codes=pools[1],
                         scale_zero=pools[3])
    hip.oscar_decode_step(args=args, demote_k=dk, demote_v=dv)
    torch.cuda.synchronize()
    compare_quant("k", host(pools[0]), host(pools[2], np.uint16), kc_ref, ks_ref, dk_ref, d)
    compare_quant("v", host(pools[1]), host(pools[3], np.uint16), vc_ref, vs_ref, dv_ref, d)

#!/usr/bin/env python3
"""Decode-step benchmark of INT2 three-segment decode attention on one MI355X.

Workload (default): one Qwen3-32B-shaped decode layer, batch 1, 64 query heads,
8 KV heads, head_dim 128, 100 000-token context = 64 BF16 sink + 99 680 INT2
history (1558 pages of 64 tokens, random physical order) + 256 BF16 recent.
Inputs are seeded synthetic data (bf16 N(0,1) K/V with 3 outlier channels per
head scaled x20; rotations from a random SPD eigenbasis x Hadamard x
bit-reversal; 99.9th-percentile clip thresholds).  The history pages are made
by the library's own demotion kernel (bulk demotion of the history).

One step = the whole hot path for one new token per request: demote the
oldest recent token of K and V into INT2 history (rotate, clip, quantise,
pack), then decode attention (q rotation, INT2 history scan + BF16 windows,
merge and output rotation).  Every step reads a different replica of the
cache; the replicas together exceed 1 GiB, so the 256 MB Infinity Cache
cannot serve repeated reads.  Steps are replayed from HIP graphs; W warmup
steps run first (eagerly), every captured graph is replayed once untimed (its
first launch uploads it to the GPU), then exactly K steps are timed between
two synchronisations.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MALL_BYTES = 256 << 20
WORKLOADS = {"qwen3-32b-100k": 3, "qwen3-8b-32k": 1, "qwen3-8b-b28-100k": 4}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3-32b-100k", choices=sorted(WORKLOADS))
    ap.add_argument("--replicas", type=int, default=0, help="cache replicas (0: enough for >= 1 GiB)")
    ap.add_argument("--codebook", default="uniform", choices=("uniform", "lloyd-max"),
                    help="INT2 codebook the history is demoted with and read by (oscar.h)")
    ap.add_argument("--groups", type=int, default=0, choices=(0, 64, 32),
                    help="channels per (scale, zero) group: 0 = the whole head, 64 or 32 = sub-head groups")
    ap.add_argument("--prefix-cascade", action="store_true",
                    help="read the shared prefix in cascade blocks where oscar.h allows it (prefix_cascade = 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only the selected workload (no 28-request and bulk-demotion sub-records)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (torch.neg) 3 times: the known-size "
                         "kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


class Timer:
    """HIP-graph capture and event timing on the current torch stream (the
    stream the library's launches go to)."""

    def __init__(self, torch):
        self.torch = torch

    def capture(self, fn, idxs):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=s):
            for i in idxs:
                fn(i)
        torch.cuda.synchronize()
        # one untimed replay: a graph's first launch also uploads it, a cost
        # that would otherwise land in the timed region
        g.replay()
        torch.cuda.synchronize()
        return g

    def timed_fn(self, fn):
        torch = self.torch
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3, time.perf_counter() - w0

    def timed(self, graph_all, graph_rem, n_full):
        def run():
            for _ in range(n_full):
                graph_all.replay()
            if graph_rem is not None:
                graph_rem.replay()
        return self.timed_fn(run)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this decode path runs on one GPU only; there is no multi-GPU mode "
              "(how it would shard is described in DESIGN.md). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_rotated_kv_attn_amd as hip

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    hip.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tm = Timer(torch)

    head = decode_workload(args.workload, args, args.steps, args.warmup, not args.no_bf16, tm)
    cfg, rec = head.pop("cfg"), head
    B = cfg["batch"]
    result = {
        "metric": "decode-attn tokens/s + achieved HBM GB/s (% peak) at 100k ctx, INT2 vs BF16",
        "value": B / (rec["ms_per_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": hip.COMPUTE_DTYPE, "data": "synthetic",
        "config": rec["config"],
        "roofline": rec["roofline"],
        "kv_tokens_per_s": rec["kv_tokens_per_s"],
        "int2_decode_us": rec["int2_decode_us"],
        "decode_GBps": rec["decode_GBps"],
    }
    for k in ("bf16_comparator", "speedup_int2_vs_bf16_decode"):
        if k in rec:
            result[k] = rec[k]

    # ---- what this part's HBM sustains for a plain stream: a 1 GiB device copy
    # (512 MiB read + 512 MiB written per torch.neg), beside the spec peak of the roofline
    n = (512 << 20) // 4
    src = torch.randn(n, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)
    reps_copy = 10
    copy_sec, _ = tm.timed_fn(lambda: [torch.neg(src, out=dst) for _ in range(reps_copy)])
    copy_gbs = 2 * n * 4 * reps_copy / copy_sec / 1e9
    achieved = rec["roofline"]["achieved"]
    result["hbm_copy_probe"] = {"GBps": copy_gbs, "bytes_per_copy": 2 * n * 4, "kernel": "torch.neg",
                                "scan_frac_of_copy": achieved / copy_gbs}
    log(f"copy probe: {copy_gbs:.0f} GB/s; the scan reaches {achieved / copy_gbs:.1%} of it")
    del src, dst

    # ---- the other workloads, each in its own sub-record of the same line
    if not args.no_extra:
        extra = {}
        if args.workload != "qwen3-8b-b28-100k":
            torch.cuda.empty_cache()
            sub = decode_workload("qwen3-8b-b28-100k", args, min(args.steps, 40), min(args.warmup, 5),
                                  not args.no_bf16, tm)
            sub.pop("cfg")
            sub["tokens_per_s"] = sub["config"]["batch"] / (sub["ms_per_step"] * 1e-3)
            extra["qwen3-8b-b28-100k"] = sub
        torch.cuda.empty_cache()
        extra["bulk-demotion"] = bulk_demotion(args, tm)
        result["workloads"] = extra

    # ---- CPU oracle on a bounded sample (reported baseline, not a target)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds, "lloyd_max" if args.codebook == "lloyd-max"
                                              else "uniform", args.groups or None)
    print(json.dumps(result), flush=True)


def decode_workload(name, args, K, warmup, with_bf16, tm):
    """Time the decode step, the scan and the three-launch decode on one decode
    workload; returns the record fields (and the generated inputs as "cfg")."""
    import numpy as np
    import torch

    import bit_rotated_kv_attn_amd as hip
    import synth

    dev = torch.device("cuda:0")
    cfg_index = WORKLOADS[name]
    lm = args.codebook == "lloyd-max"
    cb_flag = hip.CODEBOOK_LLOYD_MAX if lm else hip.CODEBOOK_UNIFORM
    grouped = args.groups > 0
    q_flags = cb_flag | {0: 0, 64: hip.GROUPS_64, 32: hip.GROUPS_32}[args.groups]
    shape = synth.DECODE_SHAPES[cfg_index]
    t0 = time.time()
    cfg = ensure_free_slot(synth.make_decode_config(cfg_index))
    log(f"generated {shape.name} in {time.time() - t0:.1f}s")
    B, Hq, d = cfg["q"].shape
    n_kv, P = cfg["n_kv"], cfg["n_pages"]
    hl = int(cfg["hist_len"].max())

    def t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    # ---- shared inputs
    q, r_k, r_v = t(cfg["q"]), t(cfg["r_k"]), t(cfg["r_v"])
    table = t(cfg["block_table"])
    sink_len, recent_len, hist_len = t(cfg["sink_len"]), t(cfg["recent_len"]), t(cfg["hist_len"])
    hist_k, hist_v, hist_slot = t(cfg["hist_k"]), t(cfg["hist_v"]), t(cfg["hist_slot"])
    # the token each step demotes: ring slot 0 of every request's recent window goes to
    # the next free history slot (beyond hist_len, so this step's decode does not read it)
    nxt = cfg["hist_len"]
    step_slot = t((cfg["block_table"][np.arange(B), nxt // 64] * 64 + nxt % 64).astype(np.int32))
    cap = cfg["recent_k"].shape[2]
    step_src = t((np.arange(B) * n_kv * cap).astype(np.int32))

    # algorithmic bytes: every history token of a physical page once (a page
    # shared by several requests' tables needs reading only once), the BF16
    # windows and the block-table entries
    ng = hip.groups_per_head(d, args.groups)   # (scale, zero) pairs per token and head
    hist_bytes = unique_tokens(cfg["block_table"], cfg["hist_len"]) * n_kv * (2 * d // 4 + 2 * 4 * ng)
    win_bytes = int((cfg["sink_len"] + cfg["recent_len"]).sum()) * n_kv * 4 * d
    table_bytes = int(sum(-(-int(h) // 64) for h in cfg["hist_len"])) * 4
    scan_bytes = hist_bytes + win_bytes + table_bytes
    # the whole decode also reads q, R_K and R_V, and writes the output
    decode_bytes = scan_bytes + q.numel() * 2 + 2 * r_k.numel() * 4 + B * Hq * d * 4
    per_replica = (P * n_kv * 64 * (2 * d // 4 + 8 * ng) + 2 * cfg["sink_k"].nbytes + 2 * cfg["recent_k"].nbytes)
    R = args.replicas or max(2, math.ceil((1 << 30) / per_replica))
    log(f"replicas: {R} x {per_replica / 1e6:.1f} MB = {R * per_replica / 2**30:.2f} GiB "
        f"(MALL {MALL_BYTES >> 20} MiB)")

    # ---- replicas: page pools demoted by the library, private BF16 windows
    reps = []
    t0 = time.time()
    for r in range(R):
        kc = torch.zeros((P, n_kv, 64 * d // 4), dtype=torch.uint8, device=dev)
        vc = torch.zeros_like(kc)
        ks = torch.zeros((P, n_kv, 64 * ng, 2), dtype=torch.int16, device=dev)
        vs = torch.zeros_like(ks)
        hip.oscar_quantize_pack(hip.KIND_K | q_flags, hist_k, r_k, float(cfg["tau_k"]), hist_slot, kc, ks)
        hip.oscar_quantize_pack(hip.KIND_V | q_flags, hist_v, r_v, float(cfg["tau_v"]), hist_slot, vc, vs)
        rep = dict(k_codes=kc, v_codes=vc, k_sz=ks, v_sz=vs, sink_k=t(cfg["sink_k"]), sink_v=t(cfg["sink_v"]),
                   recent_k=t(cfg["recent_k"]), recent_v=t(cfg["recent_v"]),
                   out=torch.empty((B, Hq, d), dtype=torch.float32, device=dev))
        reps.append(rep)
    torch.cuda.synchronize()
    log(f"demoted the history into {R} replicas in {time.time() - t0:.1f}s")
    del hist_k, hist_v
    # a prefix-cache hit: the leading history pages every request holds at the same ids
    shared = min(shape.shared_hist_pages, shape.hist_pages)
    ws_bytes = hip.oscar_decode_workspace_bytes(B, Hq, n_kv, d, hl, cfg["sink_k"].shape[2], cap)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    dargs = [hip.decode_args(q=q, sink_k=rp["sink_k"], sink_v=rp["sink_v"], recent_k=rp["recent_k"],
                             recent_v=rp["recent_v"], sink_len=sink_len, recent_len=recent_len,
                             hist_len=hist_len, max_hist_len=hl, k_codes=rp["k_codes"], v_codes=rp["v_codes"],
                             k_sz=rp["k_sz"], v_sz=rp["v_sz"], block_table=table, r_k=r_k, r_v=r_v,
                             out=rp["out"], workspace=ws, sm_scale=float(cfg["sm_scale"]),
                             shared_pages=shared, codebook=cb_flag, group_channels=args.groups,
                             prefix_cascade=args.prefix_cascade) for rp in reps]

    # the step demotes ring slot 0 of every request's recent window (K and V) in
    # the decode's last launch
    dem = []
    for r in range(R):
        rp = reps[r]
        common = dict(src_idx=step_src, n_src=B * n_kv * cap, x_tok_stride=d, x_head_stride=cap * d)
        dem.append((hip.demote_args(x=rp["recent_k"], rot=r_k, clip=float(cfg["tau_k"]), dst_slot=step_slot,
                                    codes=rp["k_codes"], scale_zero=rp["k_sz"], **common),
                    hip.demote_args(x=rp["recent_v"], rot=r_v, clip=float(cfg["tau_v"]), dst_slot=step_slot,
                                    codes=rp["v_codes"], scale_zero=rp["v_sz"], **common)))

    def step(r):
        hip.oscar_decode_step(args=dargs[r], demote_k=dem[r][0], demote_v=dem[r][1])

    # ---- warmup (eager), then graphs
    log(f"{name}: warmup {warmup} steps")
    for i in range(warmup):
        step(i % R)
    torch.cuda.synchronize()
    g_all = tm.capture(step, range(R))
    g_rem = tm.capture(step, range(K % R)) if K % R else None
    log(f"{name}: timing {K} steps")
    sec, wall = tm.timed(g_all, g_rem, K // R)
    ms_per_step = sec * 1e3 / K
    log(f"step: {ms_per_step * 1e3:.2f} us (host wall clock {wall * 1e6 / K:.2f} us per step)")

    if args.copy_probe:
        n = (256 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"copy probe: 3 x torch.neg over {n * 4} bytes read + {n * 4} bytes written")
        del src, dst

    # ---- dominant kernel: the scan, R launches back to back per graph replay
    g_scan = tm.capture(lambda r: hip.oscar_decode_scan(args=dargs[r]), range(R))
    n_scan = max(1, K // R)
    scan_sec, _ = tm.timed(g_scan, None, n_scan)
    scan_us = scan_sec * 1e6 / (n_scan * R)
    g_dec = tm.capture(lambda r: hip.oscar_decode_attn(args=dargs[r]), range(R))
    dec_sec, _ = tm.timed(g_dec, None, n_scan)
    dec_us = dec_sec * 1e6 / (n_scan * R)
    achieved = scan_bytes / (scan_us * 1e-6) / 1e9
    dec_gbs = decode_bytes / (dec_us * 1e-6) / 1e9
    log(f"scan kernel: {scan_us:.2f} us, {achieved:.0f} GB/s algorithmic ({achieved / HBM_PEAK_GBS:.1%} of peak); "
        f"decode (3 kernels): {dec_us:.2f} us, {dec_gbs:.0f} GB/s ({dec_gbs / HBM_PEAK_GBS:.1%})")

    rec = {
        "cfg": cfg, "ms_per_step": ms_per_step, "step_us": ms_per_step * 1e3,
        "config": {"workload": shape.name, "batch": B, "context": shape.context, "n_q_heads": Hq,
                   "n_kv_heads": n_kv, "head_dim": d, "sink": int(cfg["sink_len"][0]),
                   "history": hl, "recent": int(cfg["recent_len"][0]), "page_tokens": 64,
                   "cache_replicas": R, "shared_prefix_pages": shared, "codebook": args.codebook,
                   "group_channels": args.groups, "prefix_cascade": bool(args.prefix_cascade),
                   "step": "oscar_decode_step: demote K,V of 1 token/request + decode attention"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(name + ("-lloyd-max" if lm else "") + (f"-groups{args.groups}" if grouped else "")
                                                 + ("-cascade" if args.prefix_cascade else "")),
                     "kernel": "decode_main_kernel (oscar_decode_scan)", "kernel_us": scan_us,
                     "bytes_per_launch": scan_bytes},
        "kv_tokens_per_s": float(cfg["hist_len"].sum() + cfg["sink_len"].sum() + cfg["recent_len"].sum())
                           / (ms_per_step * 1e-3),
        "int2_decode_us": dec_us,
        # the whole decode (q rotation, scan, merge): its bytes over the three launches' time
        "decode_GBps": dec_gbs, "decode_frac_of_peak": dec_gbs / HBM_PEAK_GBS, "decode_bytes": decode_bytes,
    }
    del g_all, g_rem, g_scan, g_dec, dargs, dem, reps, ws

    # ---- BF16 comparator (same layer, whole context in BF16 pages)
    if with_bf16:
        t0 = time.time()
        bf = synth.bf16_context_pages(cfg)
        log(f"bf16 pages of {name} in {time.time() - t0:.1f}s")
        bf_bytes = bf["k_pages"].nbytes + bf["v_pages"].nbytes
        Rb = max(2, math.ceil((1 << 30) / bf_bytes))
        kp0, vp0 = t(bf["k_pages"]), t(bf["v_pages"])
        bt, ctx = t(bf["block_table"]), t(bf["ctx_len"])
        ctx_max = int(bf["ctx_len"].max())
        bws = torch.empty(hip.oscar_decode_bf16_workspace_bytes(B, Hq, n_kv, d, ctx_max), dtype=torch.uint8,
                          device=dev)
        bre = [(kp0, vp0)] + [(kp0.clone(), vp0.clone()) for _ in range(Rb - 1)]
        bout = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)

        def bf16_step(r):
            hip.oscar_decode_attn_bf16(q=q, k_pages=bre[r][0], v_pages=bre[r][1], block_table=bt, ctx_len=ctx,
                                       max_ctx_len=ctx_max, out=bout, workspace=bws,
                                       sm_scale=float(cfg["sm_scale"]))
        for r in range(Rb):
            bf16_step(r)
        g_bf = tm.capture(bf16_step, range(Rb))
        nb = max(1, K // Rb)
        bf_sec, _ = tm.timed(g_bf, None, nb)
        bf_us = bf_sec * 1e6 / (nb * Rb)
        bf_need = unique_tokens(bf["block_table"], bf["ctx_len"]) * n_kv * 4 * d
        rec["bf16_comparator"] = {"decode_us": bf_us, "tokens_per_s": B / (bf_us * 1e-6),
                                  "algorithmic_GBps": bf_need / (bf_us * 1e-6) / 1e9, "replicas": Rb,
                                  "kernel": "oscar_decode_attn_bf16"}
        rec["speedup_int2_vs_bf16_decode"] = bf_us / dec_us
        log(f"bf16 comparator: {bf_us:.2f} us/decode; INT2 decode speedup {bf_us / dec_us:.2f}x")
        del bre, kp0, vp0, g_bf
    return rec


def bulk_demotion(args, tm):
    """Bulk demotion of 131072 tokens x 8 KV heads x 128 for K and for V, in
    one oscar_quantize_pack launch per tensor, timed over repeated launches
    (K, V, K, V, ...) between HIP events on the launching stream.  Algorithmic
    bytes per tensor: read the bf16 tokens, R and the slots; write the codes
    and the (scale, zero) pairs.  Flops: the rotation x R, 2 d^2 per token
    and head."""
    import numpy as np
    import torch

    import bit_rotated_kv_attn_amd as hip
    import synth

    dev = torch.device("cuda:0")
    t0 = time.time()
    cfg = synth.make_bulk_demotion_config()
    log(f"generated {cfg['name']} in {time.time() - t0:.1f}s")
    n_tok, n_kv, d, P = cfg["x_k"].shape[0], cfg["n_kv"], cfg["head_dim"], cfg["n_pages"]

    def t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    x = {k: t(cfg["x_" + k]) for k in ("k", "v")}
    rot = {k: t(cfg["r_" + k]) for k in ("k", "v")}
    slot = t(cfg["dst_slot"])
    ng = hip.groups_per_head(d, args.groups)   # (scale, zero) pairs per token and head
    pools = {k: (torch.zeros((P, n_kv, 64 * d // 4), dtype=torch.uint8, device=dev),
                 torch.zeros((P, n_kv, 64 * ng, 2), dtype=torch.int16, device=dev)) for k in ("k", "v")}
    gflag = {0: 0, 64: hip.GROUPS_64, 32: hip.GROUPS_32}[args.groups]
    kinds = {"k": hip.KIND_K | gflag, "v": hip.KIND_V | gflag}

    def launch(i):
        k = "kv"[i % 2]
        hip.oscar_quantize_pack(kinds[k], x[k], rot[k], float(cfg["tau_" + k]), slot, *pools[k])

    for i in range(4):
        launch(i)
    torch.cuda.synchronize()
    n = 2 * max(4, min(args.steps, 20))
    g = tm.capture(launch, range(n))
    sec, _ = tm.timed(g, None, 1)
    us = sec * 1e6 / n
    bytes_per = n_tok * n_kv * (2 * d + d // 4 + 4 * ng) + rot["k"].numel() * 4 + slot.numel() * 4
    flops_per = 2.0 * d * d * n_kv * n_tok
    gbs = bytes_per / (us * 1e-6) / 1e9
    tfs = flops_per / (us * 1e-6) / 1e12
    peak = hip.DEMOTION_MATMUL_PEAK_TFLOPS
    log(f"bulk demotion: {us:.1f} us per tensor, {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM peak), "
        f"{tfs:.1f} TFLOP/s ({tfs / peak:.1%} of the {hip.DEMOTION_MATMUL_DTYPE} matrix peak)")
    del g, x, pools
    return {"config": {"workload": cfg["name"], "tokens": n_tok, "n_kv_heads": n_kv, "head_dim": d,
                       "group_channels": args.groups, "tensors": "K and V, one oscar_quantize_pack call each",
                       "kernel": "quantize_mfma_kernel (certified fast pass, then each block's marked tokens exactly)"},
            "us_per_tensor": us, "tokens_per_s": n_tok / (2 * us * 1e-6),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": bytes_per, "kernel_us": us},
            "contraction": {"dtype": hip.DEMOTION_MATMUL_DTYPE, "achieved": tfs, "peak": peak, "unit": "TFLOP/s",
                            "frac": tfs / peak, "flops_per_launch": flops_per}}


SCAN_SOURCES = ("bit_rotated_kv_attn_amd/csrc/decode.hip", "bit_rotated_kv_attn_amd/csrc/common.hpp")


def scan_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in SCAN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per scan launch from the committed counter summary of this
    workload (FETCH_SIZE + WRITE_SIZE, each scaled by the copy-kernel
    calibration), or None when the summary is missing or was taken on other
    kernel sources than the ones built now."""
    path = os.path.join(ROOT, "profiles", f"traffic_decode_main_kernel_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256_16") != scan_source_hash():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def unique_tokens(table, lens) -> int:
    """Tokens per KV head counted once per physical page slot: the valid
    tokens of each page are the most that any request holding it uses."""
    used = {}
    for b, h in enumerate(lens):
        h = int(h)
        for i in range(-(-h // 64)):
            pid = int(table[b, i])
            used[pid] = max(used.get(pid, 0), min(64, h - 64 * i))
    return sum(used.values())


def ensure_free_slot(cfg):
    """Give every request a free history slot for the token a step demotes:
    when a request's history ends on a page boundary, append one page to the
    pool and to that request's block-table row."""
    import numpy as np
    nxt = cfg["hist_len"]
    table = cfg["block_table"]
    need = nxt // 64 >= table.shape[1]
    if not need.any():
        return cfg
    extra = np.full((table.shape[0], 1), -1, np.int32)
    extra[need, 0] = cfg["n_pages"] + np.arange(int(need.sum()))
    cfg = dict(cfg)
    cfg["block_table"] = np.concatenate([table, extra], axis=1)
    cfg["n_pages"] = cfg["n_pages"] + int(need.sum())
    return cfg


def cpu_baseline(cfg, budget_s: float, codebook: str = "uniform", group=None):
    """Time the oracle (as it stands) on whole KV heads of the same workload:
    one step's demotion of the new token plus decode attention for the G
    query heads of a KV head over the full context.  KV heads are added until
    the budget is spent; the per-step time is scaled to all KV heads."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = 1
    B, Hq, d = cfg["q"].shape
    n_kv, P = cfg["n_kv"], cfg["n_pages"]
    G = Hq // n_kv
    cfg = ensure_free_slot(cfg)
    P = cfg["n_pages"]
    spent, done = 0.0, 0
    setup = {}
    g = 0
    while spent < budget_s or done == 0:
        if g not in setup:
            sub = dict(cfg)
            sub.update(q=cfg["q"][:, g * G:(g + 1) * G], sink_k=cfg["sink_k"][:, g:g + 1],
                       sink_v=cfg["sink_v"][:, g:g + 1], recent_k=cfg["recent_k"][:, g:g + 1],
                       recent_v=cfg["recent_v"][:, g:g + 1], r_k=cfg["r_k"][g:g + 1], r_v=cfg["r_v"][g:g + 1])
            kc = np.zeros((P, 1, 64 * d // 4), np.uint8)
            vc = np.zeros_like(kc)
            ks = np.zeros((P, 1, 64 * (d // group if group else 1), 2), np.uint16)
            vs = np.zeros_like(ks)
            oracle.quantize_pack_ref("k", cfg["hist_k"][:, g:g + 1], sub["r_k"], cfg["tau_k"], cfg["hist_slot"], kc, ks,
                                     codebook=codebook, group=group)
            oracle.quantize_pack_ref("v", cfg["hist_v"][:, g:g + 1], sub["r_v"], cfg["tau_v"], cfg["hist_slot"], vc, vs,
                                     codebook=codebook, group=group)
            sub["codebook"] = codebook
            setup[g] = (sub, kc, vc, ks, vs)
        sub, kc, vc, ks, vs = setup[g]
        nxt = cfg["hist_len"]
        slot = (cfg["block_table"][np.arange(B), nxt // 64] * 64 + nxt % 64).astype(np.int32)
        w0 = time.perf_counter()
        oracle.quantize_pack_ref("k", sub["recent_k"][:, :, 0, :], sub["r_k"], cfg["tau_k"], slot, kc.copy(), ks.copy(),
                                 codebook=codebook, group=group)
        oracle.quantize_pack_ref("v", sub["recent_v"][:, :, 0, :], sub["r_v"], cfg["tau_v"], slot, vc.copy(), vs.copy(),
                                 codebook=codebook, group=group)
        oracle.decode_attn_ref(sub, kc, vc, ks, vs)
        spent += time.perf_counter() - w0
        done += 1
        log(f"cpu oracle: KV head {g} done ({done} head-steps, {spent:.1f}s)")
        g = (g + 1) % n_kv
    step_s = spent / done * n_kv
    return {"value": B / step_s, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} KV-head steps of the same layer ({G} query heads each over the full "
                      f"{cfg['shape'].context}-token context: demotion of the step's token + decode attention); "
                      f"per-step time = mean per KV head x {n_kv} KV heads",
            "seconds_measured": spent, "step_seconds": step_s}


if __name__ == "__main__":
    main()

"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C ABI binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import bit_rotated_kv_attn_amd as hip
import oracle

PAGE = 64
# tolerances fixed for the decode output (max-abs, relative L2 over the tensor)
MAX_ABS = 2e-3
REL_L2 = 1e-3
# codes may differ from the oracle only when the rotated value sits within this
# relative distance of a bin edge
BIN_EDGE_REL = 1e-5


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t: torch.Tensor, np_dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(np_dtype) if np_dtype is not None else a


def empty_pools(n_pages: int, n_kv: int, d: int, device="cuda", ng: int = 1):
    codes = torch.zeros((n_pages, n_kv, PAGE * d // 4), dtype=torch.uint8, device=device)
    sz = torch.zeros((n_pages, n_kv, PAGE * ng, 2), dtype=torch.int16, device=device)
    return codes, sz


# codebook name (oracle, cfg["codebook"]) -> the C ABI flag
CODEBOOK_FLAG = {"uniform": hip.CODEBOOK_UNIFORM, "lloyd_max": hip.CODEBOOK_LLOYD_MAX}


def oracle_pools(cfg: dict):
    """K/V pools of a decode config filled by the oracle quantiser (with the
    config's codebook, uniform by default, and its group_channels, 0 = whole
    head by default)."""
    cb = cfg.get("codebook", "uniform")
    d, nkv, P = cfg["head_dim"], cfg["n_kv"], cfg["n_pages"]
    group = cfg.get("group_channels", 0) or d
    kc = np.zeros((P, nkv, PAGE * d // 4), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.zeros((P, nkv, PAGE * (d // group), 2), np.uint16)
    vs = np.zeros_like(ks)
    oracle.quantize_pack_ref("k", cfg["hist_k"], cfg["r_k"], cfg["tau_k"], cfg["hist_slot"], kc, ks, codebook=cb,
                             group=group)
    oracle.quantize_pack_ref("v", cfg["hist_v"], cfg["r_v"], cfg["tau_v"], cfg["hist_slot"], vc, vs, codebook=cb,
                             group=group)
    return kc, vc, ks, vs


def gpu_decode(cfg: dict, pools, *, block_table=None, hist_len=None, sink_len=None, recent_len=None,
               max_hist_len=None, reps: int = 1, shared_pages: int = 0, prefix_cascade: bool = False) -> np.ndarray:
    kc, vc, ks, vs = (p if isinstance(p, torch.Tensor) else dev(p) for p in pools)
    q = dev(cfg["q"])
    B, Hq, d = cfg["q"].shape
    table = cfg["block_table"] if block_table is None else block_table
    hl = cfg["hist_len"] if hist_len is None else hist_len
    mh = int(np.max(hl)) if max_hist_len is None else max_hist_len
    ws_bytes = hip.oscar_decode_workspace_bytes(B, Hq, cfg["r_k"].shape[0], d, mh,
                                                cfg["sink_k"].shape[2], cfg["recent_k"].shape[2])
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    args = dict(q=q, sink_k=dev(cfg["sink_k"]), sink_v=dev(cfg["sink_v"]), recent_k=dev(cfg["recent_k"]),
                recent_v=dev(cfg["recent_v"]),
                sink_len=dev(cfg["sink_len"] if sink_len is None else sink_len),
                recent_len=dev(cfg["recent_len"] if recent_len is None else recent_len),
                hist_len=dev(hl), max_hist_len=mh, k_codes=kc, v_codes=vc, k_sz=ks, v_sz=vs,
                block_table=dev(table), r_k=dev(cfg["r_k"]), r_v=dev(cfg["r_v"]), out=out, workspace=ws,
                sm_scale=float(cfg["sm_scale"]), shared_pages=shared_pages,
                codebook=CODEBOOK_FLAG[cfg.get("codebook", "uniform")],
                group_channels=int(cfg.get("group_channels", 0)), prefix_cascade=prefix_cascade)
    for _ in range(reps):
        hip.oscar_decode_attn(**args)
    torch.cuda.synchronize()
    return host(out)


def gpu_quantize(kind: str, x: np.ndarray, rot: np.ndarray, clip, dst_slot: np.ndarray, n_pages: int,
                 src_idx=None, pools=None, codebook: str = "uniform", group_channels: int = 0):
    """Demote on the GPU with the given codebook and group size (0: the whole
    head; 64 or 32 channels) into fresh pools (or ``pools``)."""
    n_kv, d = rot.shape[0], rot.shape[-1]
    ng = hip.groups_per_head(d, group_channels)
    codes, sz = pools if pools is not None else empty_pools(n_pages, n_kv, d, ng=ng)
    flags = CODEBOOK_FLAG[codebook] | {0: 0, 64: hip.GROUPS_64, 32: hip.GROUPS_32}[group_channels]
    hip.oscar_quantize_pack((hip.KIND_K if kind == "k" else hip.KIND_V) | flags, dev(x), dev(rot),
                            float(clip),
                            dev(dst_slot.astype(np.int32)), codes, sz,
                            src_idx=None if src_idx is None else dev(src_idx.astype(np.int32)))
    torch.cuda.synchronize()
    return host(codes), host(sz, np.uint16)


def compare_out(got: np.ndarray, ref: np.ndarray, max_abs=MAX_ABS, rel_l2=REL_L2, what=""):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    ma = err.max() if err.size else 0.0
    rl = np.linalg.norm(err) / max(np.linalg.norm(ref.astype(np.float64)), 1e-30)
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max-abs {ma:.3e} (<= {max_abs}), rel-L2 {rl:.3e} (<= {rel_l2})"
    return ma, rl


def compare_quant(kind: str, gpu_codes, gpu_sz, ref_codes, ref_sz, diag, d: int, exact: bool = False,
                  codebook: str = "uniform"):
    """Quantiser parity: scale/zero bit-exact; code bytes bit-exact except
    codes that differ by one level where the oracle's rotated value lies
    within BIN_EDGE_REL (relative) of the bin edge between them.  Bytes and
    scale/zero outside the written slots must match too (both start zeroed)."""
    assert np.array_equal(gpu_sz, ref_sz), "scale/zero differ"
    if np.array_equal(gpu_codes, ref_codes):
        return 0
    assert not exact, "codes differ where bit-exact results are required"
    slots = diag["slot"]
    pages, offs = slots // PAGE, slots % PAGE
    pos = oracle.k_byte_offsets(offs, d) if kind == "k" else oracle.v_byte_offsets(offs, d)
    n_kv = gpu_codes.shape[1]
    mask = np.zeros(gpu_codes.shape, bool)
    for g in range(n_kv):
        mask[pages[:, None], g, pos] = True
    assert np.array_equal(gpu_codes[~mask], ref_codes[~mask]), "bytes outside written slots differ"
    n_bad = 0
    for g in range(n_kv):
        gc = oracle.unpack_codes_row(gpu_codes[pages[:, None], g, pos])
        rc = oracle.unpack_codes_row(ref_codes[pages[:, None], g, pos])
        diff = np.argwhere(gc != rc)
        for t, c in diff:
            a, b = int(gc[t, c]), int(rc[t, c])
            assert abs(a - b) == 1, f"code differs by more than one level (token {t}, head {g}, ch {c})"
            zd, sd = diag["zero16"][t, g], diag["scale16"][t, g]
            if np.ndim(zd):   # per-group diagnostics: the group of channel c
                zd, sd = zd[c * len(zd) // d], sd[c * len(sd) // d]
            z = float(np.array(zd).view(np.float16))
            s = float(np.array(sd).view(np.float16))
            if codebook == "uniform":
                e = z + (min(a, b) + 0.5) * s
            else:   # the threshold between Lloyd-Max codes a and b
                e = float(np.float32(z + s * oracle.LM_THRESHOLDS[min(a, b)]))
            y = float(diag["yc"][t, g, c])
            assert abs(y - e) <= BIN_EDGE_REL * max(abs(e), s), f"code mismatch away from a bin edge ({y} vs {e})"
            n_bad += 1
    return n_bad

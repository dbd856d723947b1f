"""Python binding of liboscar (include/oscar.h): INT2 three-segment decode
attention and the INT2 demotion kernel for AMD gfx950.

Argument marshalling only: each function checks dtypes and shapes, passes raw
device pointers and the current HIP stream to the C ABI, and turns a non-OK
status into an exception.  Every step of the computation runs in the HIP
kernels of liboscar.so.  There is no fallback: if the library is not built,
every call raises.  Build it with ``python -m bit_rotated_kv_attn_amd.build``.

PyTorch is used for device memory and streams only.

The offline calibration that produces the rotations and clip thresholds these
calls take (``bit_rotated_kv_attn_amd.calibrate``) is a separate host-side
step, run once per model before any decode; it is not part of the decode path.
"""
from __future__ import annotations

import ctypes
import math
import os

PAGE = 64
KIND_K, KIND_V = 0, 1
# INT2 codebooks (oscar.h); the Lloyd-Max flag is OR'ed into a demotion's kind
CODEBOOK_UNIFORM, CODEBOOK_LLOYD_MAX = 0, 0x100
# 64- and 32-channel quantisation groups (oscar.h); at most one is OR'ed into a demotion's kind
GROUPS_64, GROUPS_32 = 0x200, 0x400
# arithmetic the kernels of this build compute in (reported by bench.py)
COMPUTE_DTYPE = ("QK i8 MFMA (exact integer digits), PV f16 MFMA (fp16 weight pairs) + f32 sums and softmax; "
                 "bf16x3 MFMA rotation with certified decisions and fp64 exact recomputes in demotion")
# the bulk demotion's rotation x R runs on the bf16 matrix cores (MI355X dense bf16 MFMA peak)
DEMOTION_MATMUL_DTYPE, DEMOTION_MATMUL_PEAK_TFLOPS = "bf16", 2500.0
OSCAR_OK, OSCAR_EINVAL, OSCAR_EUNSUPPORTED, OSCAR_EWORKSPACE, OSCAR_EHIP, OSCAR_ESCRATCH = range(6)
# bytes of the static per-GPU scratch buffer of oscar_decode_step_static (oscar.h)
STATIC_SCRATCH_BYTES = 32 << 20
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liboscar.so")
ABI_VERSION = 5   # OSCAR_ABI_VERSION of the oscar.h these mirrors follow

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class DecodeArgs(ctypes.Structure):
    """Mirror of ``oscar_decode_args``."""
    _fields_ = [("batch", _i32), ("n_q_heads", _i32), ("n_kv_heads", _i32), ("head_dim", _i32),
                ("sm_scale", _f32), ("q", _vp), ("sink_k", _vp), ("sink_v", _vp), ("recent_k", _vp),
                ("recent_v", _vp), ("sink_cap", _i32), ("recent_cap", _i32), ("sink_len", _vp),
                ("recent_len", _vp), ("hist_len", _vp), ("max_hist_len", _i32), ("k_codes", _vp),
                ("v_codes", _vp), ("k_sz", _vp), ("v_sz", _vp), ("n_pages", _i64),
                ("block_table", _vp), ("max_pages", _i32), ("r_k", _vp), ("r_v", _vp), ("out", _vp),
                ("shared_pages", _i32), ("codebook", _i32), ("group_channels", _i32),
                ("prefix_cascade", _i32)]


class DemoteArgs(ctypes.Structure):
    """Mirror of ``oscar_demote_args``."""
    _fields_ = [("x", _vp), ("n_src", _i64), ("x_tok_stride", _i64), ("x_head_stride", _i64),
                ("src_idx", _vp), ("n_tok", _i64), ("rot", _vp), ("clip", _f32), ("dst_slot", _vp),
                ("codes", _vp), ("scale_zero", _vp), ("n_pages", _i64)]


class Bf16DecodeArgs(ctypes.Structure):
    """Mirror of ``oscar_bf16_decode_args``."""
    _fields_ = [("batch", _i32), ("n_q_heads", _i32), ("n_kv_heads", _i32), ("head_dim", _i32),
                ("sm_scale", _f32), ("q", _vp), ("k_pages", _vp), ("v_pages", _vp), ("n_pages", _i64),
                ("block_table", _vp), ("max_pages", _i32), ("ctx_len", _vp), ("max_ctx_len", _i32),
                ("out", _vp)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load liboscar.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m bit_rotated_kv_attn_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.oscar_abi_version.restype = ctypes.c_int
    L.oscar_abi_version.argtypes = []
    L.oscar_status_str.restype = ctypes.c_char_p
    L.oscar_status_str.argtypes = [ctypes.c_int]
    L.oscar_quantize_pack.restype = ctypes.c_int
    L.oscar_quantize_pack.argtypes = [_i32, _vp, _i64, _i64, _i64, _vp, _i64, _i32, _i32, _vp, _f32, _vp,
                                      _vp, _vp, _i64, _vp]
    L.oscar_decode_workspace_bytes.restype = _sz
    L.oscar_decode_workspace_bytes.argtypes = [_i32] * 7
    for name in ("oscar_decode_attn", "oscar_decode_rotate_query", "oscar_decode_scan", "oscar_decode_merge"):
        getattr(L, name).restype = ctypes.c_int
        getattr(L, name).argtypes = [ctypes.POINTER(DecodeArgs), _vp, _sz, _vp]
    L.oscar_decode_step.restype = ctypes.c_int
    L.oscar_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(DemoteArgs),
                                    ctypes.POINTER(DemoteArgs), _vp, _sz, _vp]
    L.oscar_decode_step_static.restype = ctypes.c_int
    L.oscar_decode_step_static.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(DemoteArgs),
                                           ctypes.POINTER(DemoteArgs), _vp]
    L.oscar_decode_bf16_workspace_bytes.restype = _sz
    L.oscar_decode_bf16_workspace_bytes.argtypes = [_i32] * 5
    L.oscar_decode_attn_bf16.restype = ctypes.c_int
    L.oscar_decode_attn_bf16.argtypes = [ctypes.POINTER(Bf16DecodeArgs), _vp, _sz, _vp]
    if L.oscar_abi_version() != ABI_VERSION:
        raise RuntimeError("liboscar ABI version mismatch")
    _lib = L
    return L


def oscar_abi_version() -> int:
    return lib().oscar_abi_version()


def oscar_status_str(status: int) -> str:
    return lib().oscar_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status == OSCAR_OK:
        return
    msg = f"{what}: {oscar_status_str(status)} (status {status})"
    if status == OSCAR_EHIP:
        raise RuntimeError(msg)
    raise ValueError(msg)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t, itemsize=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if itemsize is not None and t.element_size() != itemsize:
        raise ValueError(f"{name} must have {itemsize}-byte elements")
    return t.data_ptr()


def groups_per_head(head_dim: int, group_channels: int) -> int:
    """(scale, zero) groups per (token, head): 1 for whole-head groups
    (group_channels 0, or at least head_dim), else head_dim / group_channels."""
    return 1 if group_channels <= 0 or group_channels >= head_dim else head_dim // group_channels


def kind_group_channels(kind: int) -> int:
    """The group size a demotion kind's flags select (0: the whole head)."""
    return 64 if int(kind) & GROUPS_64 else 32 if int(kind) & GROUPS_32 else 0


def oscar_quantize_pack(kind: int, x, rot, clip: float, dst_slot, codes, scale_zero, *, src_idx=None,
                        n_src=None, x_tok_stride=None, x_head_stride=None, stream=None) -> None:
    """Demote tokens of one tensor into INT2 pages (see oscar_quantize_pack in oscar.h).

    kind: KIND_K or KIND_V, optionally | CODEBOOK_LLOYD_MAX and / or | GROUPS_64 or GROUPS_32.

    x: bf16 bits; by default a contiguous [n_src][n_kv][d] tensor.  For other
    layouts pass n_src, x_tok_stride and x_head_stride (elements).
    rot fp32 [n_kv][d][d]; dst_slot int32 [n_tok]; codes uint8 [n_pages][n_kv][64*d/4];
    scale_zero 16-bit [n_pages][n_kv][64*ng][2] (ng groups per head); src_idx int32 [n_tok] or None."""
    n_kv, d = rot.shape[0], rot.shape[-1]
    if x_tok_stride is None:
        if x.dim() != 3 or x.shape[1:] != (n_kv, d):
            raise ValueError("x must be [n_src][n_kv][d]")
        n_src, x_tok_stride, x_head_stride = x.shape[0], n_kv * d, d
    n_tok = dst_slot.numel()
    if src_idx is not None and src_idx.numel() != n_tok:
        raise ValueError("src_idx and dst_slot lengths differ")
    ng = groups_per_head(d, kind_group_channels(kind))
    if codes.shape[1:] != (n_kv, PAGE * d // 4) or scale_zero.shape[1:] != (n_kv, PAGE * ng, 2):
        raise ValueError("pool shapes do not match [n_pages][n_kv][...]")
    if dst_slot.dtype.itemsize != 4 or (src_idx is not None and src_idx.dtype.itemsize != 4):
        raise ValueError("dst_slot / src_idx must be int32")
    st = lib().oscar_quantize_pack(int(kind), _ptr(x, 2, "x"), int(n_src), int(x_tok_stride),
                                   int(x_head_stride), _ptr(src_idx, 4, "src_idx"), int(n_tok), int(n_kv),
                                   int(d), _ptr(rot, 4, "rot"), float(clip), _ptr(dst_slot, 4, "dst_slot"),
                                   _ptr(codes, 1, "codes"), _ptr(scale_zero, 2, "scale_zero"),
                                   int(codes.shape[0]), _stream(stream))
    _check(st, "oscar_quantize_pack")


def oscar_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_hist_len, sink_cap=64,
                                 recent_cap=256) -> int:
    return int(lib().oscar_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_hist_len,
                                                  sink_cap, recent_cap))


def decode_args(*, q, sink_k, sink_v, recent_k, recent_v, sink_len, recent_len, hist_len, max_hist_len: int,
                k_codes, v_codes, k_sz, v_sz, block_table, r_k, r_v, out, workspace=None,
                sm_scale: float | None = None, shared_pages: int = 0, codebook: int = CODEBOOK_UNIFORM,
                group_channels: int = 0, prefix_cascade: bool = False):
    """Marshal tensors into (DecodeArgs, workspace pointer, workspace bytes).

    q bf16 [B][Hq][d]; sink_k/v bf16 [B][n_kv][sink_cap][d]; recent_k/v bf16
    [B][n_kv][recent_cap][d]; *_len int32 [B]; pools as for oscar_quantize_pack;
    block_table int32 [B][max_pages]; r_k/r_v fp32 [n_kv][d][d]; out fp32
    [B][Hq][d]; workspace uint8 device tensor (size from oscar_decode_workspace_bytes;
    None for oscar_decode_step_static, which brings its own);
    shared_pages: leading history pages every request holds at the same ids (0: none);
    codebook: CODEBOOK_UNIFORM or CODEBOOK_LLOYD_MAX, as the pools were demoted;
    group_channels: 0 (whole-head groups), 64 or 32, as the pools were demoted;
    prefix_cascade: read the splits inside the shared prefix in cascade blocks
    where oscar.h allows it (one page read per group of 16 requests).
    The returned DecodeArgs holds a reference to every tensor it points to
    (``keep``), so tensors made inline stay allocated while the args live; a
    captured graph that replays the call must keep the args alive too."""
    B, Hq, d = q.shape
    n_kv = sink_k.shape[1]
    if tuple(out.shape) != (B, Hq, d):
        raise ValueError("out must be [B][Hq][d] fp32")
    pairs = PAGE * groups_per_head(d, group_channels)   # (scale, zero) pairs per (page, head)
    for name, sz in (("k_sz", k_sz), ("v_sz", v_sz)):
        if sz.dim() != 4 or sz.shape[2:] != (pairs, 2):
            raise ValueError(f"{name} must be [n_pages][n_kv][{pairs}][2] for group_channels={group_channels}")
    a = DecodeArgs(batch=B, n_q_heads=Hq, n_kv_heads=n_kv, head_dim=d,
                   sm_scale=float(1.0 / math.sqrt(d) if sm_scale is None else sm_scale),
                   q=_ptr(q, 2, "q"), sink_k=_ptr(sink_k, 2, "sink_k"), sink_v=_ptr(sink_v, 2, "sink_v"),
                   recent_k=_ptr(recent_k, 2, "recent_k"), recent_v=_ptr(recent_v, 2, "recent_v"),
                   sink_cap=sink_k.shape[2], recent_cap=recent_k.shape[2],
                   sink_len=_ptr(sink_len, 4, "sink_len"), recent_len=_ptr(recent_len, 4, "recent_len"),
                   hist_len=_ptr(hist_len, 4, "hist_len"), max_hist_len=int(max_hist_len),
                   k_codes=_ptr(k_codes, 1, "k_codes"), v_codes=_ptr(v_codes, 1, "v_codes"),
                   k_sz=_ptr(k_sz, 2, "k_sz"), v_sz=_ptr(v_sz, 2, "v_sz"), n_pages=k_codes.shape[0],
                   block_table=_ptr(block_table, 4, "block_table"), max_pages=block_table.shape[1],
                   r_k=_ptr(r_k, 4, "r_k"), r_v=_ptr(r_v, 4, "r_v"), out=_ptr(out, 4, "out"),
                   shared_pages=int(shared_pages), codebook=int(codebook), group_channels=int(group_channels),
                   prefix_cascade=int(bool(prefix_cascade)))
    a.keep = (q, sink_k, sink_v, recent_k, recent_v, sink_len, recent_len, hist_len, k_codes, v_codes, k_sz, v_sz,
              block_table, r_k, r_v, out, workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return a, _ptr(workspace, name="workspace"), nbytes


def _decode(name: str, args, stream, kw):
    a, ws, nbytes = args if args is not None else decode_args(**kw)
    st = getattr(lib(), name)(ctypes.byref(a), ws, nbytes, _stream(stream))
    _check(st, name)


def oscar_decode_attn(*, args=None, stream=None, **kw) -> None:
    """Three-segment decode attention (see oscar_decode_attn in oscar.h).
    Pass the tensors as keywords (see :func:`decode_args`) or a prebuilt
    ``args=decode_args(...)`` tuple."""
    _decode("oscar_decode_attn", args, stream, kw)


def oscar_decode_rotate_query(*, args=None, stream=None, **kw) -> None:
    """Phase 1 of oscar_decode_attn: q_rot = q R_K per query head."""
    _decode("oscar_decode_rotate_query", args, stream, kw)


def oscar_decode_scan(*, args=None, stream=None, **kw) -> None:
    """Phase 2 of oscar_decode_attn: INT2 history split-K scan and BF16 tiles."""
    _decode("oscar_decode_scan", args, stream, kw)


def oscar_decode_merge(*, args=None, stream=None, **kw) -> None:
    """Phase 3 of oscar_decode_attn: merge partials, apply R_V^T, normalise."""
    _decode("oscar_decode_merge", args, stream, kw)


def demote_args(*, x, rot, clip: float, dst_slot, codes, scale_zero, src_idx=None, n_src=None,
                x_tok_stride=None, x_head_stride=None) -> DemoteArgs:
    """Marshal one tensor's demotion for :func:`oscar_decode_step` (arguments
    as for :func:`oscar_quantize_pack`).  The returned DemoteArgs holds a
    reference to every tensor it points to (``keep``)."""
    n_kv, d = rot.shape[0], rot.shape[-1]
    if x_tok_stride is None:
        if x.dim() != 3 or x.shape[1:] != (n_kv, d):
            raise ValueError("x must be [n_src][n_kv][d]")
        n_src, x_tok_stride, x_head_stride = x.shape[0], n_kv * d, d
    n_tok = dst_slot.numel()
    if src_idx is not None and src_idx.numel() != n_tok:
        raise ValueError("src_idx and dst_slot lengths differ")
    # the step decides the groups (its args' group_channels); oscar_decode_step checks this pool against them
    if codes.shape[1:] != (n_kv, PAGE * d // 4) or scale_zero.shape[1:] not in (
            (n_kv, PAGE * groups_per_head(d, gc), 2) for gc in (0, 64, 32)):
        raise ValueError("pool shapes do not match [n_pages][n_kv][...]")
    if dst_slot.dtype.itemsize != 4 or (src_idx is not None and src_idx.dtype.itemsize != 4):
        raise ValueError("dst_slot / src_idx must be int32")
    a = DemoteArgs(x=_ptr(x, 2, "x"), n_src=int(n_src), x_tok_stride=int(x_tok_stride),
                   x_head_stride=int(x_head_stride), src_idx=_ptr(src_idx, 4, "src_idx"), n_tok=int(n_tok),
                   rot=_ptr(rot, 4, "rot"), clip=float(clip), dst_slot=_ptr(dst_slot, 4, "dst_slot"),
                   codes=_ptr(codes, 1, "codes"), scale_zero=_ptr(scale_zero, 2, "scale_zero"),
                   n_pages=int(codes.shape[0]))
    a.sz_pairs = int(scale_zero.shape[2])   # (scale, zero) pairs per (page, head) of this pool
    a.keep = (x, src_idx, rot, dst_slot, codes, scale_zero)
    return a


def oscar_decode_step(*, args, demote_k=None, demote_v=None, stream=None) -> None:
    """One decode step (see oscar_decode_step in oscar.h): the demotions
    (:func:`demote_args` results, or None) run in the decode's last launch.
    ``args`` is a :func:`decode_args` tuple."""
    a, ws, nbytes = args
    pairs = PAGE * groups_per_head(a.head_dim, a.group_channels)
    for name, dm in (("demote_k", demote_k), ("demote_v", demote_v)):
        if dm is not None and getattr(dm, "sz_pairs", pairs) != pairs:
            raise ValueError(f"{name}: its scale/zero pool holds {dm.sz_pairs} pairs per (page, head); "
                             f"group_channels={a.group_channels} writes {pairs}")
    st = lib().oscar_decode_step(ctypes.byref(a), ctypes.byref(demote_k) if demote_k is not None else None,
                                 ctypes.byref(demote_v) if demote_v is not None else None, ws, nbytes,
                                 _stream(stream))
    _check(st, "oscar_decode_step")


def oscar_decode_step_static(*, args, demote_k=None, demote_v=None, stream=None) -> None:
    """oscar_decode_step with its workspace in the library's static per-GPU
    scratch buffer (see oscar_decode_step_static in oscar.h): for callers that
    cannot allocate device memory.  ``args`` is a :func:`decode_args` tuple;
    its workspace, if any, is not used.  Raises ValueError (OSCAR_ESCRATCH)
    when the sizes need more than STATIC_SCRATCH_BYTES.  Calls that can
    overlap on one GPU race on the shared buffer."""
    a = args[0]
    pairs = PAGE * groups_per_head(a.head_dim, a.group_channels)
    for name, dm in (("demote_k", demote_k), ("demote_v", demote_v)):
        if dm is not None and getattr(dm, "sz_pairs", pairs) != pairs:
            raise ValueError(f"{name}: its scale/zero pool holds {dm.sz_pairs} pairs per (page, head); "
                             f"group_channels={a.group_channels} writes {pairs}")
    st = lib().oscar_decode_step_static(ctypes.byref(a),
                                        ctypes.byref(demote_k) if demote_k is not None else None,
                                        ctypes.byref(demote_v) if demote_v is not None else None, _stream(stream))
    _check(st, "oscar_decode_step_static")


def oscar_decode_bf16_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_ctx_len) -> int:
    return int(lib().oscar_decode_bf16_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_ctx_len))


def oscar_decode_attn_bf16(*, q, k_pages, v_pages, block_table, ctx_len, max_ctx_len: int, out, workspace,
                           sm_scale: float | None = None, stream=None) -> None:
    """BF16 paged decode attention comparator (see oscar_decode_attn_bf16 in oscar.h)."""
    B, Hq, d = q.shape
    n_kv = k_pages.shape[1]
    a = Bf16DecodeArgs(batch=B, n_q_heads=Hq, n_kv_heads=n_kv, head_dim=d,
                       sm_scale=float(1.0 / math.sqrt(d) if sm_scale is None else sm_scale),
                       q=_ptr(q, 2, "q"), k_pages=_ptr(k_pages, 2, "k_pages"), v_pages=_ptr(v_pages, 2, "v_pages"),
                       n_pages=k_pages.shape[0], block_table=_ptr(block_table, 4, "block_table"),
                       max_pages=block_table.shape[1], ctx_len=_ptr(ctx_len, 4, "ctx_len"),
                       max_ctx_len=int(max_ctx_len), out=_ptr(out, 4, "out"))
    st = lib().oscar_decode_attn_bf16(ctypes.byref(a), _ptr(workspace, name="workspace"),
                                      workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "oscar_decode_attn_bf16")

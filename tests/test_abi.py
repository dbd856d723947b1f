"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/oscar.h, and rejects invalid arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import bit_rotated_kv_attn_amd as hip

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "oscar.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"OSCAR_API\s+[\w\s\*]*?\b(oscar_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("oscar_quantize_pack", "oscar_decode_attn", "oscar_decode_workspace_bytes",
              "oscar_decode_attn_bf16", "oscar_decode_bf16_workspace_bytes", "oscar_status_str",
              "oscar_abi_version"):
        assert n in names


def test_library_exports_every_declared_function():
    L = hip.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert hip.oscar_abi_version() == hip.ABI_VERSION == 5
    # the binding offers a function of the same name for each entry point
    for n in declared_functions():
        assert callable(getattr(hip, n)), n


def test_status_strings():
    for s in range(6):
        assert hip.oscar_status_str(s) != "unknown status"
    assert hip.oscar_status_str(99) == "unknown status"


def _qp(**kw):
    a = dict(kind=0, x=1, n_src=1, tok=128, head=128, src=None, n_tok=1, n_kv=1, d=128, rot=1, clip=1.0,
             dst=1, codes=1, sz=1, n_pages=1)
    a.update(kw)
    vp = lambda v: None if v is None else ctypes.c_void_p(v)
    return hip.lib().oscar_quantize_pack(a["kind"], vp(a["x"]), a["n_src"], a["tok"], a["head"], vp(a["src"]),
                                         a["n_tok"], a["n_kv"], a["d"], vp(a["rot"]), a["clip"], vp(a["dst"]),
                                         vp(a["codes"]), vp(a["sz"]), a["n_pages"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(kind=2), hip.OSCAR_EINVAL),
    (dict(kind=0x800), hip.OSCAR_EINVAL),                            # an unknown flag
    (dict(kind=0x600), hip.OSCAR_EINVAL),                            # both group sizes
    (dict(kind=0x102), hip.OSCAR_EINVAL),
    (dict(d=96), hip.OSCAR_EUNSUPPORTED),
    (dict(clip=0.0), hip.OSCAR_EINVAL),
    (dict(clip=float("nan")), hip.OSCAR_EINVAL),
    (dict(clip=float("inf")), hip.OSCAR_EINVAL),
    (dict(clip=65505.0), hip.OSCAR_EINVAL),
    (dict(n_tok=-1), hip.OSCAR_EINVAL),
    (dict(n_kv=0), hip.OSCAR_EINVAL),
    (dict(x=None), hip.OSCAR_EINVAL),
    (dict(rot=None), hip.OSCAR_EINVAL),
    (dict(dst=None), hip.OSCAR_EINVAL),
    (dict(codes=None), hip.OSCAR_EINVAL),
    (dict(n_tok=0, x=None, rot=None), hip.OSCAR_OK),     # no-op without touching anything
])
def test_quantize_pack_validation(kw, status):
    assert _qp(**kw) == status


def _decode_args(**kw):
    a = hip.DecodeArgs(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, sm_scale=0.088, q=1, sink_k=1,
                       sink_v=1, recent_k=1, recent_v=1, sink_cap=64, recent_cap=256, sink_len=1, recent_len=1,
                       hist_len=1, max_hist_len=100, k_codes=1, v_codes=1, k_sz=1, v_sz=1, n_pages=2,
                       block_table=1, max_pages=2, r_k=1, r_v=1, out=1)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), hip.OSCAR_EUNSUPPORTED),
    (dict(n_q_heads=24, n_kv_heads=8), hip.OSCAR_EUNSUPPORTED),     # G = 3
    (dict(n_q_heads=9), hip.OSCAR_EINVAL),                           # not a multiple
    (dict(sm_scale=0.0), hip.OSCAR_EINVAL),
    (dict(sm_scale=float("nan")), hip.OSCAR_EINVAL),
    (dict(q=None), hip.OSCAR_EINVAL),
    (dict(out=None), hip.OSCAR_EINVAL),
    (dict(k_codes=None), hip.OSCAR_EINVAL),
    (dict(max_pages=1), hip.OSCAR_EINVAL),                           # 64 < max_hist_len
    (dict(n_pages=0), hip.OSCAR_EINVAL),
    (dict(sink_cap=5000), hip.OSCAR_EINVAL),
    (dict(max_hist_len=-1), hip.OSCAR_EINVAL),
    (dict(shared_pages=-1), hip.OSCAR_EINVAL),
    (dict(shared_pages=2), hip.OSCAR_EINVAL),                        # 2 pages > max_hist_len 100
    (dict(codebook=1), hip.OSCAR_EINVAL),
    (dict(group_channels=16), hip.OSCAR_EINVAL),
    (dict(group_channels=48), hip.OSCAR_EINVAL),
    (dict(prefix_cascade=2), hip.OSCAR_EINVAL),
    (dict(prefix_cascade=-1), hip.OSCAR_EINVAL),
    (dict(batch=0, q=None, out=None), hip.OSCAR_OK),
])
def test_decode_validation(kw, status):
    a = _decode_args(**kw)
    assert hip.lib().oscar_decode_attn(ctypes.byref(a), ctypes.c_void_p(256), 1 << 30, None) == status


def test_decode_workspace_checks():
    a = _decode_args()
    need = hip.oscar_decode_workspace_bytes(1, 8, 2, 128, 100, 64, 256)
    assert need > 0
    L = hip.lib()
    assert L.oscar_decode_attn(ctypes.byref(a), None, need, None) == hip.OSCAR_EWORKSPACE
    assert L.oscar_decode_attn(ctypes.byref(a), ctypes.c_void_p(256), need - 1, None) == hip.OSCAR_EWORKSPACE
    assert L.oscar_decode_attn(ctypes.byref(a), ctypes.c_void_p(260), need, None) == hip.OSCAR_EWORKSPACE
    assert hip.oscar_decode_workspace_bytes(1, 8, 2, 96, 100, 64, 256) == 0


def test_workspace_sizes_are_positive():
    assert hip.oscar_decode_workspace_bytes(1, 64, 8, 128, 32448) > 0
    assert hip.oscar_decode_workspace_bytes(1, 64, 8, 128, 99680) > 0
    assert hip.oscar_decode_workspace_bytes(1, 64, 8, 128, 0) > 0
    assert hip.oscar_decode_bf16_workspace_bytes(28, 32, 8, 128, 100000) > 0


def _demote(**kw):
    d = hip.DemoteArgs(x=1, n_src=4, x_tok_stride=256, x_head_stride=128, src_idx=None, n_tok=1, rot=1, clip=3.0,
                       dst_slot=1, codes=1, scale_zero=1, n_pages=2)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(n_tok=-1), hip.OSCAR_EINVAL),
    (dict(n_tok=(1 << 24)), hip.OSCAR_EINVAL),                      # > 2^24 / n_kv
    (dict(clip=0.0), hip.OSCAR_EINVAL),
    (dict(clip=float("inf")), hip.OSCAR_EINVAL),
    (dict(x=None), hip.OSCAR_EINVAL),
    (dict(rot=None), hip.OSCAR_EINVAL),
    (dict(codes=None), hip.OSCAR_EINVAL),
    (dict(n_src=-2), hip.OSCAR_EINVAL),
    (dict(n_tok=0, x=None, rot=None, codes=None), None),            # nothing to demote: decode checks decide
])
def test_decode_step_validation(kw, status):
    """Step arguments are checked on the host before any HIP call: bad
    demotion arguments fail even when the decode arguments are valid."""
    L = hip.lib()
    a = _decode_args(q=None)                                         # decode itself invalid
    good = _decode_args()
    dk = _demote(**kw)
    if status is None:
        assert L.oscar_decode_step(ctypes.byref(a), ctypes.byref(dk), None, ctypes.c_void_p(256), 1 << 30,
                                   None) == hip.OSCAR_EINVAL
        return
    assert L.oscar_decode_step(ctypes.byref(good), ctypes.byref(dk), None, ctypes.c_void_p(260), 1 << 30,
                               None) == hip.OSCAR_EWORKSPACE   # workspace checked first
    assert L.oscar_decode_step(ctypes.byref(_decode_args(batch=0, q=None, out=None)), None, ctypes.byref(dk),
                               None, 0, None) == status


def test_static_step_checks_sizes_before_any_hip_call():
    """oscar_decode_step_static: sizes past its static scratch buffer return
    OSCAR_ESCRATCH, and invalid arguments OSCAR_EINVAL, with no HIP call
    (this host has no GPU)."""
    big = hip.DecodeArgs(batch=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, sm_scale=0.088, sink_cap=64,
                         recent_cap=256, max_hist_len=99680, max_pages=1558, n_pages=1)
    need = hip.oscar_decode_workspace_bytes(4096, 32, 8, 128, 99680)
    assert need > hip.STATIC_SCRATCH_BYTES
    assert hip.lib().oscar_decode_step_static(ctypes.byref(big), None, None, None) == hip.OSCAR_ESCRATCH
    small = hip.DecodeArgs(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, sm_scale=0.088, sink_cap=64,
                           recent_cap=256, max_hist_len=99680, max_pages=1558, n_pages=1)   # null pointers
    assert hip.oscar_decode_workspace_bytes(1, 32, 8, 128, 99680) <= hip.STATIC_SCRATCH_BYTES
    assert hip.lib().oscar_decode_step_static(ctypes.byref(small), None, None, None) == hip.OSCAR_EINVAL
    assert hip.lib().oscar_decode_step_static(None, None, None, None) == hip.OSCAR_EINVAL

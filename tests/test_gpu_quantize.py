"""GPU parity of oscar_quantize_pack against the oracle quantiser."""
import numpy as np
import pytest
import torch

import oracle
import pins
import synth
from gpu_util import compare_quant, dev, empty_pools, gpu_quantize, host

pytestmark = pytest.mark.gpu
PAGE = 64


def _oracle(kind, x, rot, clip, slots, n_pages, src_idx=None):
    n_kv, d = rot.shape[0], rot.shape[-1]
    c = np.zeros((n_pages, n_kv, PAGE * d // 4), np.uint8)
    s = np.zeros((n_pages, n_kv, PAGE, 2), np.uint16)
    diag = oracle.quantize_pack_ref(kind, x, rot, clip, slots, c, s, src_idx=src_idx)
    return c, s, diag


def _inputs(seed, n_tok, n_kv, d, n_pages):
    rng = np.random.default_rng(seed)
    outl = synth.outlier_channels(rng, n_kv, d, 3)
    x = synth.kv_tokens(rng, (n_tok,), n_kv, d, outl)
    slots = (rng.permutation(n_pages * PAGE)[:n_tok]).astype(np.int32)
    return rng, x, slots


@pytest.mark.parametrize("n_tok", [7, 300])          # one block per token / 32-token tiles
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", ["k", "v"])
def test_signed_permutation_bit_exact(d, kind, n_tok):
    """R a signed permutation: every rotated value is exact, so codes, scales
    and zeros must match the oracle bit for bit with no exception."""
    rng, x, slots = _inputs(1, n_tok, 3, d, 6)
    rot = np.stack([pins.signed_permutation(d, rng)[0] for _ in range(3)])
    ref = _oracle(kind, x, rot, 9.5, slots, 6)
    got = gpu_quantize(kind, x, rot, 9.5, slots, 6)
    compare_quant(kind, got[0], got[1], ref[0], ref[1], ref[2], d, exact=True)


@pytest.mark.parametrize("kind", ["k", "v"])
def test_tiny_config_history(kind):
    cfg = synth.make_decode_config(0)
    x = cfg["hist_" + kind]
    rot, tau = cfg["r_" + kind], cfg["tau_" + kind]
    ref = _oracle(kind, x, rot, tau, cfg["hist_slot"], cfg["n_pages"])
    got = gpu_quantize(kind, x, rot, tau, cfg["hist_slot"], cfg["n_pages"])
    compare_quant(kind, got[0], got[1], ref[0], ref[1], ref[2], cfg["head_dim"])


@pytest.mark.parametrize("n_tok", [41, 101])         # one block per token / 32-token tiles
@pytest.mark.parametrize("kind", ["k", "v"])
def test_edge_cases(kind, n_tok):
    """Degenerate groups, fully clipped groups, skipped slots and source rows,
    a gather index, and a ragged token count."""
    d, n_kv, n_pages = 128, 2, 3
    rng = np.random.default_rng(5)
    rot = np.stack([pins.random_orthogonal(d, rng) for _ in range(n_kv)])
    x = synth.f32_to_bf16_bits(rng.standard_normal((n_tok, n_kv, d)).astype(np.float32))
    x[3] = 0                                                   # all-zero token: scale 0
    x[4] = synth.f32_to_bf16_bits(np.full((n_kv, d), 1e4, np.float32))   # clipped everywhere
    slots = rng.permutation(n_pages * PAGE)[:n_tok].astype(np.int32)
    slots[7] = -5
    slots[8] = n_pages * PAGE + 3
    src = rng.permutation(n_tok).astype(np.int32)
    src[9] = n_tok
    src[10] = -1
    ref = _oracle(kind, x, rot, 2.0, slots, n_pages, src_idx=src)
    got = gpu_quantize(kind, x, rot, 2.0, slots, n_pages, src_idx=src)
    compare_quant(kind, got[0], got[1], ref[0], ref[1], ref[2], d)


def test_strided_source_recent_ring():
    """Demote straight out of a [B][n_kv][cap][d] recent window with token
    and head strides (the steady-state step moves the oldest recent token)."""
    import bit_rotated_kv_attn_amd as hip
    cfg = synth.make_decode_config(0)
    B, n_kv, cap, d = cfg["recent_k"].shape
    ring_head = np.array([17], np.int32)                       # oldest token's ring slot per request
    src = (np.arange(B) * n_kv * cap + ring_head).astype(np.int32)
    slot = np.array([5 * PAGE + 63], np.int32)                 # any free history slot
    n_pages = cfg["n_pages"]
    codes, sz = empty_pools(n_pages, n_kv, d)
    hip.oscar_quantize_pack(hip.KIND_K, dev(cfg["recent_k"]), dev(cfg["r_k"]), float(cfg["tau_k"]),
                            dev(slot), codes, sz, src_idx=dev(src), n_src=B * n_kv * cap,
                            x_tok_stride=d, x_head_stride=cap * d)
    torch.cuda.synchronize()
    x_tok = cfg["recent_k"][0, :, 17, :][None]                  # [1][n_kv][d]
    ref = _oracle("k", x_tok, cfg["r_k"], cfg["tau_k"], slot, n_pages)
    compare_quant("k", host(codes), host(sz, np.uint16), ref[0], ref[1], ref[2], d)


@pytest.mark.parametrize("d", [64, 128])
def test_bulk_unaligned_source_rows(d):
    """The 32-token tiles read a token's channels as 16-byte vectors only when
    the row is 16-byte aligned: with a token stride of n_kv*d + 3 elements most
    rows are not, and those are read element by element."""
    import bit_rotated_kv_attn_amd as hip
    n_tok, n_kv, n_pages = 150, 2, 4
    rng, x, slots = _inputs(8, n_tok, n_kv, d, n_pages)
    rot = np.stack([pins.random_orthogonal(d, rng) for _ in range(n_kv)])
    stride = n_kv * d + 3
    buf = np.zeros(n_tok * stride + 8, np.uint16)
    for t in range(n_tok):
        buf[t * stride: t * stride + n_kv * d] = x[t].reshape(-1)
    codes, sz = empty_pools(n_pages, n_kv, d)
    xb = dev(buf)
    hip.oscar_quantize_pack(hip.KIND_V, xb, dev(rot), 3.0, dev(slots), codes, sz, n_src=n_tok,
                            x_tok_stride=stride, x_head_stride=d)
    torch.cuda.synchronize()
    ref = _oracle("v", x, rot, 3.0, slots, n_pages)
    compare_quant("v", host(codes), host(sz, np.uint16), ref[0], ref[1], ref[2], d)


def test_zero_tokens_is_noop():
    import bit_rotated_kv_attn_amd as hip
    codes, sz = empty_pools(2, 1, 64)
    hip.oscar_quantize_pack(hip.KIND_V, dev(np.zeros((0, 1, 64), np.uint16)),
                            dev(np.eye(64, dtype=np.float32)[None]), 1.0, dev(np.zeros(0, np.int32)), codes, sz)
    torch.cuda.synchronize()
    assert not host(codes).any() and not host(sz).any()


def test_invalid_arguments_raise():
    import bit_rotated_kv_attn_amd as hip
    codes, sz = empty_pools(1, 1, 64)
    x = dev(np.zeros((1, 1, 64), np.uint16))
    rot = dev(np.eye(64, dtype=np.float32)[None])
    with pytest.raises(ValueError):
        hip.oscar_quantize_pack(hip.KIND_K, x, rot, 0.0, dev(np.zeros(1, np.int32)), codes, sz)
    with pytest.raises(ValueError):
        hip.oscar_quantize_pack(7, x, rot, 1.0, dev(np.zeros(1, np.int32)), codes, sz)

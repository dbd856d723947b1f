"""Pins for the seeded input generator (rotation, threshold, data shapes)."""
import math

import numpy as np
import pytest
import torch

import synth


@pytest.mark.parametrize("d", [4, 8, 64, 128])
def test_hadamard_orthonormal(d):
    h = synth.hadamard(d)
    assert np.abs(h @ h.T - np.eye(d)).max() < 1e-12
    assert np.all(np.abs(np.abs(h) * math.sqrt(d) - 1) < 1e-12)


def test_bit_reversal_known_values_and_involution():
    p = synth.bit_reversal_perm(8)
    # bit reversal on 3 bits: 1 -> 4, 3 -> 6, 6 -> 3
    assert p[1, 4] == 1 and p[3, 6] == 1 and p[6, 3] == 1 and p[0, 0] == 1 and p[7, 7] == 1
    assert np.array_equal(p @ p, np.eye(8))


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_orthogonal_and_eigen(d):
    rng = np.random.default_rng(1)
    c, w, u = synth.spd_eigenbasis(d, rng)
    assert np.all(np.diff(w) <= 0)
    assert np.abs(c @ u - u * w).max() <= 1e-10 * np.abs(c).max()
    r = synth.make_rotation(d, np.random.default_rng(1))
    assert r.dtype == np.float32
    assert np.abs(r.astype(np.float64).T @ r.astype(np.float64) - np.eye(d)).max() <= 1e-5


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 30,
                        np.float32([1.00390625, 1.01171875, -3e-3, 0.0, -0.0, 1e-40])])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_tiny_config_shapes_and_determinism():
    a = synth.make_decode_config(0)
    b = synth.make_decode_config(0)
    for k in ("q", "sink_k", "recent_v", "hist_k", "hist_v", "block_table", "r_k", "r_v"):
        assert np.array_equal(a[k], b[k]), k
    assert a["tau_k"] == b["tau_k"] and a["tau_v"] == b["tau_v"]
    assert a["q"].shape == (1, 4, 64)
    assert a["sink_k"].shape == (1, 2, 64, 64) and a["recent_k"].shape == (1, 2, 256, 64)
    assert a["hist_len"][0] == 704 and a["n_pages"] == 11
    assert sorted(a["block_table"][0].tolist()) == list(range(11))
    # outlier channels really are ~20x larger
    x = synth.bf16_bits_to_f32(a["hist_k"]).astype(np.float64)
    for g in range(2):
        std = x[:, g, :].std(axis=0)
        big = np.argsort(-std)[:3]
        assert set(big.tolist()) == set(a["outliers_k"][g].tolist())
        assert std[big].min() > 10 * np.median(std)


def test_clip_threshold_is_percentile():
    a = synth.make_decode_config(0)
    x = synth.bf16_bits_to_f32(a["hist_k"]).astype(np.float64)
    vals = np.concatenate([np.abs(x[:, g] @ a["r_k"][g].astype(np.float64)).ravel() for g in range(2)])
    frac = (vals <= a["tau_k"]).mean()
    assert abs(frac - 0.999) < 2e-4


def test_shared_prefix_table():
    shape = synth.DecodeShape("t", 3, 8, 2, 64, 64 + 256 + 64 * 10 + 32, shared_hist_pages=4)
    cfg = synth.make_decode_config(0, shape=shape, seed_index=40)
    t = cfg["block_table"]
    assert t.shape == (3, 11)
    assert np.all(t[:, :4] == t[0, :4])
    priv = t[:, 4:].ravel()
    assert len(set(priv.tolist())) == priv.size
    assert cfg["n_pages"] == 4 + 3 * 7
    assert cfg["hist_k"].shape[0] == 4 * 64 + 3 * (6 * 64 + 32)

"""Pins of the offline calibration tool (bit_rotated_kv_attn_amd.calibrate)
against definitions written out independently: brute-force sums on tiny
inputs, closed forms, a covariance with a planted eigenbasis, the stand-in
rotation recipe of the input generator (a different Hadamard construction),
and hand-computed percentiles.  CPU only."""
import math

import numpy as np
import pytest

from bit_rotated_kv_attn_amd import calibrate as cal
import synth


@pytest.mark.parametrize("d", [1, 2, 4, 8, 64, 128])
def test_hadamard_is_orthogonal_sylvester(d):
    h = cal.hadamard(d)
    assert np.allclose(h @ h.T, np.eye(d), atol=1e-12)
    assert np.allclose(np.abs(h), 1 / math.sqrt(d))
    assert np.allclose(h, synth.hadamard(d))                 # block recursion [[H, H], [H, -H]]
    if d >= 2:   # the recursion written out for one level
        half = cal.hadamard(d // 2) / math.sqrt(2)
        assert np.allclose(h, np.block([[half, half], [half, -half]]))


@pytest.mark.parametrize("d", [2, 8, 64])
def test_bit_reversal(d):
    p = cal.bit_reversal(d)
    assert np.array_equal(p @ p, np.eye(d))                  # an involution
    nb = d.bit_length() - 1
    for i in range(d):                                       # the index bits, written as a string, reversed
        assert p[i, int(format(i, f"0{nb}b")[::-1], 2)] == 1
    assert np.array_equal(p, synth.bit_reversal_perm(d))


def test_query_covariance_brute_force():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((7, 5))
    ref = np.zeros((5, 5))
    for n in range(7):
        for i in range(5):
            for j in range(5):
                ref[i, j] += q[n, i] * q[n, j] / 7
    assert np.allclose(cal.query_covariance(q), ref, atol=1e-14)


def test_score_weighted_value_covariance_brute_force():
    rng = np.random.default_rng(2)
    nq, nk, d, sm = 4, 6, 3, 0.7
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    pos = np.array([0, 2, 3, 5])
    o = np.zeros((nq, d))
    for a in range(nq):
        logits = [sm * sum(q[a, c] * k[j, c] for c in range(d)) for j in range(pos[a] + 1)]
        top = max(logits)
        w = [math.exp(x - top) for x in logits]
        for j in range(pos[a] + 1):
            o[a] += w[j] / sum(w) * v[j]
    ref = sum(np.outer(o[a], o[a]) for a in range(nq)) / nq
    s = cal.causal_scores(q, k, sm, pos)
    assert np.allclose(s.sum(axis=1), 1.0) and np.all(s[0, 1:] == 0.0)
    assert np.allclose(cal.score_weighted_value_covariance(s, v), ref, atol=1e-13)


def test_eigenbasis_of_planted_covariance():
    rng = np.random.default_rng(3)
    d = 16
    qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    w = rng.permutation(np.linspace(1.0, 9.0, d))            # distinct eigenvalues, shuffled
    c = qm @ np.diag(w) @ qm.T
    wv, u = cal.eigenbasis(c)
    assert np.allclose(wv, np.sort(w)[::-1], atol=1e-10)
    order = np.argsort(-w)
    for col in range(d):                                     # the planted vectors, up to sign
        ref = qm[:, order[col]]
        assert np.isclose(abs(u[:, col] @ ref), 1.0, atol=1e-9)
        assert u[np.argmax(np.abs(u[:, col])), col] > 0      # the sign rule
    assert np.allclose(u.T @ c @ u, np.diag(wv), atol=1e-9)


def test_rotation_matches_the_stand_in_recipe():
    """The input generator builds R from a seeded SPD covariance with its own
    Hadamard and eigen-ordering code; the tool, given that covariance, must
    build the same R."""
    for d in (64, 128):
        c, _, _ = synth.spd_eigenbasis(d, np.random.default_rng(11 + d))
        r_tool = cal.rotation(c)
        r_gen = synth.make_rotation(d, np.random.default_rng(11 + d))
        assert np.allclose(r_tool, r_gen, atol=1e-6)
        assert np.allclose(r_tool.T @ r_tool, np.eye(d), atol=1e-12)


def test_rotation_puts_the_dominant_query_direction_on_the_first_eigenvector():
    rng = np.random.default_rng(4)
    d = 64
    u0 = rng.standard_normal(d)
    u0 /= np.linalg.norm(u0)
    q = rng.standard_normal((500, d)) * 0.1 + np.outer(rng.standard_normal(500) * 5, u0)
    _, u = cal.eigenbasis(cal.query_covariance(q))
    assert abs(u[:, 0] @ u0) > 0.999
    # R maps the top eigenvector to a vector spread evenly over all channels (the first row of H P)
    y = u[:, 0] @ cal.rotation(cal.query_covariance(q))
    assert np.allclose(y, 1 / math.sqrt(d), atol=1e-12)


def test_clip_threshold_percentile_by_hand():
    x = np.arange(1000, dtype=np.float64).reshape(1000, 1, 1)
    rot = np.ones((1, 1, 1))
    # 99.9th percentile of 0..999 with linear interpolation: rank 0.999 * 999 = 998.001
    assert np.isclose(cal.clip_threshold(x, rot), 998.001)
    assert np.isclose(cal.clip_threshold(x, -rot, percentile=50.0), 499.5)


def test_calibrate_layer_shapes_and_properties():
    rng = np.random.default_rng(5)
    n, hq, n_kv, d = 96, 8, 2, 16
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((n, n_kv, d)) * np.where(np.arange(d) == 3, 20.0, 1.0)   # an outlier channel
    v = rng.standard_normal((n, n_kv, d))
    out = cal.calibrate_layer(q, k, v, sm_scale=1 / math.sqrt(d))
    assert out["r_k"].shape == (n_kv, d, d) and out["r_k"].dtype == np.float32
    for g in range(n_kv):
        for r in (out["r_k"][g], out["r_v"][g]):
            assert np.allclose(r.astype(np.float64).T @ r, np.eye(d), atol=1e-6)
        # C_Q of KV head g is the covariance of its own 4 query heads' rows
        assert np.allclose(out["c_q"][g], cal.query_covariance(q[:, 4 * g:4 * g + 4, :].reshape(-1, d)))
        # C_S: causal attention outputs of those heads, averaged over N*G rows
        o = np.concatenate([cal.causal_scores(q[:, 4 * g + j], k[:, g], 1 / math.sqrt(d), np.arange(n)) @ v[:, g]
                            for j in range(4)])
        assert np.allclose(out["c_s"][g], o.T @ o / (n * 4))
    # the rotation spreads the outlier channel: the threshold drops far below the outlier scale
    assert out["tau_k"] < 0.5 * np.abs(k).max()
    assert out["tau_k"] == np.float32(cal.clip_threshold(k, out["r_k"].astype(np.float64)))


def test_calibrate_layer_rejects_bad_shapes():
    with pytest.raises(ValueError):
        cal.calibrate_layer(np.zeros((4, 6, 8)), np.zeros((4, 4, 8)), np.zeros((4, 4, 8)), 0.3)
    with pytest.raises(ValueError):
        cal.hadamard(12)

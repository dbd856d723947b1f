"""Offline calibration: the fixed rotations R_K, R_V and the clip thresholds.

This is the step before the decode path, run once per model on the host
(gist.science technical summary of "OSCAR: Offline Spectral Covariance-Aware
Rotation for 2-bit KV Cache Quantization", section 2.2A, offline calibration:
covariance estimation, rotation derivation, composite rotation, clipping
thresholds; the aicoding.csdn.net explainer, section 3, item 1).  It turns
calibration activations of one layer into the inputs that
``oscar_quantize_pack`` and ``oscar_decode_attn`` take: R_K and R_V per KV
head, tau_K and tau_V per layer.  Nothing here runs during decode, and nothing
here touches the GPU.

Row-vector convention throughout: a token x (1 x d) is stored as y = x R.

* Key target: C_Q = (1/N) sum_n q_n^T q_n over the calibration queries that
  read the KV head (its G query heads, every token).  A key's quantisation
  error e enters a logit as q . (e R^T), so the query covariance, not the key
  covariance, says which directions matter.
* Value target: C_S = (1/N) (S V)^T (S V), with S the attention scores of
  those queries over the head's calibration keys (causal, each query over the
  keys up to its own position) and V the values.  A value's error reaches the
  output weighted by the scores.
* Eigenbasis U: the eigenvectors of the target, columns by descending
  eigenvalue.  Each column's sign is fixed so that its largest-magnitude entry
  is positive (any sign is a valid eigenvector; this one is reproducible).
* Composite rotation: R = U . H . P_br, with H the Sylvester Hadamard matrix
  scaled by 1/sqrt(d) and P_br the permutation that reverses the bits of the
  channel index.
* Clip threshold: a high percentile (default 99.9) of |x R| over the layer's
  rotated calibration keys (or values), every head and channel.
"""
from __future__ import annotations

import numpy as np

DEFAULT_PERCENTILE = 99.9


def hadamard(d: int) -> np.ndarray:
    """Normalised Sylvester Hadamard matrix: H[i, j] = (-1)^popcount(i & j) / sqrt(d)."""
    if d < 1 or d & (d - 1):
        raise ValueError("the Hadamard order must be a power of two")
    i = np.arange(d)
    parity = np.zeros((d, d), dtype=np.int64)
    x = i[:, None] & i[None, :]
    while x.any():
        parity ^= x & 1
        x = x >> 1
    return (1.0 - 2.0 * parity) / np.sqrt(d)


def bit_reversal(d: int) -> np.ndarray:
    """Permutation matrix P_br with P_br[i, rev(i)] = 1, rev reversing log2(d) bits."""
    if d < 1 or d & (d - 1):
        raise ValueError("bit reversal needs a power-of-two size")
    nb = d.bit_length() - 1
    rev = np.zeros(d, dtype=np.int64)
    for b in range(nb):
        rev |= ((np.arange(d) >> b) & 1) << (nb - 1 - b)
    p = np.zeros((d, d))
    p[np.arange(d), rev] = 1.0
    return p


def query_covariance(q: np.ndarray) -> np.ndarray:
    """C_Q = (1/N) sum_n q_n^T q_n for query rows q [N][d] (float64)."""
    q = np.asarray(q, dtype=np.float64).reshape(-1, np.shape(q)[-1])
    return q.T @ q / q.shape[0]


def causal_scores(q: np.ndarray, k: np.ndarray, sm_scale: float, positions=None) -> np.ndarray:
    """Softmax scores S [Nq][Nk] of queries q [Nq][d] over keys k [Nk][d].

    ``positions`` (int [Nq]) is each query's token position: it attends keys
    0..position.  None means every key."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    logits = (q @ k.T) * float(sm_scale)
    if positions is not None:
        mask = np.arange(k.shape[0])[None, :] > np.asarray(positions)[:, None]
        logits = np.where(mask, -np.inf, logits)
    logits -= logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    return w / w.sum(axis=1, keepdims=True)


def score_weighted_value_covariance(s: np.ndarray, v: np.ndarray) -> np.ndarray:
    """C_S = (1/N) (S V)^T (S V) for scores s [N][Nk] and values v [Nk][d]."""
    o = np.asarray(s, dtype=np.float64) @ np.asarray(v, dtype=np.float64)
    return o.T @ o / o.shape[0]


def eigenbasis(c: np.ndarray):
    """(eigenvalues descending, U) of a symmetric matrix, columns sign-fixed."""
    c = np.asarray(c, dtype=np.float64)
    if c.ndim != 2 or c.shape[0] != c.shape[1] or not np.allclose(c, c.T, rtol=0, atol=1e-9 * np.abs(c).max()):
        raise ValueError("the target covariance must be a symmetric square matrix")
    w, u = np.linalg.eigh((c + c.T) / 2)
    order = np.argsort(-w, kind="stable")
    w, u = w[order], u[:, order]
    lead = np.argmax(np.abs(u), axis=0)
    u = u * np.where(u[lead, np.arange(u.shape[1])] < 0, -1.0, 1.0)
    return w, u


def rotation(c: np.ndarray) -> np.ndarray:
    """R = U . H . P_br for a target covariance c (float64)."""
    d = c.shape[0]
    _, u = eigenbasis(c)
    return u @ hadamard(d) @ bit_reversal(d)


def clip_threshold(x: np.ndarray, rot: np.ndarray, percentile: float = DEFAULT_PERCENTILE) -> float:
    """Percentile of |x R| over tokens, heads and channels.

    x [N][n_kv][d] (float), rot [n_kv][d][d]; numpy's linear interpolation
    between order statistics."""
    x = np.asarray(x, dtype=np.float64)
    vals = np.concatenate([np.abs(x[:, g, :] @ np.asarray(rot[g], dtype=np.float64)).ravel()
                           for g in range(rot.shape[0])])
    return float(np.percentile(vals, percentile))


def calibrate_layer(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float,
                    percentile: float = DEFAULT_PERCENTILE, causal: bool = True) -> dict:
    """Rotations and thresholds of one layer from its calibration activations.

    q [N][Hq][d], k and v [N][n_kv][d] (float: the model's activations for N
    calibration tokens; bf16 values widened).  Query head h reads KV head
    h // (Hq / n_kv).  Returns r_k, r_v (float32 [n_kv][d][d]), tau_k, tau_v
    (float32) and the targets c_q, c_s (float64 [n_kv][d][d])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, d = q.shape
    n_kv = k.shape[1]
    if k.shape != (n, n_kv, d) or v.shape != k.shape or hq % n_kv:
        raise ValueError("q [N][Hq][d], k and v [N][n_kv][d] with Hq a multiple of n_kv")
    G = hq // n_kv
    pos = np.arange(n) if causal else None
    c_q = np.empty((n_kv, d, d))
    c_s = np.empty((n_kv, d, d))
    r_k = np.empty((n_kv, d, d))
    r_v = np.empty((n_kv, d, d))
    for g in range(n_kv):
        qg = q[:, g * G:(g + 1) * G, :]
        c_q[g] = query_covariance(qg)
        acc = np.zeros((d, d))
        for j in range(G):   # scores of each query head of the group, N rows each
            o = causal_scores(qg[:, j, :], k[:, g, :], sm_scale, pos) @ v[:, g, :]
            acc += o.T @ o
        c_s[g] = acc / (n * G)
        r_k[g] = rotation(c_q[g])
        r_v[g] = rotation(c_s[g])
    return dict(r_k=r_k.astype(np.float32), r_v=r_v.astype(np.float32),
                tau_k=np.float32(clip_threshold(k, r_k, percentile)),
                tau_v=np.float32(clip_threshold(v, r_v, percentile)), c_q=c_q, c_s=c_s)

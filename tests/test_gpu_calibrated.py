"""The calibration tool's outputs as the path's inputs: rotations and clip
thresholds calibrated on synthetic activations of the tiny layer (queries
concentrated on a few directions, keys with outlier channels), then the GPU
demotion and decode against the oracle with those same inputs."""
import math

import numpy as np
import pytest

import oracle
import synth
from bit_rotated_kv_attn_amd import calibrate as cal
from gpu_util import compare_out, compare_quant, gpu_decode, gpu_quantize

pytestmark = pytest.mark.gpu


def test_calibrated_inputs_demote_and_decode():
    cfg = dict(synth.make_decode_config(0))
    B, Hq, d = cfg["q"].shape
    n_kv = cfg["n_kv"]
    rng = np.random.default_rng(77)
    n_cal = 256
    basis = np.linalg.qr(rng.standard_normal((d, 4)))[0]          # queries live near a 4-dim subspace
    q_cal = rng.standard_normal((n_cal, Hq, 4)) @ basis.T * 3 + rng.standard_normal((n_cal, Hq, d)) * 0.2
    k_cal = synth.bf16_bits_to_f32(cfg["hist_k"][:n_cal])
    v_cal = synth.bf16_bits_to_f32(cfg["hist_v"][:n_cal])
    got = cal.calibrate_layer(q_cal, k_cal, v_cal, sm_scale=1 / math.sqrt(d))
    cfg.update(r_k=got["r_k"], r_v=got["r_v"], tau_k=got["tau_k"], tau_v=got["tau_v"])
    pools = []
    for kind in ("k", "v"):
        c = np.zeros((cfg["n_pages"], n_kv, 64 * d // 4), np.uint8)
        s = np.zeros((cfg["n_pages"], n_kv, 64, 2), np.uint16)
        diag = oracle.quantize_pack_ref(kind, cfg["hist_" + kind], cfg["r_" + kind], cfg["tau_" + kind],
                                        cfg["hist_slot"], c, s)
        gc, gs = gpu_quantize(kind, cfg["hist_" + kind], cfg["r_" + kind], cfg["tau_" + kind], cfg["hist_slot"],
                              cfg["n_pages"])
        compare_quant(kind, gc, gs, c, s, diag, d)
        pools.append((c, s))
    (kc, ks), (vc, vs) = pools
    ref = oracle.decode_attn_ref(cfg, kc, vc, ks, vs)
    compare_out(gpu_decode(cfg, (kc, vc, ks, vs)), ref, what="calibrated tiny layer")

"""Oracle pins: rotate -> clip -> INT2 quantise -> pack."""
import numpy as np
import pytest

import oracle
import pins


def test_closed_forms():
    pins.check_quant_closed_forms()


@pytest.mark.parametrize("seed", [3, 31])
def test_bruteforce_exact_arithmetic(seed):
    pins.check_quant_bruteforce(seed=seed)


def test_pack_literals():
    pins.check_pack_literals()


def test_layout_literals():
    pins.check_layout_literals()


def test_column_permutation_invariance():
    pins.check_column_permutation_invariance()


def test_slots_and_scatter():
    pins.check_quantize_pack_slots()


@pytest.mark.parametrize("clip", [0.0, -1.0, float("nan"), float("inf"), 70000.0])
def test_invalid_clip_rejected(clip):
    x = np.zeros((1, 1, 16), np.uint16)
    with pytest.raises(ValueError):
        oracle.quantize_pack_ref("k", x, np.eye(16, dtype=np.float32)[None], clip, np.zeros(1, np.int32),
                                 np.zeros((1, 1, 256), np.uint8), np.zeros((1, 1, 64, 2), np.uint16))


def test_dequant_error_bound():
    """|y_c - x_hat| <= scale/2 + |zero - min| + 3 |scale - range/3| (+ fp32 slack)."""
    rng = np.random.default_rng(21)
    y = (rng.standard_normal((500, 128)) * 4).astype(np.float32)
    codes, s16, z16, info = oracle.quantize_group(y, 9.0)
    s = oracle.f16_bits_to_f64(s16)[:, None]
    z = oracle.f16_bits_to_f64(z16)[:, None]
    xh = z + codes * s
    bound = s / 2 + np.abs(z - info["mn"][:, None]) + 3 * np.abs(s - info["range3"][:, None]) + 1e-5
    assert np.all(np.abs(info["yc"] - xh) <= bound)

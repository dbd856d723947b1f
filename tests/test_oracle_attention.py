"""Oracle pins: three-segment decode attention."""
import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("rot", ["orth", "signed_perm", "identity"])
def test_decode_vs_torch_sdpa(rot):
    pins.check_decode_vs_sdpa(rot=rot)


def test_inverse_rotation_direction():
    pins.check_inverse_rotation_direction()


def test_rotated_space_identity():
    pins.check_rotated_space_identity()


def test_special_cases():
    pins.check_decode_special_cases()


def test_invariances():
    pins.check_decode_invariances()


def test_partition_merge():
    pins.check_partition_merge()


def test_bf16_paged_vs_sdpa():
    pins.check_bf16_paged_vs_sdpa()


def test_bad_page_and_lengths_raise():
    cfg, pools, _ = pins.make_small_cache(seed=30)
    t = cfg["block_table"].copy()
    t[0, 0] = pools[0].shape[0]
    with pytest.raises(ValueError):
        oracle.decode_attn_ref(cfg, *pools, block_table=t)
    with pytest.raises(ValueError):
        oracle.decode_attn_ref(cfg, *pools, sink_len=np.array([7, 0], np.int32))

"""Checks the Python binding makes before any pointer reaches the library
(CPU): scale/zero pools must match the declared quantisation groups, since
the library cannot see a pool's shape and a grouped call writes two pairs
per (token, head)."""
import pytest
import torch

import bit_rotated_kv_attn_amd as hip


def _decode_kw(group_channels, sz_pairs):
    B, Hq, n_kv, d = 1, 8, 2, 128
    f = lambda *s, dt=torch.int16: torch.zeros(s, dtype=dt)
    return dict(q=f(B, Hq, d), sink_k=f(B, n_kv, 64, d), sink_v=f(B, n_kv, 64, d), recent_k=f(B, n_kv, 256, d),
                recent_v=f(B, n_kv, 256, d), sink_len=f(B, dt=torch.int32), recent_len=f(B, dt=torch.int32),
                hist_len=f(B, dt=torch.int32), max_hist_len=64, k_codes=f(4, n_kv, 2048, dt=torch.uint8),
                v_codes=f(4, n_kv, 2048, dt=torch.uint8), k_sz=f(4, n_kv, sz_pairs, 2), v_sz=f(4, n_kv, sz_pairs, 2),
                block_table=f(B, 1, dt=torch.int32), r_k=f(n_kv, d, d, dt=torch.float32),
                r_v=f(n_kv, d, d, dt=torch.float32), out=f(B, Hq, d, dt=torch.float32),
                workspace=f(256, dt=torch.uint8), group_channels=group_channels)


@pytest.mark.parametrize("group_channels,sz_pairs", [(64, 64), (0, 128), (32, 128), (64, 256)])
def test_decode_args_rejects_pools_of_the_other_grouping(group_channels, sz_pairs):
    with pytest.raises(ValueError, match="k_sz must be"):
        hip.decode_args(**_decode_kw(group_channels, sz_pairs))


@pytest.mark.parametrize("group_channels,sz_pairs", [(64, 128), (0, 64), (32, 256)])
def test_decode_args_accepts_matching_pools(group_channels, sz_pairs):
    # the shape checks pass; the pointer check then refuses host tensors
    with pytest.raises(ValueError, match="device tensor"):
        hip.decode_args(**_decode_kw(group_channels, sz_pairs))


def test_quantize_pack_checks_the_pool_against_the_kind():
    x = torch.zeros((3, 2, 128), dtype=torch.int16)
    rot = torch.zeros((2, 128, 128))
    codes = torch.zeros((4, 2, 2048), dtype=torch.uint8)
    slot = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="pool shapes"):
        hip.oscar_quantize_pack(hip.KIND_K | hip.GROUPS_64, x, rot, 1.0, slot, codes, torch.zeros((4, 2, 64, 2)))
    with pytest.raises(ValueError, match="pool shapes"):
        hip.oscar_quantize_pack(hip.KIND_K, x, rot, 1.0, slot, codes, torch.zeros((4, 2, 128, 2)))
    with pytest.raises(ValueError, match="pool shapes"):
        hip.oscar_quantize_pack(hip.KIND_K | hip.GROUPS_32, x, rot, 1.0, slot, codes, torch.zeros((4, 2, 128, 2)))


def test_decode_step_checks_the_demotion_pools_against_the_groups():
    a = hip.DecodeArgs(head_dim=128, group_channels=64)
    dk = hip.DemoteArgs()
    dk.sz_pairs = 64                      # a whole-head pool, but the step writes two pairs per token
    with pytest.raises(ValueError, match="demote_k"):
        hip.oscar_decode_step(args=(a, None, 0), demote_k=dk)
    a32 = hip.DecodeArgs(head_dim=128, group_channels=32)
    dk.sz_pairs = 128                     # a 64-channel pool, but the step writes four pairs per token
    with pytest.raises(ValueError, match="demote_k"):
        hip.oscar_decode_step(args=(a32, None, 0), demote_k=dk)


def test_groups_per_head():
    assert [hip.groups_per_head(128, g) for g in (0, 64, 32, 128)] == [1, 2, 4, 1]
    assert [hip.groups_per_head(64, g) for g in (0, 64, 32)] == [1, 1, 2]
    assert [hip.kind_group_channels(k) for k in (hip.KIND_V, hip.KIND_K | hip.GROUPS_64, hip.GROUPS_32)] == [0, 64, 32]

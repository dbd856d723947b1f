"""Shared-prefix packing of the history scan (group size 4): the splits that
lie inside a declared shared prefix are read once for each pack of requests,
four per wave (uniform codebook, whole-head groups, d = 128, batches of four
or more) or two per wave (otherwise).  Parity with the oracle on ragged
private parts, requests past the last whole pack and two split partitions;
the pack checks (rows that differ inside the prefix, a history shorter than
the prefix) that turn exactly that pack's rows into NaN; and group sizes that
ignore the declaration."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import compare_out, gpu_decode, oracle_pools

pytestmark = pytest.mark.gpu


def prefix_cache(seed_index, B, G, d, hist_pages, shared, n_kv=2, tail=37):
    """B requests whose first `shared` history pages are the same physical
    pages; request b's history is `tail + 3b` tokens shorter than the full
    hist_pages (ragged last pages, all beyond the prefix)."""
    ctx = 64 + 256 + 64 * hist_pages
    shape = synth.DecodeShape(f"prefix-b{B}-g{G}-d{d}", B, n_kv * G, n_kv, d, ctx, shared_hist_pages=shared)
    cfg = synth.make_decode_config(0, shape=shape, seed_index=40 + seed_index)
    pools = oracle_pools(cfg)
    hl = cfg["hist_len"].copy()
    hl -= (tail + 3 * np.arange(B)).astype(np.int32)
    assert hl.min() >= 64 * shared
    cfg["hist_len"] = hl
    return cfg, pools


@pytest.mark.parametrize("B", [2, 3, 5])
@pytest.mark.parametrize("d", [64, 128])
def test_prefix_pairs_match_oracle(B, d):
    cfg, pools = prefix_cache(B, B, 4, d, hist_pages=21, shared=13)
    ref = oracle.decode_attn_ref(cfg, *pools)
    got = gpu_decode(cfg, pools, shared_pages=13)
    compare_out(got, ref, what=f"prefix pairs B={B} d={d}")
    plain = gpu_decode(cfg, pools)
    compare_out(plain, ref, what=f"no prefix declared B={B} d={d}")


def test_prefix_pairs_other_partition():
    """A larger max_hist_len gives several pages per split: only the splits
    wholly inside the prefix are packed, the one across its end is not."""
    cfg, pools = prefix_cache(7, 4, 4, 128, hist_pages=40, shared=29)
    ref = oracle.decode_attn_ref(cfg, *pools)
    wide = np.full((4, 200), -1, np.int32)
    wide[:, : cfg["block_table"].shape[1]] = cfg["block_table"]
    got = gpu_decode(cfg, pools, block_table=wide, max_hist_len=64 * 200, shared_pages=29)
    compare_out(got, ref, what="prefix pairs, wide partition")


def test_declared_prefix_shorter_than_shared_part():
    """Declaring fewer pages than are shared is fine (the rest is read per request)."""
    cfg, pools = prefix_cache(8, 3, 4, 128, hist_pages=21, shared=13)
    ref = oracle.decode_attn_ref(cfg, *pools)
    for declared in (1, 6, 12):
        compare_out(gpu_decode(cfg, pools, shared_pages=declared), ref, what=f"declared {declared}")


def test_mismatched_rows_poison_the_pair():
    cfg, pools = prefix_cache(9, 3, 4, 128, hist_pages=21, shared=13)
    ref = oracle.decode_attn_ref(cfg, *pools)
    table = cfg["block_table"].copy()
    table[1, 4] = table[1, 15]                   # request 1 leaves the prefix at page 4
    got = gpu_decode(cfg, pools, block_table=table, shared_pages=13)
    assert np.all(np.isnan(got[0])) and np.all(np.isnan(got[1]))
    compare_out(got[2:], ref[2:], what="request outside the pair")


def test_short_history_poisons_the_pair():
    cfg, pools = prefix_cache(10, 3, 4, 128, hist_pages=21, shared=13)
    ref = oracle.decode_attn_ref(cfg, *pools)
    hl = cfg["hist_len"].copy()
    hl[1] = 64 * 13 - 5                          # ends inside the declared prefix
    got = gpu_decode(cfg, pools, hist_len=hl, shared_pages=13)
    assert np.all(np.isnan(got[0])) and np.all(np.isnan(got[1]))
    compare_out(got[2:], ref[2:], what="request outside the pair")


@pytest.mark.parametrize("G", [1, 2, 8])
def test_other_group_sizes_ignore_the_prefix(G):
    cfg, pools = prefix_cache(11 + G, 2, G, 128, hist_pages=21, shared=13)
    base = gpu_decode(cfg, pools)
    compare_out(base, oracle.decode_attn_ref(cfg, *pools), what=f"G={G}")
    assert np.array_equal(gpu_decode(cfg, pools, shared_pages=13), base)


@pytest.mark.parametrize("B", [4, 6, 8, 11])
def test_prefix_quads_match_oracle(B):
    """Four requests per wave: whole packs, and one to three requests past the
    last whole pack read on their own."""
    cfg, pools = prefix_cache(20 + B, B, 4, 128, hist_pages=21, shared=13)
    ref = oracle.decode_attn_ref(cfg, *pools)
    compare_out(gpu_decode(cfg, pools, shared_pages=13), ref, what=f"prefix quads B={B}")


@pytest.mark.parametrize("codebook,groups", [("lloyd_max", 0), ("uniform", 64), ("uniform", 32)])
def test_prefix_pairs_for_other_formats(codebook, groups):
    """The Lloyd-Max codebook and 64- or 32-channel groups pack two requests
    per wave even in batches of four or more."""
    from gpu_util import oracle_pools as pools_of
    ctx = 64 + 256 + 64 * 21
    shape = synth.DecodeShape("prefix-fmt-b5", 5, 8, 2, 128, ctx, shared_hist_pages=13)
    cfg = synth.make_decode_config(0, shape=shape, seed_index=60 + groups)
    cfg["codebook"] = codebook
    cfg["group_channels"] = groups
    pools = pools_of(cfg)
    ref = oracle.decode_attn_ref(cfg, *pools)
    compare_out(gpu_decode(cfg, pools, shared_pages=13), ref, what=f"prefix {codebook} groups {groups}")


def test_mismatched_rows_poison_the_quad():
    cfg, pools = prefix_cache(30, 6, 4, 128, hist_pages=21, shared=13)
    ref = oracle.decode_attn_ref(cfg, *pools)
    table = cfg["block_table"].copy()
    table[2, 7] = table[2, 16]                   # request 2 leaves the prefix at page 7
    got = gpu_decode(cfg, pools, block_table=table, shared_pages=13)
    assert np.all(np.isnan(got[:4]))
    compare_out(got[4:], ref[4:], what="requests outside the quad")


def test_short_history_poisons_the_quad():
    cfg, pools = prefix_cache(31, 5, 4, 128, hist_pages=21, shared=13)
    ref = oracle.decode_attn_ref(cfg, *pools)
    hl = cfg["hist_len"].copy()
    hl[3] = 64 * 13 - 9                          # ends inside the declared prefix
    got = gpu_decode(cfg, pools, hist_len=hl, shared_pages=13)
    assert np.all(np.isnan(got[:4]))
    compare_out(got[4:], ref[4:], what="request outside the quad")

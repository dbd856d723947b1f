"""Shared-prefix packing of the history scan (group size 4): the splits that
lie inside a declared shared prefix are read once for each pack of requests,
four per wave (uniform codebook, whole-head groups, d = 128, batches of four
or more) or two per wave (otherwise); on request (prefix_cascade), with
sixteen requests or more and a prefix of at least 64 pages, once for each
group of up to four packs (cascade blocks).  Parity with the oracle on ragged
private parts, requests past the last whole pack and two split partitions;
the pack checks (rows that differ inside the prefix, a history shorter than
the prefix) that turn exactly that pack's rows into NaN; and group sizes and
sizes that ignore the declaration or the request."""
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


@pytest.mark.parametrize("B", [16, 19, 24])
def test_prefix_cascade_matches_oracle(B):
    """Sixteen requests or more with a prefix of at least 64 pages: the splits
    inside it run as cascade blocks, each page staged once for a group of up
    to four packs (16 requests).  B = 19 leaves three requests past the last
    whole pack; B = 24 gives a second group with two packs and two idle waves.
    Without the request the same launch reads the prefix in packs."""
    cfg, pools = prefix_cache(50 + B, B, 4, 128, hist_pages=80, shared=70)
    ref = oracle.decode_attn_ref(cfg, *pools)
    compare_out(gpu_decode(cfg, pools, shared_pages=70, prefix_cascade=True), ref, what=f"cascade B={B}")
    compare_out(gpu_decode(cfg, pools, shared_pages=70), ref, what=f"packs B={B}")


@pytest.mark.parametrize("B,shared,codebook", [(15, 70, "uniform"), (16, 63, "uniform"), (16, 70, "lloyd_max")])
def test_cascade_request_ignored_where_it_does_not_apply(B, shared, codebook):
    """Fewer than 16 requests, a prefix shorter than one cascade split, or the
    Lloyd-Max codebook: the request changes nothing, bit for bit."""
    cfg, pools = prefix_cache(70 + B + shared, B, 4, 128, hist_pages=80, shared=shared)
    if codebook != "uniform":
        from gpu_util import oracle_pools as pools_of
        cfg["codebook"] = codebook
        pools = pools_of(cfg)
    base = gpu_decode(cfg, pools, shared_pages=shared)
    compare_out(base, oracle.decode_attn_ref(cfg, *pools), what=f"B={B} shared={shared} {codebook}")
    assert np.array_equal(gpu_decode(cfg, pools, shared_pages=shared, prefix_cascade=True), base)


def test_mismatched_row_poisons_the_cascade_group():
    cfg, pools = prefix_cache(60, 20, 4, 128, hist_pages=80, shared=70)
    ref = oracle.decode_attn_ref(cfg, *pools)
    table = cfg["block_table"].copy()
    table[6, 30] = table[6, 75]                  # request 6 (group 0) leaves the prefix at page 30
    got = gpu_decode(cfg, pools, block_table=table, shared_pages=70, prefix_cascade=True)
    assert np.all(np.isnan(got[:16]))
    compare_out(got[16:], ref[16:], what="requests outside the poisoned group")


def test_short_history_poisons_the_cascade_group():
    cfg, pools = prefix_cache(61, 20, 4, 128, hist_pages=80, shared=70)
    ref = oracle.decode_attn_ref(cfg, *pools)
    hl = cfg["hist_len"].copy()
    hl[17] = 64 * 30 - 5                         # request 17 (group 1: requests 16-19) ends inside the prefix
    got = gpu_decode(cfg, pools, hist_len=hl, shared_pages=70, prefix_cascade=True)
    assert np.all(np.isnan(got[16:]))
    compare_out(got[:16], ref[:16], what="requests outside the poisoned group")

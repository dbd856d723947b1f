"""Host-side helpers of bench.py (CPU): the algorithmic byte count counts a
shared physical page once, and every request gets a free slot for the token
a decode step demotes."""
import numpy as np

import bench
import synth


def test_unique_tokens_counts_shared_pages_once():
    table = np.array([[5, 7, 9], [5, 7, 2], [5, 1, -1]], np.int32)
    lens = np.array([64 * 2 + 10, 64 * 3, 64 + 3])
    # page 5 full (all three), page 7 full, page 9: 10 tokens, page 2: 64, page 1: 3
    assert bench.unique_tokens(table, lens) == 64 + 64 + 10 + 64 + 3
    assert bench.unique_tokens(table[:1], lens[:1]) == int(lens[0])


def test_unique_tokens_of_the_shared_prefix_workload():
    cfg = synth.make_decode_config(4, materialize_history=False)
    shared = cfg["shape"].shared_hist_pages
    private = cfg["shape"].hist_len - 64 * shared
    assert bench.unique_tokens(cfg["block_table"], cfg["hist_len"]) == 64 * shared + cfg["batch"] * private


def test_ensure_free_slot_appends_pages_only_where_needed():
    shape = synth.DecodeShape("t", 3, 4, 2, 64, 64 + 256 + 64 * 4)   # history ends on a page boundary
    cfg = synth.make_decode_config(0, shape=shape, materialize_history=False)
    out = bench.ensure_free_slot(cfg)
    assert out["block_table"].shape[1] == cfg["block_table"].shape[1] + 1
    assert out["n_pages"] == cfg["n_pages"] + 3
    nxt = out["hist_len"]
    slots = out["block_table"][np.arange(3), nxt // 64]
    assert np.all(slots >= cfg["n_pages"]) and len(set(slots.tolist())) == 3
    shape2 = synth.DecodeShape("t2", 2, 4, 2, 64, 64 + 256 + 64 * 4 + 5)
    cfg2 = synth.make_decode_config(0, shape=shape2, materialize_history=False)
    assert bench.ensure_free_slot(cfg2) is cfg2

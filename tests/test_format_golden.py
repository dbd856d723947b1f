"""The storage format against the numbers the pages print (tests/golden)."""
import json
import os

import numpy as np

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_format_numbers.json")))


def bits_per_element(L, d=128):
    """Average stored bits per K/V element of one head for a context of L
    tokens: INT2 history (codes + fp16 scale and zero per token-head) plus
    the BF16 sink and recent windows."""
    n_bf16 = min(L, GOLD["sink_tokens"]["value"] + GOLD["recent_tokens"]["value"])
    hist = L - n_bf16
    hist_bytes_per_token = oracle.page_block_bytes(d) / oracle.PAGE + 2 * 2   # codes + fp16 scale + fp16 zero
    return (hist * hist_bytes_per_token * 8 + n_bf16 * d * 16) / (L * d)


def test_codes_per_byte():
    c = np.array([3, 0, 1, 2] * 4, np.uint8)
    assert oracle.pack_codes_row(c).size * GOLD["codes_per_byte"]["value"] == c.size


def test_effective_bits_match_pages():
    for key in ("effective_bits_general", "effective_bits_qwen3_8b_32k"):
        g = GOLD[key]
        assert round(bits_per_element(g["context_tokens"]), g["digits"]) == g["value"], key


def test_memory_reduction():
    bf16 = GOLD["bf16_bytes_per_channel_kv"]["value"]
    int2 = GOLD["int2_bytes_per_channel_kv"]["value"]
    codes_only = 2 * oracle.page_block_bytes(128) / oracle.PAGE / 128   # K and V code bytes per channel
    assert codes_only == int2
    assert bf16 / int2 == GOLD["memory_reduction_vs_bf16"]["value"]

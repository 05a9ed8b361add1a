"""Numbers the pages print (tests/golden/page_numbers.json) against the oracle's accounting."""

import json
import math
import os

import numpy as np

from oracle import dgq_oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def test_memory_formula_identifier_overhead():
    """DGQ article 3.3: the 1-bit identifier costs about 17 MB at 128K for Llama-3-8B."""
    g = GOLD["dgq_memory_formula"]
    inp = g["inputs"]
    fp16, dgq = O.page_formula_bytes(inp["num_layers"], inp["num_heads"], inp["head_dim"], inp["seq_len"])
    ident = dgq - 2 * inp["num_layers"] * inp["num_heads"] * inp["head_dim"] * inp["seq_len"]
    assert round(ident / 1e6) == g["printed_identifier_overhead_MB"]
    # the layout the library uses stores exactly the formula's bytes (codes + bits), per layer
    per_layer = O.compressed_bytes([inp["seq_len"]], inp["num_heads"], inp["head_dim"])
    assert (per_layer["codes"] + per_layer["bits"]) * inp["num_layers"] == dgq


def test_memory_formula_ratio_is_two_not_four():
    """The printed 4.02:1 contradicts the printed formula: INT8 codes of fp16 values save at most
    2:1.  The formula itself gives 1.999:1; the reading used throughout is the formula."""
    g = GOLD["dgq_memory_formula"]
    inp = g["inputs"]
    fp16, dgq = O.page_formula_bytes(inp["num_layers"], inp["num_heads"], inp["head_dim"], inp["seq_len"])
    ratio = fp16 / dgq
    assert 1.99 < ratio < 2.0
    assert abs(ratio - g["printed_ratio"]) > 1.0
    assert g["printed_fp16_GB"] / g["printed_dgq_GB"] > 4.0  # what the page claims instead


def test_kv_bytes_per_token():
    """PagedAttention article: 4096/32*2 = 256 B per layer, head and token (one of K or V),
    8 KB over 32 layers, 8 MB per 1000 tokens."""
    g = GOLD["kv_bytes_per_token"]
    head_dim = g["d_model"] // g["n_head"]
    fp16_one_head_one_token, _ = O.page_formula_bytes(1, 1, head_dim, 1)
    per_tensor = fp16_one_head_one_token // 2           # the formula counts K and V
    assert per_tensor == g["printed_bytes_per_layer_head_token"]
    assert per_tensor * g["num_layers"] == g["printed_KB_all_layers"] * 1024
    assert round(per_tensor * g["num_layers"] * g["tokens"] / 1e6) == g["printed_MB_for_tokens"]


def test_window_and_segment_constants():
    g = GOLD["dgq_window_and_segments"]
    assert O.WIN == g["win_size"]
    assert O.MAX_SEGMENTS == g["segments_max"]
    # with the forced first cut a sequence of >= 32 tokens has at least 2 segments; the page's
    # lower bound of 3 is not forced (see the design notes: 2..5)
    x = np.zeros((64, 8), np.float16)
    assert len(O.segment_starts(x)) >= 2
    hc = O.compress_head(x, x)
    assert hc.bits.size == 64 * g["identifier_bits_per_token"]


def test_length_aware_rule_constants():
    """DGQ article 3.2 length-aware group counts (kept for the segment-count policies)."""
    g = GOLD["length_aware_groups"]

    def n_groups(length):
        if length < g["printed_threshold_short"]:
            return g["printed_groups_short"]
        if length < g["printed_threshold_mid"]:
            return g["printed_groups_mid"]
        return min(g["printed_cap"], int(math.log2(length / g["printed_log_base"])) + g["printed_offset"])

    assert n_groups(2047) == 2 and n_groups(2048) == 3 and n_groups(16383) == 3
    assert n_groups(16384) == 5 and n_groups(131072) == 5

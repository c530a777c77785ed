"""The work accounting the bench prices rooflines on, pinned to the pages' printed figures
(tests/golden/pages_figures.json, each entry citing its page and item) and to brute force."""
import json
from pathlib import Path

import numpy as np
import pytest

from transformer_attention_varlen_amd import metrics

FIG = json.loads((Path(__file__).parent / "golden" / "pages_figures.json").read_text())


def test_kv_append_bytes_match_the_page():
    f = FIG["kv_append_bytes_per_tensor_per_layer"]
    assert metrics.kv_row_bytes(f["geometry"]["kv_heads"]) == f["value"]


def test_kv_concat_bytes_match_the_page():
    f = FIG["kv_concat_bytes_per_token_at_1142"]
    g = f["geometry"]
    b = metrics.kv_concat_bytes_per_token(g["kv_heads"], g["position"], g["layers"])
    assert round(b / 1e6, 1) == f["value_mb"]


def test_score_matrix_size_matches_the_page():
    f = FIG["score_matrix_elements_at_1142"]
    e = metrics.score_matrix_elements(f["geometry"]["heads"], f["geometry"]["seq"])
    assert round(e / 1e6, 1) == f["value_millions"]
    assert round(e * 4 / 1e6, 1) == f["bytes_mb"]


def test_repeat_kv_size_matches_the_page():
    f = FIG["repeat_kv_copy_mb"]
    g = f["geometry"]
    assert round(g["heads"] * g["seq"] * g["head_dim"] * 4 / 1e6, 1) == f["value_mb"]


@pytest.mark.parametrize("window,causal", [(-1, False), (-1, True), (0, False), (5, False),
                                           (128, False), (9, True)])
def test_visible_pairs_by_brute_force(window, causal):
    lengths = [1, 7, 64, 130, 0]
    brute = 0
    for n in lengths:
        for i in range(n):
            for j in range(n):
                ok = (window < 0 or abs(i - j) <= window // 2) and (not causal or j <= i)
                brute += ok
    assert metrics.visible_pairs_per_head(lengths, window, causal) == brute


def test_pair_counts_of_closed_forms():
    # global: n^2; causal: n(n+1)/2; window w=128 on n >= 65: 129 n - 64*65
    assert metrics.visible_pairs_per_head([37, 91]) == 37 ** 2 + 91 ** 2
    assert metrics.visible_pairs_per_head([2048] * 16, causal=True) == 16 * 2048 * 2049 // 2
    assert metrics.visible_pairs_per_head([512], window=128) == 129 * 512 - 64 * 65


def test_decode_bytes():
    used = np.array([1143, 8192])
    b = metrics.decode_bytes(used, 9, 3)
    assert b == 1536 * (1142 + 8191) + 2 * (9 * 256 + 4 * 768 + 9 * 256)


def test_chunk_pairs_count_every_visible_cache_row():
    # brute force over the rows: query i of a chunk after `off` filled rows sees off + i + 1 keys
    lengths, offsets = [3, 0, 7, 1], [0, 5, 12, 99]
    brute = sum(o + i + 1 for n, o in zip(lengths, offsets) for i in range(n))
    assert metrics.chunk_pairs_per_head(lengths, offsets) == brute
    assert metrics.chunk_flops(lengths, offsets, 9) == 256 * 9 * brute

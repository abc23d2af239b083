"""The few numbers the pages print for the stored format, checked against the
oracle's grouping and storage accounting (fixture: tests/golden/pages_numbers.json)."""
import json
import os

import pytest

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
PAGES = json.load(open(os.path.join(HERE, "golden", "pages_numbers.json")))


def test_group_count_example():
    ex = PAGES["group_count_example"]
    assert O.n_groups_total(ex["rows"], ex["cols"], ex["group_size"]) == ex["groups"]


@pytest.mark.parametrize("case", PAGES["compression_vs_fp16"]["cases"])
def test_compression_ratio(case):
    tol = PAGES["compression_vs_fp16"]["relative_tolerance"]
    ratio = 16.0 / O.storage_bits_per_weight(case["bits"], case["group_size"])
    assert abs(ratio / case["ratio"] - 1.0) <= tol


def test_packed_words_per_column():
    # dense b-bit storage: in*b/32 int32 words per output channel
    import numpy as np
    for bits in (2, 3, 4, 8):
        q = O.pack(np.zeros((2, 64), dtype=np.int64), bits)
        assert q.shape == (64 * bits // 32, 2)

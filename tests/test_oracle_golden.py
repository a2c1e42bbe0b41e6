"""Pin of the oracle's select + paged compaction against the memory ratios the pages print.

Budgeted selection keeps exactly B of L tokens and forward packing frees every page past
ceil(B / page); the fraction of pages still held must reproduce the printed ratios
(tests/golden/memory_ratios.json, each entry with its citation).
"""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "memory_ratios.json")


def _pages_after_compaction(L, B, page, window=128, seed=0):
    rng = np.random.default_rng(seed)
    n_pages = -(-L // page)
    pool = np.arange(n_pages * page, dtype=np.float64).reshape(n_pages, 1, 1, page, 1)
    bt = rng.permutation(n_pages)
    kept = oracle.select_top_b(rng.standard_normal(L), L, B, window)
    _, _, freed, new_len = oracle.compact_paged_sequence(pool, None, bt, L, {(0, 0): kept}, page)
    assert new_len == len(kept) == min(B, L)
    return n_pages - len(freed), n_pages


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_printed_memory_ratios(case):
    held, total = _pages_after_compaction(case["context_tokens"], case["budget"], case["page"])
    frac = held / total
    if "printed_memory_fraction" in case:
        assert abs(frac - case["printed_memory_fraction"]) <= case["fraction_tolerance"]
        assert abs(1.0 / frac - case["printed_reduction"]) <= case["reduction_tolerance"]
    if "printed_compression" in case:
        assert abs(total / held - case["printed_compression"]) <= case["compression_tolerance"]

"""The oracle's reporting formulas against the values the pages print
(tests/golden/formulas.json, each entry cited)."""
import json
import os

import pytest

from oracle import formulas

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "formulas.json")))


@pytest.mark.parametrize("case", GOLD["layer_skip_speedup_c0.3"]["cases"])
def test_layer_skip_optima(case):
    c = GOLD["layer_skip_speedup_c0.3"]["c"]
    sp = {k: formulas.speedup_layer_skip(case["alpha"], k, c) for k in range(1, 13)}
    best = max(sp, key=sp.get)
    if "best_k" in case:
        assert best in case["best_k"]
        assert abs(sp[best] - case["speedup_approx"]) < 0.03
    else:
        assert max(sp.values()) < case["max_speedup_below"]


def test_expected_tokens_limits():
    assert formulas.expected_tokens(0.0, 5) == 1.0
    assert formulas.expected_tokens(1.0, 5) == 6.0
    # E(k) is the sum of alpha^i for i = 0..k
    assert abs(formulas.expected_tokens(0.5, 3) - (1 + 0.5 + 0.25 + 0.125)) < 1e-15


@pytest.mark.parametrize("case", GOLD["block_speedup"]["cases"])
def test_block_speedup(case):
    s = formulas.speedup_block(case["a"], case["K"], case["t_over_T"])
    assert abs(s - case["speedup_approx"]) < 0.005


@pytest.mark.parametrize("row", GOLD["tree_batch_sizes"]["rows"])
def test_tree_table_batch_identity(row):
    assert row["K"] * (row["M"] + 1) == row["batch"]


def test_k_schedule():
    assert formulas.next_k(0.2, 2, 16, 0.3, 0.7) == 2
    assert formulas.next_k(0.9, 2, 16, 0.3, 0.7) == 16
    assert formulas.next_k(0.5, 2, 16, 0.3, 0.7) == 9
    assert abs(formulas.confidence(0.5, 0.1, 0.5) - (0.2 + 0.15 + 0.15)) < 1e-15

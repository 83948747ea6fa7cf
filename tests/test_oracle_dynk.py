"""The windowed dynamic draft length and its context-cost cut-off
(self-speculative decoding page, §3.2 and §5.3): the oracle against closed
forms and the page's own speedup table, and the library's host controller
against the oracle, decision for decision."""
import json
import os

import numpy as np
import pytest

from oracle import spec

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "formulas.json")))


def test_window_counts_only_the_last_rounds():
    st = spec.DynKState(4)
    for _ in range(70):
        spec.dynk_update(st, 1, 4)
    for _ in range(10):
        spec.dynk_update(st, 3, 4)
    # the window holds 54 rounds of 1/4 and 10 of 3/4
    assert len(st.window) == 64
    assert st.alpha == (54 * 1 + 10 * 3) / (64 * 4)


def test_additive_steps_and_clamps():
    up = spec.DynKState(2)
    ks = [spec.dynk_update(up, 5, 5) for _ in range(10)]  # alpha = 1 > 0.85 every round
    assert ks == [3, 4, 5, 6, 7, 8, 8, 8, 8, 8]
    down = spec.DynKState(8)
    ks = [spec.dynk_update(down, 0, 4) for _ in range(10)]  # alpha = 0 < 0.7
    assert ks == [7, 6, 5, 4, 3, 2, 2, 2, 2, 2]
    mid = spec.DynKState(5)
    assert [spec.dynk_update(mid, 4, 5) for _ in range(5)] == [5] * 5  # alpha = 0.8: no change


def test_no_draft_round_leaves_the_window():
    st = spec.DynKState(5)
    spec.dynk_update(st, 2, 5)
    before = (list(st.window), st.alpha, st.k)
    spec.dynk_update(st, 0, 0)
    assert (st.window, st.alpha, st.k) == before


@pytest.mark.parametrize("case", GOLD["layer_skip_speedup_c0.3"]["cases"])
def test_context_rule_follows_the_speedup_table(case):
    """With the page's c = 0.3 the cut-off picks the page's optimal k; at
    alpha = 0.6, where no k reaches 1.3x and longer drafts lose, the best k is
    1, below min_k, so drafting is turned off."""
    c = GOLD["layer_skip_speedup_c0.3"]["c"]
    st = spec.DynKState(8, alpha=case["alpha"])
    k = spec.dynk_update(st, 0, 0, c_draft=c)
    if "best_k" in case:
        assert k in case["best_k"], (case, k)
    else:
        assert k == 0, (case, k)


def test_context_rule_turns_drafting_off_when_it_cannot_pay():
    st = spec.DynKState(8, alpha=0.6)
    assert spec.dynk_update(st, 0, 0, c_draft=0.9) == 0
    st = spec.DynKState(8, alpha=0.0)
    assert spec.dynk_update(st, 0, 0, c_draft=0.05) == 0
    st = spec.DynKState(6, alpha=1.0)
    assert spec.dynk_update(st, 0, 0, c_draft=0.3) == 6  # alpha = 1: the controller's k is the limit


def test_library_controller_matches_oracle():
    from verification_verify_step_amd import binding as B
    cfg = B.dynk_cfg()
    rng = np.random.default_rng(11)
    for trial in range(10):
        k0 = int(rng.integers(1, 12))
        lib = B.vs_dynk_init(cfg, k0)
        ora = spec.DynKState(max(2, min(8, k0)))
        assert lib.k == ora.k
        k_next = ora.k
        for r in range(150):
            k_used = k_next if k_next > 0 else (0 if rng.random() < 0.5 else int(rng.integers(1, 9)))
            bias = rng.random()
            a = int(rng.binomial(k_used, bias)) if k_used else 0
            c = float(rng.choice([0.0, 0.1, 0.3, 0.5, 0.9]))
            k_lib = B.vs_dynk_update(cfg, lib, a, k_used, c)
            k_next = spec.dynk_update(ora, a, k_used, c)
            assert (k_lib, lib.k, lib.alpha) == (k_next, ora.k, ora.alpha), (trial, r)


def test_library_controller_rejects_bad_input():
    from verification_verify_step_amd import binding as B
    cfg = B.dynk_cfg()
    st = B.vs_dynk_init(cfg, 4)
    for a, k in ((5, 4), (-1, 4), (0, -1)):
        with pytest.raises(B.VsError):
            B.vs_dynk_update(cfg, st, a, k)
    assert st.n == 0 and st.k == 4
    for bad in (B.dynk_cfg(window=0), B.dynk_cfg(window=B.VS_DYNK_MAX_WINDOW + 1), B.dynk_cfg(min_k=3, max_k=2),
                B.dynk_cfg(up=0.6, down=0.7)):
        with pytest.raises(B.VsError):
            B.vs_dynk_init(bad, 4)

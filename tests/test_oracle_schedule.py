"""The confidence schedule of the draft length ("DSpark" page, §2.2-§2.3):
the oracle's functions against closed forms and limiting cases, and the
library's host scheduler against the oracle, decision for decision."""
import ctypes

import numpy as np
import pytest

from oracle import spec


def test_row_confidence_closed_forms():
    # p = (0.5, 0.3, 0.2): top-1 0.5, gap 0.2
    t1, g = spec.row_confidence([np.log([0.5, 0.3, 0.2])])
    assert abs(t1 - 0.5) < 1e-15 and abs(g - 0.2) < 1e-15
    # uniform over V: top-1 1/V, gap 0
    t1, g = spec.row_confidence([np.zeros(64)])
    assert abs(t1 - 1 / 64) < 1e-15 and g == 0.0
    # two equal maxima: gap 0 whatever the rest
    z = np.array([3.0, 1.0, 3.0, -2.0])
    t1, g = spec.row_confidence([z])
    assert abs(g) < 1e-15 and abs(t1 - np.exp(3) / np.exp(z).sum()) < 1e-15
    # the temperature rescales the logits before the softmax
    t1, g = spec.row_confidence([np.log([0.5, 0.3, 0.2]) * 2.0], T=2.0)
    assert abs(t1 - 0.5) < 1e-15 and abs(g - 0.2) < 1e-15
    # the block value is the mean of the rows' values
    rows = [np.log([0.5, 0.3, 0.2]), np.log([0.9, 0.05, 0.05])]
    t1, g = spec.row_confidence(rows)
    assert abs(t1 - 0.7) < 1e-15 and abs(g - (0.2 + 0.85) / 2) < 1e-15


def test_ema_closed_form():
    """Full acceptance r times from 0.5: ema = 1 - 0.5 * 0.8^r; no acceptance:
    ema = 0.5 * 0.8^r."""
    up, down = spec.SchedState(4), spec.SchedState(4)
    for r in range(1, 12):
        spec.schedule_update(up, up.k, 0.5, 0.1)
        spec.schedule_update(down, 0, 0.5, 0.1)
        assert abs(up.ema - (1 - 0.5 * 0.8 ** r)) < 1e-12
        assert abs(down.ema - 0.5 * 0.8 ** r) < 1e-12


def test_linear_map_and_clamps():
    st = spec.SchedState(8)
    # C = 0.4*1 + 0.3*1 + 0.3*(0.2 + 0.8*0.5) = 0.88 -> above high -> max_k
    k, C = spec.schedule_update(st, 8, 1.0, 1.0)
    assert abs(C - 0.88) < 1e-12 and k == 16
    # low confidence with some acceptance: C below low -> min_k
    st = spec.SchedState(8)
    k, C = spec.schedule_update(st, 1, 0.0, 0.0)
    assert C < 0.3 and k == 2
    # a C in between maps linearly: choose inputs with C = 0.5 exactly in
    # binary-friendly steps: ema after a = k/2 from 0.5 stays 0.5
    st = spec.SchedState(8)
    k, C = spec.schedule_update(st, 4, 0.5, 0.1)  # 0.2 + 0.15 + 0.15
    assert abs(C - 0.5) < 1e-12 and k == int(2 + 14 * 0.5)
    # the gap term saturates at 5 * gap = 1
    a, b = spec.SchedState(8), spec.SchedState(8)
    assert spec.schedule_update(a, 4, 0.5, 0.2)[1] == spec.schedule_update(b, 4, 0.5, 0.9)[1]


def test_first_token_reject_drops_to_min_k():
    st = spec.SchedState(12, ema=0.99)
    k, C = spec.schedule_update(st, 0, 1.0, 1.0)
    assert C > 0.7 and k == 2


def test_k_monotone_in_confidence():
    ks = []
    for t1 in np.linspace(0, 1, 41):
        st = spec.SchedState(8)
        ks.append(spec.schedule_update(st, 3, t1, 0.05)[0])
    assert ks == sorted(ks) and ks[0] == 2 and ks[-1] > 2


def test_library_scheduler_matches_oracle():
    """The C ABI's host scheduler (no GPU involved) makes the oracle's decision
    and keeps the oracle's average, bit for bit, over random rounds."""
    from verification_verify_step_amd import binding as B
    cfg = B.sched_cfg()
    rng = np.random.default_rng(7)
    for trial in range(20):
        k0 = int(rng.integers(1, 20))
        lib_st = B.vs_sched_init(cfg, k0)
        ora = spec.SchedState(max(2, min(16, k0)))
        assert lib_st.k == ora.k and lib_st.ema == ora.ema
        for r in range(40):
            a = int(rng.integers(0, ora.k + 1)) if rng.random() < 0.8 else ora.k
            t1 = float(rng.random())
            g = float(rng.random() * t1)
            B.vs_sched_update(cfg, lib_st, a, t1, g)
            spec.schedule_update(ora, a, t1, g)
            assert lib_st.k == ora.k and lib_st.ema == ora.ema, (trial, r)
            assert lib_st.rounds == r + 1 and lib_st.last_a == a


def test_library_scheduler_rejects_bad_input():
    from verification_verify_step_amd import binding as B
    cfg = B.sched_cfg()
    st = B.vs_sched_init(cfg, 4)
    before = (st.k, st.ema, st.rounds)
    for a, t1, g in ((5, 0.5, 0.1), (-1, 0.5, 0.1), (2, float("nan"), 0.1)):
        with pytest.raises(B.VsError):
            B.vs_sched_update(cfg, st, a, t1, g)
        assert (st.k, st.ema, st.rounds) == before
    with pytest.raises(B.VsError):
        B.vs_sched_init(B.sched_cfg(min_k=3, max_k=2), 4)
    with pytest.raises(B.VsError):
        B.vs_sched_init(B.sched_cfg(low=0.7, high=0.3), 4)

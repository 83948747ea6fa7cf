"""The top-p variant of stochastic verification ("self-speculative" page,
§3.4: the draft keeps its full distribution, the verify truncates the target
to its top-p set and renormalises it there, then the ratio test runs on the
full draft distribution).  The oracle's truncation against hand cases and
against the properties that define the set; the emitted token against the
truncated target by chi-square."""
import numpy as np
import pytest
from scipy import stats

from oracle import spec
from tests.test_oracle_sampling import P8, Q8, TRIALS, _single_position_counts, _uniform_block


def test_hand_cases():
    assert np.array_equal(spec.top_p_filter([0.5, 0.3, 0.2], 0.5), [1.0, 0.0, 0.0])  # 0.5 reaches 0.5
    assert np.allclose(spec.top_p_filter([0.5, 0.3, 0.2], 0.6), [0.625, 0.375, 0.0], atol=1e-15)
    assert np.array_equal(spec.top_p_filter([0.25] * 4, 0.5), [0.5, 0.5, 0.0, 0.0])  # ties: lower ids first
    assert np.array_equal(spec.top_p_filter([0.2, 0.5, 0.3], 1.0), [0.2, 0.5, 0.3])
    assert np.array_equal(spec.top_p_filter([0.0, 1.0, 0.0], 0.9), [0.0, 1.0, 0.0])


def test_kept_set_properties():
    """The kept set K reaches top_p; dropping its least likely member falls
    short of it; nothing outside K is more likely than anything inside (and
    among equals the inside has the lower ids); the output is p / p(K) on K."""
    rng = np.random.default_rng(3)
    for _ in range(400):
        V = int(rng.integers(2, 9))
        p = rng.integers(0, 6, size=V).astype(np.float64)
        if p.sum() == 0:
            continue
        p /= p.sum()
        top_p = float(rng.choice([rng.random(), 0.5, 1.0]))
        out = spec.top_p_filter(p, top_p)
        K = np.nonzero(out)[0]
        mass = p[K].sum()
        assert mass >= top_p - 1e-12
        if len(K) > 1:
            weakest = min(K, key=lambda j: (p[j], -j))
            assert mass - p[weakest] < top_p + 1e-12
        for j in range(V):
            if j not in K:
                for i in K:
                    assert p[j] < p[i] or (p[j] == p[i] and j > i)
        assert np.allclose(out[K], p[K] / mass, atol=1e-15)


def test_margin():
    assert abs(spec.top_p_margin([0.5, 0.3, 0.2], 0.6) - 0.1) < 1e-15
    assert spec.top_p_margin([0.5, 0.3, 0.2], 0.5) == 0.0


@pytest.mark.parametrize("top_p", [0.5, 0.8])
def test_emitted_token_follows_truncated_target(top_p):
    """Drafts from the full q, the test against the truncated p': the emitted
    token is distributed as p', ids outside the top-p set never appear, and a
    draft is accepted with probability sum_x min(p'(x), q(x))."""
    U = _uniform_block(TRIALS, rnd=3)
    pt = spec.top_p_filter(P8, top_p)
    counts, accepted = _single_position_counts(pt, Q8, U)
    assert counts[pt == 0].sum() == 0
    nz = pt > 0
    _, pval = stats.chisquare(counts[nz], TRIALS * pt[nz])
    assert pval > 1e-3, (counts, pval)
    alpha = np.minimum(pt, Q8).sum()
    sd = np.sqrt(TRIALS * alpha * (1 - alpha))
    assert abs(accepted - TRIALS * alpha) < 4 * sd

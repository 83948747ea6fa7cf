"""Pins of the oracle's stochastic acceptance to the mathematics the pages
state: with drafts x ~ q accepted with probability min(1, p(x)/q(x)) and
rejections resampled from normalize(max(0, p - q)), the emitted token is
distributed exactly as p, whatever q is (self-speculative decoding page,
m.lqnn.cn/news/278124, §2.4; "推测解码技术原理与实践" page, §2.2).  Checked by
chi-square on seeded trials, by the acceptance rate sum_x min(p, q), and the
sampler by exact rational arithmetic."""
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

import synth
from oracle import spec

TRIALS = 100000


def _u(trial, rnd=0):
    return synth.uniforms(synth.SEED_UNIFORMS, synth.stream_uniform(trial, rnd), spec.N_UNIFORMS)


def _uniform_block(n_trials, rnd=0):
    """[n_trials][48] uniforms, trial t = request t."""
    out = np.empty((n_trials, spec.N_UNIFORMS))
    for t in range(n_trials):
        out[t] = _u(t, rnd)
    return out


@pytest.fixture(scope="module")
def U():
    return _uniform_block(TRIALS)


def test_sampler_matches_exact_inverse_cdf():
    rng = np.random.default_rng(5)
    for _ in range(200):
        w = rng.integers(0, 5, size=8).astype(np.float64)
        if w.sum() == 0:
            continue
        wf = [Fraction(int(x)) for x in w]
        S = sum(wf)
        for u in rng.random(20):
            uf = Fraction(u)
            C, want = Fraction(0), None
            for j, x in enumerate(wf):
                C += x
                if uf * S < C:
                    want = j
                    break
            assert spec.sample_index(w, u) == want
            assert w[spec.sample_index(w, u)] > 0


def test_sampler_never_picks_zero_weight_at_the_top():
    w = np.array([0.2, 0.3, 0.0, 0.0])
    assert spec.sample_index(w, 1.0 - 2.0 ** -53) == 1


def _single_position_counts(p, q, U):
    counts = np.zeros(len(p), dtype=np.int64)
    accepted = 0
    for t in range(len(U)):
        u = U[t]
        d = spec.sample_index(q, u[0])
        a, y, _ = spec.accept_stochastic_chain([0, d], [p, p], [q], u)
        tok = d if a == 1 else y
        accepted += a
        counts[tok] += 1
    return counts, accepted


P8 = np.array([0.30, 0.00, 0.10, 0.05, 0.25, 0.00, 0.20, 0.10])
Q8 = np.array([0.10, 0.30, 0.00, 0.25, 0.05, 0.00, 0.20, 0.10])


def test_chi_square_single_position(U):
    counts, accepted = _single_position_counts(P8, Q8, U)
    assert counts[P8 == 0].sum() == 0  # impossible tokens never appear
    nz = P8 > 0
    _, pval = stats.chisquare(counts[nz], TRIALS * P8[nz])
    assert pval > 1e-3, (counts, pval)
    # acceptance probability of one draft is sum_x min(p(x), q(x))
    alpha = np.minimum(P8, Q8).sum()
    sd = np.sqrt(TRIALS * alpha * (1 - alpha))
    assert abs(accepted - TRIALS * alpha) < 4 * sd


def test_p_equal_q_always_accepts(U):
    counts, accepted = _single_position_counts(P8, P8, U[:5000])
    assert accepted == 5000


def test_residual_fallback_to_p():
    """When max(0, p - q) sums to zero (p <= q within rounding) a rejected
    draft is resampled from p itself."""
    p = np.array([0.25, 0.25, 0.5])
    q = p * (1 + 1e-12)
    u = np.zeros(spec.N_UNIFORMS)
    u[spec.SLOT_ACCEPT] = 1.0 - 2.0 ** -53  # above p/q = 1 - 1e-12: reject
    u[spec.SLOT_RESAMPLE] = 0.6
    a, y, _ = spec.accept_stochastic_chain([0, 1], [p, p], [q], u)
    assert a == 0 and y == spec.sample_index(p, 0.6) == 2


def test_markov_harness_two_positions():
    """Bigram target/draft tables on V=8, k=2 plus bonus: the joint law of the
    first two emitted tokens equals the target's p(x1|x0) p(x2|x1)."""
    rng = np.random.default_rng(11)
    V, x0 = 8, 3
    Pt = rng.dirichlet(np.ones(V) * 0.7, size=V)
    Pd = rng.dirichlet(np.ones(V) * 0.7, size=V)
    Pt[:, 5] = 0  # a token the target never emits
    Pt /= Pt.sum(1, keepdims=True)
    n = 40000
    U = _uniform_block(n, rnd=1)
    counts = np.zeros((V, V), dtype=np.int64)
    for t in range(n):
        u = U[t]
        d1 = spec.sample_index(Pd[x0], u[0])
        d2 = spec.sample_index(Pd[d1], u[1])
        toks = [x0, d1, d2]
        a, y, _ = spec.accept_stochastic_chain(toks, [Pt[x0], Pt[d1], Pt[d2]], [Pd[x0], Pd[d1]], u)
        out = toks[1:a + 1] + [y]
        if len(out) < 2:  # first draft rejected: the second token comes from the next round
            u2 = _u(t, rnd=2)
            d = spec.sample_index(Pd[out[0]], u2[0])
            a2, y2, _ = spec.accept_stochastic_chain([out[0], d], [Pt[out[0]], Pt[d]], [Pd[out[0]]], u2)
            out.append(d if a2 == 1 else y2)
        counts[out[0], out[1]] += 1
    joint = Pt[x0][:, None] * Pt
    assert counts[joint == 0].sum() == 0
    nz = joint > 0
    _, pval = stats.chisquare(counts[nz], n * joint[nz] / joint[nz].sum())
    assert pval > 1e-3, pval


def test_flag_band():
    p = np.array([0.5, 0.5])
    q = np.array([0.5, 0.5])
    u = np.zeros(spec.N_UNIFORMS)
    u[spec.SLOT_ACCEPT] = 0.9995  # ratio 1, |1 - u| < 1e-3
    _, _, flags = spec.accept_stochastic_chain([0, 1], [p, p], [q], u)
    assert flags == [0]

"""Prompt-copy (n-gram) drafting with a full-depth verify ("self-speculative"
page, §2.2): the oracle's proposal against hand cases and the properties that
define it, the library's host proposal against the oracle, and the
losslessness of the rounds on the oracle decoder."""
import numpy as np

from oracle import spec
from oracle.decoder import KVCache
from synth.workloads import TINY
from tests import gpu_common as G


def test_hand_cases():
    h = [5, 1, 2, 3, 9, 1, 2, 3, 4, 1, 2, 3]
    assert spec.ngram_propose(h, len(h), 1, 3, 4) == [4, 1, 2, 3]  # latest earlier (1, 2, 3)
    assert spec.ngram_propose(h, len(h), 1, 3, 2) == [4, 1]        # at most k_max
    assert spec.ngram_propose(h, 6, 1, 3, 4) == [9, 1]             # only the first 6 tokens are searched
    assert spec.ngram_propose([1, 2, 3, 4], 4, 1, 3, 4) == []      # nothing repeats
    assert spec.ngram_propose([7, 7, 7, 7], 4, 1, 3, 4) == [7]     # overlapping occurrence
    assert spec.ngram_propose([1, 2, 9, 2], 4, 2, 3, 4) == []      # only 1-grams match, below min


def _brute(h, search_len, lo, hi, k):
    n, limit = len(h), min(len(h), search_len)
    best = None
    for g in range(lo, hi + 1):
        if g > n - 1:
            continue
        for i in range(n):
            if i + g < limit and h[i:i + g] == h[n - g:]:
                if best is None or (g, i) > best:
                    best = (g, i)
    if best is None:
        return []
    g, i = best
    return h[i + g:min(i + g + k, limit)]


def test_matches_the_definition():
    """The longest suffix that occurs earlier wins, then its latest
    occurrence, checked against an exhaustive scan over (length, start)."""
    rng = np.random.default_rng(4)
    for _ in range(2000):
        n = int(rng.integers(1, 14))
        h = [int(x) for x in rng.integers(0, 3, n)]
        sl = int(rng.integers(1, n + 2))
        lo = int(rng.integers(1, 3))
        hi = lo + int(rng.integers(0, 3))
        k = int(rng.integers(0, 6))
        assert spec.ngram_propose(h, sl, lo, hi, k) == _brute(h, sl, lo, hi, k), (h, sl, lo, hi, k)


def test_library_proposal_matches_oracle():
    from verification_verify_step_amd import binding as B
    rng = np.random.default_rng(5)
    for _ in range(1000):
        n = int(rng.integers(1, 40))
        h = [int(x) for x in rng.integers(0, 4, n)]
        sl = int(rng.integers(0, n + 3))
        lo = int(rng.integers(1, 4))
        hi = lo + int(rng.integers(0, 4))
        k = int(rng.integers(0, B.VS_MAX_K + 1))
        assert B.vs_ngram_propose(h, sl, lo, hi, k) == spec.ngram_propose(h, sl, lo, hi, k)


def test_rounds_are_lossless():
    """n-gram rounds produce the greedy autoregressive tokens (the tiny model
    repeats itself, so drafts are accepted)."""
    dec = G.oracle_decoder(TINY)
    p = G.prompt(TINY, 64, req=3)
    ref, _ = spec.generate_ar(dec, KVCache(TINY, 512), 0, p, 40)
    cache = KVCache(TINY, 512)
    st, _ = spec.prefill(dec, cache, 0, p)
    accepted = 0
    while len(st.tokens) - len(p) < 40:
        d, a, y, _ = spec.ngram_round(dec, cache, st, 8)
        accepted += a
    assert st.tokens[len(p):len(p) + 40] == ref
    assert accepted > 10

"""Pins of the oracle's speculative round to what the pages and the
mathematics fix: greedy speculative output equals greedy autoregressive output
token for token (self-speculative decoding page, m.lqnn.cn/news/278124, §5.2;
"DSpark" page §2.1); a full recompute without any cache agrees; the first-L KV
written by the draft equals one batched pass; and the rollback invariant
holds after every round (same page, §3.3)."""
import numpy as np
import pytest

import synth
from oracle import spec
from oracle.decoder import Decoder, KVCache, Row
from synth.model_weights import SynthWeights
from synth.workloads import TINY


class UpperScaled:
    """Weights whose W_o and W_down of layers >= L are scaled by eps: eps = 0
    makes the target equal to the draft (every draft accepted)."""

    def __init__(self, base, L, eps):
        self.base, self.L, self.eps = base, L, eps

    def get(self, t, l=0):
        a = self.base.get(t, l)
        if t in (synth.T_WO, synth.T_W_DOWN) and l >= self.L:
            return a * self.eps
        return a


def _dec(precision="f32", L=None, eps=None, cfg=TINY):
    if L is not None:
        cfg = cfg.__class__(**{**cfg.__dict__, "exit_layer": L})
    w = SynthWeights(cfg, precision=precision)
    if eps is not None:
        w = UpperScaled(w, cfg.exit_layer, eps)
    return Decoder(cfg, w)


def _prompt(n=64, req=0, vocab=TINY.vocab):
    return synth.tokens(synth.SEED_PROMPTS, synth.stream_prompt(req), vocab, n)


def brute_force_greedy(dec, prompt, n_new):
    """Greedy decode recomputing the whole sequence from scratch every token."""
    toks = [int(t) for t in prompt]
    for _ in range(n_new):
        cache = KVCache(dec.cfg, len(toks) + 1, kv_round="bf16")
        rows = [Row(0, i, i, np.arange(i + 1)) for i in range(len(toks))]
        z = dec.head(dec.forward_layers(cache, rows[-len(toks):], dec.embed(toks), 0, dec.cfg.n_layers))
        toks.append(int(np.argmax(z[-1])))
    return toks[len(prompt):]


@pytest.mark.parametrize("precision,kv", [("f32", "none"), ("bf16", "bf16")])
@pytest.mark.parametrize("k", [0, 1, 4])
def test_spec_equals_ar_greedy(precision, kv, k):
    dec = _dec(precision)
    prompt = _prompt()
    ar, _ = spec.generate_ar(dec, KVCache(dec.cfg, 160, kv), 0, prompt, 32)
    sp, st = spec.generate_spec(dec, KVCache(dec.cfg, 160, kv), 0, prompt, 32, k)
    assert sp == ar
    assert st.P == len(st.tokens) - 1


@pytest.mark.parametrize("eps", [0.0, 0.3])
def test_spec_equals_ar_with_acceptance(eps):
    """eps = 0: target == draft, so every draft is accepted (a = k); eps = 0.3
    gives a mix of accepted lengths.  Output still equals plain greedy."""
    dec = _dec("bf16", eps=eps)
    prompt = _prompt()
    ar, _ = spec.generate_ar(dec, KVCache(dec.cfg, 160), 0, prompt, 32)
    sp, st = spec.generate_spec(dec, KVCache(dec.cfg, 160), 0, prompt, 32, 4)
    assert sp == ar
    if eps == 0.0:
        assert all(a == 4 for a in st.rounds[:-1])
    else:
        assert len(set(st.rounds)) > 1


def test_exit_layer_extremes():
    """L = N: the draft is the full model, so greedy accepts every draft.
    L = 0: the draft is embedding + head, verify is the plain full forward."""
    for L in (TINY.n_layers, 0):
        dec = _dec("bf16", L=L)
        prompt = _prompt()
        ar, _ = spec.generate_ar(dec, KVCache(dec.cfg, 160), 0, prompt, 16)
        sp, st = spec.generate_spec(dec, KVCache(dec.cfg, 160), 0, prompt, 16, 3)
        assert sp == ar
        if L == TINY.n_layers:
            assert all(a == 3 for a in st.rounds[:-1])


def test_spec_equals_no_cache_recompute():
    dec = _dec("bf16", eps=0.3)
    prompt = _prompt(48, req=3)
    sp, _ = spec.generate_spec(dec, KVCache(dec.cfg, 160), 0, prompt, 12, 4)
    assert sp == brute_force_greedy(dec, prompt, 12)


def test_first_L_kv_identity():
    """The draft's k+1 sequential one-row passes leave the same first-L KV (and
    hidden_L) as one batched pass over the k+1 chain rows."""
    dec = _dec("bf16", eps=0.3)
    cache = KVCache(dec.cfg, 160)
    st, _ = spec.prefill(dec, cache, 0, _prompt())
    toks, _, hL = spec.draft_chain(dec, cache, st, 4)
    cache2 = KVCache(dec.cfg, 160)
    spec.prefill(dec, cache2, 0, _prompt())
    rows = spec.chain_rows(0, st.P, 5)
    h2 = dec.forward_layers(cache2, rows, dec.embed(toks), 0, dec.cfg.exit_layer)
    np.testing.assert_allclose(hL, h2, rtol=1e-12, atol=1e-12)
    for l in range(dec.cfg.exit_layer):
        K1, V1 = cache.get(0, l)
        K2, V2 = cache2.get(0, l)
        np.testing.assert_array_equal(K1[:, :st.P + 5], K2[:, :st.P + 5])
        np.testing.assert_array_equal(V1[:, :st.P + 5], V2[:, :st.P + 5])


def test_chain_mask_equals_causal_recompute():
    """Verify logits of the chain rows over the cache equal the last rows of a
    plain causal forward over the whole token sequence."""
    dec = _dec("bf16", eps=0.3)
    cache = KVCache(dec.cfg, 160)
    prompt = _prompt()
    st, _ = spec.prefill(dec, cache, 0, prompt)
    toks, _, hL = spec.draft_chain(dec, cache, st, 4)
    z = spec.verify_chain(dec, cache, st, toks, hL)
    full = list(prompt) + toks
    c2 = KVCache(dec.cfg, 160)
    rows = [Row(0, i, i, np.arange(i + 1)) for i in range(len(full))]
    zf = dec.head(dec.forward_layers(c2, rows, dec.embed(full), 0, dec.cfg.n_layers))
    np.testing.assert_allclose(z, zf[-5:], rtol=1e-10, atol=1e-10)


def test_rollback_invariant_and_poison():
    dec = _dec("bf16", eps=0.3)
    cache = KVCache(dec.cfg, 160)
    st, _ = spec.prefill(dec, cache, 0, _prompt())
    for _ in range(5):
        P0 = st.P
        a, y, _, _ = spec.spec_round(dec, cache, st, 4)
        assert st.P == P0 + a + 1 == len(st.tokens) - 1
        K, _ = cache.get(0, 0)
        assert not np.isnan(K[:, :st.P]).any() and np.isnan(K[:, st.P:]).all()


def test_final_norm_is_applied_before_head():
    """The head normalises first, so its logits do not depend on the scale of
    the hidden state it is fed (the pages warn that skipping the norm at an
    early exit silently ruins the drafts)."""
    dec = _dec("bf16")
    h = dec.embed([1, 2]) * 50.0  # rms ~1, so eps (1e-5) is negligible
    np.testing.assert_allclose(dec.head(h * 40.0), dec.head(h), rtol=1e-4, atol=1e-6)
    z_raw = (h * 40.0) @ dec.w.get(synth.T_HEAD).T
    assert np.abs(z_raw).max() > 5 * np.abs(dec.head(h)).max()

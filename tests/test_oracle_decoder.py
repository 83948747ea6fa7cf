"""Pins of the oracle's decoder to things other than itself: an independent
Llama implementation (HuggingFace transformers, float64), torch's own
RMSNorm / attention / bf16 conversion, and closed-form properties of RoPE."""
import numpy as np
import pytest
import torch

import synth
from oracle.decoder import Decoder, KVCache, Row, attend, bf16_round, rms_norm, rope
from synth.model_weights import SynthWeights
from synth.workloads import TINY


def test_bf16_round_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-8, 8, 100000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bf16_round(x.astype(np.float64)), want)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: even mantissa (1.0) wins.
    assert bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: even is 1+2^-6.
    assert bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    # just above the midpoint rounds up
    assert bf16_round(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7
    assert bf16_round(np.array([-2.5]))[0] == -2.5


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(1)
    x, g = rng.standard_normal((5, 64)), rng.standard_normal(64)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(rms_norm(x, g, 1e-5), want, rtol=1e-13, atol=1e-13)


def test_rope_properties():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    # position 0 is the identity
    np.testing.assert_allclose(rope(q, np.array(0), 1e4), q, atol=0)
    # each pair (i, i+64) keeps its length
    r = rope(q, np.array(37), 1e4)
    np.testing.assert_allclose(r[:64] ** 2 + r[64:] ** 2, q[:64] ** 2 + q[64:] ** 2, rtol=1e-12)
    # the score depends only on the position difference
    s1 = rope(q, np.array(100), 1e4) @ rope(k, np.array(90), 1e4)
    s2 = rope(q, np.array(1010), 1e4) @ rope(k, np.array(1000), 1e4)
    assert abs(s1 - s2) < 1e-9
    # pair 0 turns by exactly the position (inverse frequency 1)
    e0 = np.zeros(128)
    e0[0] = 1.0
    r = rope(e0, np.array(3), 1e4)
    assert abs(r[0] - np.cos(3)) < 1e-15 and abs(r[64] - np.sin(3)) < 1e-15


def test_attend_matches_torch_sdpa():
    rng = np.random.default_rng(3)
    q, K, V = rng.standard_normal(64), rng.standard_normal((10, 64)), rng.standard_normal((10, 64))
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None])
    np.testing.assert_allclose(attend(q, K, V), want[0, 0, 0].numpy(), rtol=1e-12, atol=1e-13)


def _hf_llama(cfg, weights):
    from transformers import LlamaConfig, LlamaForCausalLM
    hc = LlamaConfig(vocab_size=cfg.vocab, hidden_size=cfg.d_model, intermediate_size=cfg.d_ffn,
                     num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_heads,
                     num_key_value_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, rms_norm_eps=cfg.rms_eps,
                     rope_theta=cfg.rope_theta, tie_word_embeddings=False, attention_bias=False, mlp_bias=False,
                     max_position_embeddings=4096)
    m = LlamaForCausalLM(hc).double().eval()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(t(weights.get(synth.T_EMBED)))
        for l, layer in enumerate(m.model.layers):
            layer.input_layernorm.weight.copy_(t(weights.get(synth.T_ATTN_NORM, l)))
            layer.self_attn.q_proj.weight.copy_(t(weights.get(synth.T_WQ, l)))
            layer.self_attn.k_proj.weight.copy_(t(weights.get(synth.T_WK, l)))
            layer.self_attn.v_proj.weight.copy_(t(weights.get(synth.T_WV, l)))
            layer.self_attn.o_proj.weight.copy_(t(weights.get(synth.T_WO, l)))
            layer.post_attention_layernorm.weight.copy_(t(weights.get(synth.T_FFN_NORM, l)))
            layer.mlp.gate_proj.weight.copy_(t(weights.get(synth.T_W_GATE, l)))
            layer.mlp.up_proj.weight.copy_(t(weights.get(synth.T_W_UP, l)))
            layer.mlp.down_proj.weight.copy_(t(weights.get(synth.T_W_DOWN, l)))
        m.model.norm.weight.copy_(t(weights.get(synth.T_FINAL_NORM)))
        m.lm_head.weight.copy_(t(weights.get(synth.T_HEAD)))
    return m


@pytest.mark.parametrize("gqa", [False, True])
def test_decoder_matches_hf_llama(gqa):
    """Full-depth logits of a causal prompt equal transformers' LlamaForCausalLM
    (an independent implementation) in float64.  HF evaluates RoPE angles in
    float32, so agreement is to ~1e-6, not rounding level."""
    cfg = TINY if not gqa else TINY.__class__(**{**TINY.__dict__, "n_kv_heads": 2})
    w = SynthWeights(cfg, precision="f32")
    # scale up the weights so the layers move the residual stream visibly
    class Scaled:
        def get(self, t, l=0):
            a = w.get(t, l)
            return a if t in (synth.T_ATTN_NORM, synth.T_FFN_NORM, synth.T_FINAL_NORM, synth.T_EMBED) else a * 5.0
    sw = Scaled()
    prompt = synth.tokens(synth.SEED_PROMPTS, synth.stream_prompt(0), cfg.vocab, 24)
    dec = Decoder(cfg, sw)
    cache = KVCache(cfg, 64, kv_round="none")
    rows = [Row(0, i, i, np.arange(i + 1)) for i in range(len(prompt))]
    z = dec.head(dec.forward_layers(cache, rows, dec.embed(prompt), 0, cfg.n_layers))
    hf = _hf_llama(cfg, sw)
    with torch.no_grad():
        zr = hf(torch.from_numpy(prompt.astype(np.int64))[None]).logits[0].numpy()
    assert np.abs(z).max() > 0.5  # not a trivially small signal
    np.testing.assert_allclose(z, zr, rtol=0, atol=2e-5)


def test_kv_cache_stores_bf16_values():
    cfg = TINY
    cache = KVCache(cfg, 8, kv_round="bf16")
    rng = np.random.default_rng(4)
    k, v = rng.standard_normal((4, 64)), rng.standard_normal((4, 64))
    cache.store(0, 1, 3, k, v)
    K, V = cache.get(0, 1)
    np.testing.assert_array_equal(K[:, 3], bf16_round(k))
    np.testing.assert_array_equal(V[:, 3], bf16_round(v))
    assert np.isnan(K[:, 4]).all()

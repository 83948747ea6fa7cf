"""Canonical weights of the synthetic decoders, drawn from the seeded streams.

Canonical layout (row-major, one tensor per (tensor id, layer)):
  embed [V][d]; per layer: attn_norm [d], wq [H*hd][d], wk [Hkv*hd][d],
  wv [Hkv*hd][d], wo [d][H*hd], ffn_norm [d], w_gate [F][d], w_up [F][d],
  w_down [d][F]; final_norm [d]; head [V][d].
Matrices are N(0, 0.02) from stream (tensor, layer); norm gains are 1.
"""
import numpy as np

import synth

TENSOR_NAMES = ["embed", "attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down",
                "final_norm", "head"]
GAIN_TENSORS = (synth.T_ATTN_NORM, synth.T_FFN_NORM, synth.T_FINAL_NORM)
LAYER_TENSORS = (synth.T_ATTN_NORM, synth.T_WQ, synth.T_WK, synth.T_WV, synth.T_WO, synth.T_FFN_NORM,
                 synth.T_W_GATE, synth.T_W_UP, synth.T_W_DOWN)


def tensor_shape(cfg, t):
    d, hd, H, Hkv, F, V = cfg.d_model, cfg.head_dim, cfg.n_heads, cfg.n_kv_heads, cfg.d_ffn, cfg.vocab
    return {
        synth.T_EMBED: (V, d), synth.T_ATTN_NORM: (d,), synth.T_WQ: (H * hd, d), synth.T_WK: (Hkv * hd, d),
        synth.T_WV: (Hkv * hd, d), synth.T_WO: (d, H * hd), synth.T_FFN_NORM: (d,), synth.T_W_GATE: (F, d),
        synth.T_W_UP: (F, d), synth.T_W_DOWN: (d, F), synth.T_FINAL_NORM: (d,), synth.T_HEAD: (V, d),
    }[t]


def tensor_stream_layer(cfg, t, layer):
    """Layer index used in the stream id (global tensors use n_layers)."""
    return layer if t in LAYER_TENSORS else cfg.n_layers


def bf16_bits(cfg, t, layer, seed=synth.SEED_WEIGHTS):
    """Canonical bf16 bit patterns (uint16) of tensor t."""
    shape = tensor_shape(cfg, t)
    n = int(np.prod(shape))
    if t in GAIN_TENSORS:
        return np.full(shape, 0x3F80, dtype=np.uint16)  # 1.0
    s = synth.stream_weight(t, tensor_stream_layer(cfg, t, layer))
    return synth.normal_bf16_bits(seed, s, n).reshape(shape)


def f32_values(cfg, t, layer, seed=synth.SEED_WEIGHTS):
    """Canonical fp32 values of tensor t (the fp32-weight profile)."""
    shape = tensor_shape(cfg, t)
    n = int(np.prod(shape))
    if t in GAIN_TENSORS:
        return np.ones(shape, dtype=np.float32)
    s = synth.stream_weight(t, tensor_stream_layer(cfg, t, layer))
    return synth.normal_f32(seed, s, n).reshape(shape)


class SynthWeights:
    """Lazy fp64 view of the synthetic weights, one tensor at a time.

    precision: "bf16" (values rounded to bf16, the GPU's weights) or "f32".
    cache: keep converted tensors in memory (small models).
    """

    def __init__(self, cfg, precision="bf16", seed=synth.SEED_WEIGHTS, cache=True):
        self.cfg, self.precision, self.seed, self.cache = cfg, precision, seed, cache
        self._store = {}

    def get(self, t, layer=0):
        k = (t, layer if t in LAYER_TENSORS else -1)
        if k in self._store:
            return self._store[k]
        if self.precision == "bf16":
            a = synth.bf16_bits_to_f64(bf16_bits(self.cfg, t, layer, self.seed))
        else:
            a = f32_values(self.cfg, t, layer, self.seed).astype(np.float64)
        if self.cache:
            self._store[k] = a
        return a

"""Plain float64 Llama-style decoder with a slot-addressed KV cache (oracle).

TEST INFRASTRUCTURE: see ``oracle/__init__.py``.

The pages' interface is a layer-range forward over a shared KV cache with a
per-sequence write position, plus a separately callable final norm and LM
head (self-speculative decoding page, m.lqnn.cn/news/278124, §4.1 and the
draft/verify functions of §4.2-§4.3).  The decoder itself is the 7B
Llama shape the pages run (same page §2.3: 32 layers, 12-layer draft):
pre-norm RMSNorm, rotary position embedding on q and k, softmax attention
scaled by 1/sqrt(head_dim), SwiGLU feed-forward, untied embedding and head.

Readings where the pages are silent (each listed in the design doc):
* RMSNorm eps 1e-5, gains 1; RoPE base 10000 with the rotate-half pairing
  (i, i + hd/2) at absolute positions from 0; keys cached after RoPE.
* GQA: query head h reads KV head h // (H / Hkv).
* The KV cache stores values rounded to bf16 (the model's storage precision)
  unless kv_round="none"; all arithmetic is float64.
"""
from dataclasses import dataclass

import numpy as np

import synth

_T = synth  # tensor ids T_* live in synth (shared numbering with the C ABI)


def bf16_round(x):
    """Nearest bf16 value of each float64 (ties to even), returned as float64.

    bf16 keeps the fp32 exponent and the top 7 fraction bits, so rounding a
    float64 drops its low 45 fraction bits.  Values here are normal numbers
    well inside the fp32 range.
    """
    b = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    r = (b + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    return r.view(np.float64).reshape(np.shape(x))


def rms_norm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope(x, pos, theta):
    """Rotate-half rotary embedding of x [..., hd] at integer positions pos [...].

    Pair (i, i + hd/2) turns by angle pos * theta^(-2i/hd).
    """
    hd = x.shape[-1]
    half = hd // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / hd)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


def softmax(z):
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


@dataclass
class Row:
    """One input row of a pass: which sequence, RoPE position, KV slot written,
    and the KV slots it attends to (its own slot included)."""
    seq: int
    pos: int
    slot: int
    visible: np.ndarray


class KVCache:
    """KV cache addressed by (sequence, layer, slot); slot = index in the
    sequence's cache.  Values are stored rounded per ``kv_round``."""

    def __init__(self, cfg, capacity, kv_round="bf16"):
        self.cfg, self.capacity, self.kv_round = cfg, capacity, kv_round
        self._k, self._v = {}, {}

    def _arrays(self, seq, layer):
        key = (seq, layer)
        if key not in self._k:
            shape = (self.cfg.n_kv_heads, self.capacity, self.cfg.head_dim)
            self._k[key] = np.full(shape, np.nan)
            self._v[key] = np.full(shape, np.nan)
        return self._k[key], self._v[key]

    def store(self, seq, layer, slot, k, v):
        K, V = self._arrays(seq, layer)
        if self.kv_round == "bf16":
            k, v = bf16_round(k), bf16_round(v)
        K[:, slot, :] = k
        V[:, slot, :] = v

    def get(self, seq, layer):
        return self._arrays(seq, layer)

    def poison(self, seq, first_slot):
        """Mark slots >= first_slot of a sequence as garbage (NaN) in every layer."""
        for (s, _l), K in self._k.items():
            if s == seq:
                K[:, first_slot:, :] = np.nan
                self._v[(s, _l)][:, first_slot:, :] = np.nan

    def copy_slot(self, seq, src, dst):
        for (s, _l), K in self._k.items():
            if s == seq:
                K[:, dst, :] = K[:, src, :]
                V = self._v[(s, _l)]
                V[:, dst, :] = V[:, src, :]


def attend(q, K, V):
    """softmax(K q / sqrt(hd)) V for one query vector over the given keys."""
    s = (K @ q) / np.sqrt(q.shape[-1])
    p = softmax(s)
    return p @ V


class Decoder:
    """Float64 decoder over weights from ``weights.get(tensor_id, layer)``."""

    def __init__(self, cfg, weights):
        self.cfg, self.w = cfg, weights

    def embed(self, tokens):
        E = self.w.get(_T.T_EMBED)
        return E[np.asarray(tokens, dtype=np.int64)].copy()

    def layer(self, l, cache, rows, h):
        cfg = self.cfg
        M, H, Hkv, hd = len(rows), cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
        W = lambda t: self.w.get(t, l)  # noqa: E731
        x = rms_norm(h, W(_T.T_ATTN_NORM), cfg.rms_eps)
        q = (x @ W(_T.T_WQ).T).reshape(M, H, hd)
        k = (x @ W(_T.T_WK).T).reshape(M, Hkv, hd)
        v = (x @ W(_T.T_WV).T).reshape(M, Hkv, hd)
        pos = np.array([r.pos for r in rows], dtype=np.float64)
        q = rope(q, pos[:, None], cfg.rope_theta)
        k = rope(k, pos[:, None], cfg.rope_theta)
        # Every row of the pass stores its key/value before any row attends,
        # so in-pass ancestors are visible through ``visible``.
        for i, r in enumerate(rows):
            cache.store(r.seq, l, r.slot, k[i], v[i])
        o = np.zeros((M, H, hd))
        group = H // Hkv
        for i, r in enumerate(rows):
            K, V = cache.get(r.seq, l)
            vis = np.asarray(r.visible, dtype=np.int64)
            for hh in range(H):
                kvh = hh // group
                o[i, hh] = attend(q[i, hh], K[kvh, vis], V[kvh, vis])
        h = h + o.reshape(M, H * hd) @ W(_T.T_WO).T
        x2 = rms_norm(h, W(_T.T_FFN_NORM), cfg.rms_eps)
        g = x2 @ W(_T.T_W_GATE).T
        u = x2 @ W(_T.T_W_UP).T
        return h + (silu(g) * u) @ W(_T.T_W_DOWN).T

    def forward_layers(self, cache, rows, h, start, end):
        """Layers start..end-1 over the rows (the pages' forward_layers)."""
        for l in range(start, end):
            h = self.layer(l, cache, rows, h)
        return h

    def head(self, h):
        """LM head after the final norm: norm first, as the pages insist."""
        x = rms_norm(h, self.w.get(_T.T_FINAL_NORM), self.cfg.rms_eps)
        return x @ self.w.get(_T.T_HEAD).T

"""How far bf16-only GEMM inputs would move the verify logits, measured with
the float64 oracle alone at full depth (a script, not a collected test).

The GPU path feeds every GEMM "split bf16" inputs: hi = bf16(x) and
lo = bf16(x - hi), about 16 bits of each activation.  Dropping lo would halve
the MFMA work of the compute-bound shapes (the 70B batch), but adds the
rounding of every GEMM input to bf16.  The pages bound the verify logits at
2e-2 absolute.  This script runs the verify layers L..N-1 and the head twice
over the same chain rows (self-speculative decoding page, §4.3), on the same
weights, committed KV and layer-L rows:
* exact: the oracle decoder as it stands;
* bf16 inputs: the same layer with every GEMM input (normed rows before QKV,
  attention output before O, normed rows before gate/up, SwiGLU output before
  down, final-normed rows before the head) rounded to bf16;
and prints the max-abs logit difference, with the largest |logit|.

Inputs follow the GPU tests of these shapes: committed K and V drawn N(0, 1)
(the cache rounds them to bf16), layer-L rows N(0, 1), one sequence of k + 1
chain rows at context P.

Usage: python -m tests.act_precision {7b|70b} [P] [k] [layers]
  layers: how many of the verify layers to run (default all, N - L).
"""
import sys
import time

import numpy as np

import synth
from oracle import spec
from oracle.decoder import Decoder, KVCache, bf16_round, rms_norm, rope, attend, silu
from synth.model_weights import LAYER_TENSORS, SynthWeights
from synth.workloads import LLAMA70B, LLAMA7B


class OneLayerWeights:
    """bf16-valued float64 weights, one layer held at a time."""

    def __init__(self, cfg):
        self.base = SynthWeights(cfg, precision="bf16", cache=False)
        self.layer, self.cur, self.glob = None, {}, {}

    def get(self, t, layer=0):
        if t in LAYER_TENSORS:
            if layer != self.layer:
                self.layer, self.cur = layer, {}
            if t not in self.cur:
                self.cur[t] = self.base.get(t, layer)
            return self.cur[t]
        if t not in self.glob:
            self.glob[t] = self.base.get(t, layer)
        return self.glob[t]


def layer_bf16_inputs(dec, l, cache, rows, h):
    """The oracle layer with each GEMM input rounded to bf16."""
    cfg = dec.cfg
    M, H, Hkv, hd = len(rows), cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    W = lambda t: dec.w.get(t, l)  # noqa: E731
    x = bf16_round(rms_norm(h, W(synth.T_ATTN_NORM), cfg.rms_eps))
    q = (x @ W(synth.T_WQ).T).reshape(M, H, hd)
    k = (x @ W(synth.T_WK).T).reshape(M, Hkv, hd)
    v = (x @ W(synth.T_WV).T).reshape(M, Hkv, hd)
    pos = np.array([r.pos for r in rows], dtype=np.float64)
    q = rope(q, pos[:, None], cfg.rope_theta)
    k = rope(k, pos[:, None], cfg.rope_theta)
    for i, r in enumerate(rows):
        cache.store(r.seq, l, r.slot, k[i], v[i])
    o = np.zeros((M, H, hd))
    group = H // Hkv
    for i, r in enumerate(rows):
        K, V = cache.get(r.seq, l)
        vis = np.asarray(r.visible, dtype=np.int64)
        for hh in range(H):
            o[i, hh] = attend(q[i, hh], K[hh // group, vis], V[hh // group, vis])
    h = h + bf16_round(o.reshape(M, H * hd)) @ W(synth.T_WO).T
    x2 = bf16_round(rms_norm(h, W(synth.T_FFN_NORM), cfg.rms_eps))
    g = x2 @ W(synth.T_W_GATE).T
    u = x2 @ W(synth.T_W_UP).T
    return h + bf16_round(silu(g) * u) @ W(synth.T_W_DOWN).T


def head_bf16_inputs(dec, h):
    x = bf16_round(rms_norm(h, dec.w.get(synth.T_FINAL_NORM), dec.cfg.rms_eps))
    return x @ dec.w.get(synth.T_HEAD).T


def main():
    cfg = {"7b": LLAMA7B, "70b": LLAMA70B}[sys.argv[1]]
    P = int(sys.argv[2]) if len(sys.argv) > 2 else 512
    k = int(sys.argv[3]) if len(sys.argv) > 3 else 4
    L = cfg.exit_layer
    n_run = int(sys.argv[4]) if len(sys.argv) > 4 else cfg.n_layers - L
    rng = np.random.default_rng(2024)
    dec = Decoder(cfg, OneLayerWeights(cfg))
    rows = spec.chain_rows(0, P, k + 1)
    caches = [KVCache(cfg, P + k + 2), KVCache(cfg, P + k + 2)]
    h0 = rng.standard_normal((k + 1, cfg.d_model))
    h = [h0.copy(), h0.copy()]
    t0 = time.time()
    for l in range(L, L + n_run):
        Kc = rng.standard_normal((cfg.n_kv_heads, P, cfg.head_dim))
        Vc = rng.standard_normal((cfg.n_kv_heads, P, cfg.head_dim))
        for c in caches:
            K, V = c.get(0, l)
            K[:, :P], V[:, :P] = bf16_round(Kc), bf16_round(Vc)
        h[0] = dec.layer(l, caches[0], rows, h[0])
        h[1] = layer_bf16_inputs(dec, l, caches[1], rows, h[1])
        rel = np.abs(h[1] - h[0]).max() / np.abs(h[0]).max()
        print(f"layer {l}: max |dh| / max |h| = {rel:.3e}  ({time.time() - t0:.0f} s)", flush=True)
    z0, z1 = dec.head(h[0]), head_bf16_inputs(dec, h[1])
    err = np.abs(z1 - z0).max()
    print(f"{sys.argv[1]} P={P} rows={k + 1} layers {L}..{L + n_run - 1} + head: "
          f"max-abs logit difference {err:.3e}, max |logit| {np.abs(z0).max():.3f}, bound 2e-2", flush=True)


if __name__ == "__main__":
    main()

"""Helpers shared by the GPU tests: engines with synthetic weights, device
arrays, and reading the paged KV cache back in slot order."""
import numpy as np
import torch

import synth
from synth import gpu_weights
from synth.model_weights import LAYER_TENSORS, SynthWeights
from oracle.decoder import Decoder
from verification_verify_step_amd import binding as B
from verification_verify_step_amd.runtime import Engine

LOGIT_TOL = 2e-2  # max-abs logit agreement, bf16 weights/KV with fp32 accumulation
NEAR_TIE = 4e-2   # a greedy choice whose top-1 - top-2 gap is below this may legitimately differ


def engine(cfg, eps=None, force_host=False, head_scale=None, **kw):
    e = Engine(cfg, **kw)
    gpu_weights.load(e, cfg, eps=eps, force_host=force_host, head_scale=head_scale)
    return e


def oracle_decoder(cfg, eps=None, head_scale=None):
    w = SynthWeights(cfg, precision="bf16")
    if eps is not None or head_scale is not None:
        w = gpu_weights.ScaledWeights(w, cfg, eps, head_scale)
    return Decoder(cfg, w)


def i32(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), device="cuda")


def f64(a):
    return torch.tensor(np.asarray(a, dtype=np.float64), device="cuda")


def prompt(cfg, n, req=0):
    return synth.tokens(synth.SEED_PROMPTS, synth.stream_prompt(req), cfg.vocab, n)


def uniforms(req, rnd):
    return synth.uniforms(synth.SEED_UNIFORMS, synth.stream_uniform(req, rnd), B.VS_N_UNIFORMS)


def kv_slots(e, seq, layer, slots):
    """K, V of the given slots as float64 arrays [Hkv][n][hd]."""
    K, V, bt = e.kv_layer(layer)
    slots = np.asarray(slots)
    blocks = bt[seq].cpu().numpy()[slots // 16]
    idx_b = torch.from_numpy(blocks.astype(np.int64)).cuda()
    idx_o = torch.from_numpy((slots % 16).astype(np.int64)).cuda()
    k = K[idx_b, :, :, idx_o, :].reshape(len(slots), K.shape[1], -1).permute(1, 0, 2).double().cpu().numpy()
    v = V[idx_b, :, :, idx_o].permute(1, 0, 2).double().cpu().numpy()
    return k, v


def result_rows(res, n_seq):
    r = res[:n_seq].cpu().numpy()
    return [(int(x[0]), int(x[1]), int(x[2]), [int(p) for p in x[4:4 + x[3]]]) for x in r]


def near_tie(z, scale=1.0):
    """Top-1 - top-2 below the band (times the head's scale, which scales the
    logits and their rounding errors alike)."""
    s = np.sort(np.asarray(z, dtype=np.float64))
    return s[-1] - s[-2] < NEAR_TIE * scale


class LayerWeights:
    """The oracle's weights one layer at a time: each tensor is drawn once
    per layer and kept until another layer is asked for (a float64 copy of
    all verify layers of the 7B or 70B shape would not fit in host memory)."""

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

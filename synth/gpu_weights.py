"""Upload the synthetic weights into a library Engine (GPU).

Small tensors come from the host generator (the very bytes the oracle reads);
large ones are drawn on the device by ``libsynth_dev.so`` from the same
stream definition.  Optionally W_o and W_down of the layers >= exit_layer are
scaled by eps (a power of two, so bf16(eps * w) is exact): eps = 0 makes the
target equal to the draft, the acceptance-calibrated synthetic model.  A
head_scale (also a power of two) multiplies the LM head, which sharpens every
output distribution without moving any argmax: a synthetic model whose top-1
probabilities are far from uniform.
"""
import numpy as np
import torch

import synth
from synth import model_weights as mw

HOST_LIMIT = 1 << 22  # elements generated on the host below this size


def upper_scaled(cfg, t, layer, eps):
    return eps is not None and t in (synth.T_WO, synth.T_W_DOWN) and layer >= cfg.exit_layer


def scale_of(cfg, t, layer, eps, head_scale):
    """The factor applied to tensor (t, layer), or None."""
    if upper_scaled(cfg, t, layer, eps):
        return eps
    if head_scale is not None and t == synth.T_HEAD:
        return head_scale
    return None


def tensor_list(cfg):
    out = [(synth.T_EMBED, 0), (synth.T_FINAL_NORM, 0), (synth.T_HEAD, 0)]
    for l in range(cfg.n_layers):
        out += [(t, l) for t in mw.LAYER_TENSORS]
    return out


def device_bits(cfg, t, layer, device, stream, seed=synth.SEED_WEIGHTS, eps=None, force_host=False, head_scale=None):
    """Canonical bf16 bits of one tensor as a contiguous int16 device tensor."""
    shape = mw.tensor_shape(cfg, t)
    n = int(np.prod(shape))
    if t in mw.GAIN_TENSORS:
        src = torch.full((n,), 0x3F80, dtype=torch.int16, device=device)
    elif force_host or n <= HOST_LIMIT:
        bits = mw.bf16_bits(cfg, t, layer, seed).reshape(-1)
        src = torch.from_numpy(bits.view(np.int16)).to(device)
    else:
        src = torch.empty(n, dtype=torch.int16, device=device)
        s = synth.stream_weight(t, mw.tensor_stream_layer(cfg, t, layer))
        synth.dev_normal_bf16(seed, s, n, src.data_ptr(), stream)
    f = scale_of(cfg, t, layer, eps, head_scale)
    if f is not None:
        src = (src.view(torch.bfloat16).float() * f).to(torch.bfloat16).view(torch.int16)
    return src


def load(engine, cfg, seed=synth.SEED_WEIGHTS, eps=None, force_host=False, head_scale=None):
    for t, layer in tensor_list(cfg):
        src = device_bits(cfg, t, layer, engine.device, engine.stream, seed, eps, force_host, head_scale)
        engine.set_tensor(t, layer, src)
        del src
    torch.cuda.synchronize(engine.device)


class ScaledWeights:
    """The oracle's view of the same scaled weights (bf16-exact)."""

    def __init__(self, base, cfg, eps, head_scale=None):
        self.base, self.cfg, self.eps, self.head_scale = base, cfg, eps, head_scale

    def get(self, t, l=0):
        a = self.base.get(t, l)
        f = scale_of(self.cfg, t, l, self.eps, self.head_scale)
        return a * f if f is not None else a

"""The synthetic workloads: model shapes and run parameters of the five decoders.

Shapes follow the Llama family the pages use as their running example
(7B target with a 12-of-32-layer draft: self-speculative decoding page,
m.lqnn.cn/news/278124, §2.3; 70B with GQA for the one-GPU large case).
Every input is synthetic: random-init weights N(0, 0.02) and uniform-random
prompt ids drawn from the seeded streams in ``synth``.
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class ModelCfg:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    exit_layer: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelCfg
    batch: int
    prompt_len: int
    k: int
    mode: str  # "greedy" or "sample"
    temperature: float
    new_tokens: int
    tree: bool = False
    weight_precision: str = "bf16"  # "f32" for the tiny CPU-checkable decoder's own profile
    extra: dict = field(default_factory=dict)


TINY = ModelCfg(n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64, d_ffn=1024, vocab=2048, exit_layer=1)
LLAMA7B = ModelCfg(n_layers=32, d_model=4096, n_heads=32, n_kv_heads=32, head_dim=128, d_ffn=11008, vocab=32000,
                   exit_layer=12)
LLAMA70B = ModelCfg(n_layers=80, d_model=8192, n_heads=64, n_kv_heads=8, head_dim=128, d_ffn=28672, vocab=32000,
                    exit_layer=24)

WORKLOADS = {
    "tiny_chain_k4": Workload("tiny_chain_k4", TINY, batch=1, prompt_len=64, k=4, mode="greedy", temperature=1.0,
                              new_tokens=32, weight_precision="f32"),
    "llama7b_chain_k5": Workload("llama7b_chain_k5", LLAMA7B, batch=1, prompt_len=1024, k=5, mode="greedy",
                                 temperature=1.0, new_tokens=256),
    "llama7b_sample_k4_b8": Workload("llama7b_sample_k4_b8", LLAMA7B, batch=8, prompt_len=2048, k=4, mode="sample",
                                     temperature=1.0, new_tokens=128),
    "llama7b_tree63": Workload("llama7b_tree63", LLAMA7B, batch=1, prompt_len=4096, k=4, mode="greedy",
                               temperature=1.0, new_tokens=1, tree=True, extra={"topk": 5, "depth": 4, "nodes": 63}),
    "llama70b_ragged_b32": Workload("llama70b_ragged_b32", LLAMA70B, batch=32, prompt_len=0, k=16, mode="greedy",
                                    temperature=1.0, new_tokens=1,
                                    extra={"ctx_min": 512, "ctx_max": 8192, "k_min": 2, "k_max": 16, "block": 16}),
}


def ragged_batch(w):
    """Per-request context lengths uniform in [ctx_min, ctx_max] and draft
    lengths uniform in [k_min, k_max] (inclusive), drawn from the workload
    seed: (contexts, draft lengths, pending tokens), one entry per request."""
    import numpy as np

    import synth
    e = w.extra
    n = w.batch
    u_ctx = synth.uniforms(synth.SEED_WORKLOAD, synth.stream_workload(0), n)
    u_k = synth.uniforms(synth.SEED_WORKLOAD, synth.stream_workload(1), n)
    ctx = (e["ctx_min"] + np.floor(u_ctx * (e["ctx_max"] - e["ctx_min"] + 1))).astype(np.int64)
    ks = (e["k_min"] + np.floor(u_k * (e["k_max"] - e["k_min"] + 1))).astype(np.int64)
    pend = synth.tokens(synth.SEED_WORKLOAD, synth.stream_workload(2), w.model.vocab, n)
    return [int(c) for c in ctx], [int(k) for k in ks], [int(t) for t in pend]

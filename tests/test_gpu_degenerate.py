"""Degenerate exit layers through the C ABI on the tiny decoder (2 layers):
* L = N: the draft runs every layer, so it is the target; greedy rounds
  accept every draft, and the tokens are the oracle's greedy tokens;
* L = 0: the draft is the head on the embeddings and the verify runs every
  layer (a plain full-depth verify of k+1 rows); the tokens are again the
  oracle's greedy tokens, the accepted lengths those of the oracle's rounds.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import spec
from oracle.decoder import KVCache
from synth.workloads import TINY
from tests import gpu_common as G
from verification_verify_step_amd import binding as B

pytestmark = pytest.mark.gpu

N_NEW, K = 24, 4


def _run(cfg, req):
    e = G.engine(cfg, force_host=True, max_rows=64, max_seqs=2, max_ctx=256)
    p = G.prompt(cfg, 40, req=req)
    seq = e.open(200)
    B.vs_prefill(e.model, e.kv, seq, G.i32(p).data_ptr(), len(p), B.VS_GREEDY, 1.0, None, None, e.stream)
    toks = torch.zeros(K + 1, dtype=torch.int32, device="cuda")
    res = torch.zeros((1, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    out, accepted = [e.state()[1][seq]], []
    while len(out) < N_NEW:
        B.vs_step(e.model, e.kv, [seq], [K], B.VS_GREEDY, 1.0, None, toks.data_ptr(), res.data_ptr(), e.stream)
        a, y, _, _ = G.result_rows(res, 1)[0]
        out += toks[1:a + 1].cpu().tolist() + [y]
        accepted.append(a)
        P, pending, committed = e.state()
        assert P[seq] == len(p) + len(out) - 1 and committed[seq] == P[seq] + 1
    B.vs_seq_close(e.kv, seq)
    return p, out, accepted


def _oracle(cfg, p, n):
    dec = G.oracle_decoder(cfg)
    cache = KVCache(cfg, 256)
    st, z0 = spec.prefill(dec, cache, 0, p)
    ref, zs = [st.pending], [z0]
    while len(ref) < n:
        y, z = spec.ar_step(dec, cache, st)
        ref.append(y)
        zs.append(z)
    return dec, ref, zs


def test_exit_at_the_last_layer_accepts_everything():
    cfg = dataclasses.replace(TINY, exit_layer=TINY.n_layers)
    p, out, accepted = _run(cfg, req=40)
    assert all(a == K for a in accepted), accepted
    _, ref, zs = _oracle(cfg, p, len(out))
    tie = next((j for j in range(len(out)) if G.near_tie(zs[j])), len(out))
    assert out[:tie + 1] == ref[:tie + 1]


def test_exit_at_layer_zero_is_a_full_depth_verify():
    cfg = dataclasses.replace(TINY, exit_layer=0)
    p, out, accepted = _run(cfg, req=41)
    dec, ref, zs = _oracle(cfg, p, len(out))
    tie = next((j for j in range(len(out)) if G.near_tie(zs[j])), len(out))
    assert out[:tie + 1] == ref[:tie + 1]
    # the oracle's own rounds from the same prompt accept the same counts
    # while no draft or target choice is a near-tie
    cache = KVCache(cfg, 256)
    st, _ = spec.prefill(dec, cache, 0, p)
    for r, a_gpu in enumerate(accepted):
        toks, zd, hL = spec.draft_chain(dec, cache, st, K)
        zt = spec.verify_chain(dec, cache, st, toks, hL)
        a, y = spec.accept_greedy_chain(toks, zt)
        if any(G.near_tie(z) for z in zd) or any(G.near_tie(z) for z in zt[:a + 1]):
            break
        assert a == a_gpu, (r, a, a_gpu)
        spec.commit_chain(cache, st, toks, a, y)

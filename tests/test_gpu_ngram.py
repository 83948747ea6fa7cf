"""Prompt-copy (n-gram) drafting with a full-depth verify ("self-speculative"
page, §2.2) through the C ABI on the tiny decoder: every round's proposal
equals the oracle's proposal from the same history, the committed tokens equal
the oracle's greedy tokens up to its first near-tie, and the state invariant
holds after every round.  The random tiny model repeats itself, so copied
drafts are accepted."""
import numpy as np
import pytest
import torch

from oracle import spec
from oracle.decoder import KVCache
from synth.workloads import TINY
from tests import gpu_common as G
from verification_verify_step_amd import binding as B

pytestmark = pytest.mark.gpu

CFG = TINY
N_NEW, K_MAX, MIN_G, MAX_G = 48, 8, 1, 3


@pytest.mark.parametrize("req,prompt_only", [(1, False), (3, False), (2, True)])
def test_ngram_rounds(req, prompt_only):
    e = G.engine(CFG, force_host=True, max_rows=64, max_seqs=2, max_ctx=512)
    p = G.prompt(CFG, 64, req=req)
    seq = e.open(480)
    B.vs_prefill(e.model, e.kv, seq, G.i32(p).data_ptr(), len(p), B.VS_GREEDY, 1.0, None, None, e.stream)
    torch.cuda.synchronize()
    hist = [int(t) for t in p] + [e.state()[1][seq]]
    d_toks = torch.zeros(K_MAX + 1, dtype=torch.int32, device="cuda")
    d_res = torch.zeros((1, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    search = len(p) if prompt_only else 1 << 30
    accepted, rounds = 0, 0
    while len(hist) - len(p) < N_NEW:
        want = spec.ngram_propose(hist, min(search, len(hist)), MIN_G, MAX_G, K_MAX)
        res, k = B.vs_step_ngram(e.model, e.kv, seq, hist, search, MIN_G, MAX_G, K_MAX, d_toks.data_ptr(),
                                 d_res.data_ptr(), e.stream)
        assert k == len(want) and d_toks[1:k + 1].cpu().tolist() == want, (rounds, k, want)
        a, y = res[0], res[1]
        assert 0 <= a <= k
        hist += want[:a] + [y]
        P, pending, committed = e.state()
        assert P[seq] == len(hist) - 1 and pending[seq] == y and committed[seq] == len(hist)
        accepted += a
        rounds += 1
    # the oracle's greedy tokens
    dec = G.oracle_decoder(CFG)
    cache = KVCache(CFG, 512)
    st, z0 = spec.prefill(dec, cache, 0, p)
    ref, zs = [st.pending], [z0]
    while len(ref) < N_NEW:
        y, zz = spec.ar_step(dec, cache, st)
        ref.append(y)
        zs.append(zz)
    out = hist[len(p):len(p) + N_NEW]
    tie = next((j for j in range(N_NEW) if G.near_tie(zs[j])), N_NEW)
    assert out[:tie + 1] == ref[:tie + 1], (tie, out, ref)
    if not prompt_only:
        assert accepted > 0 and rounds < N_NEW, (accepted, rounds)
    B.vs_seq_close(e.kv, seq)

"""Limits and degenerate cases through the C ABI on the tiny decoder: the
widest pass the library takes (64 sequences x 17 rows = 1088 verify rows,
k = 16 each) against the oracle for three of its sequences, and inputs past
the limits (empty batch, too many sequences, k above 16, a context at its
capacity, a sequence listed twice) rejected before any device work, with
every state unchanged."""
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
N_SEQ, K, P0 = B.VS_MAX_SEQS, B.VS_MAX_K, 24


@pytest.fixture(scope="module")
def ctx():
    e = G.engine(CFG, force_host=True, max_rows=B.VS_MAX_PASS_ROWS, max_seqs=N_SEQ, max_ctx=128)
    prompts = [G.prompt(CFG, P0, req=100 + i) for i in range(N_SEQ)]
    seqs = []
    for p in prompts:
        s = e.open(P0 + 40)
        B.vs_prefill(e.model, e.kv, s, G.i32(p).data_ptr(), P0, B.VS_GREEDY, 1.0, None, None, e.stream)
        seqs.append(s)
    torch.cuda.synchronize()
    d = {"e": e, "seqs": seqs, "prompts": prompts}
    yield d
    for s in d["seqs"]:
        B.vs_seq_close(e.kv, s)


def _decided(z_gpu, z_ora):
    """A greedy choice both sides must make alike: the oracle's top-1 - top-2
    gap exceeds twice the largest difference between the two logit rows."""
    s = np.sort(z_ora)
    return s[-1] - s[-2] > 2 * np.abs(z_gpu - z_ora).max()


def test_widest_pass(ctx):
    """One round of 64 sequences with k = 16: 64-row draft passes and one
    1088-row verify pass, through vs_draft, vs_verify, vs_accept, vs_commit.
    Every state advances by a + 1.  For sequences 0, 31 and 63 the draft and
    verify logits match the oracle's within the logit tolerance, and the
    drafts, a and y match wherever the choice is decided (the oracle's top-2
    gap exceeds twice the row's GPU-oracle difference)."""
    e, seqs = ctx["e"], ctx["seqs"]
    M = N_SEQ * (K + 1)
    toks = torch.zeros(M, dtype=torch.int32, device="cuda")
    hL = torch.empty((M, CFG.d_model), dtype=torch.float32, device="cuda")
    zd = torch.empty((M, CFG.vocab), dtype=torch.float32, device="cuda")
    zt = torch.empty((M, CFG.vocab), dtype=torch.float32, device="cuda")
    res = torch.zeros((N_SEQ, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    P_before = [e.state()[0][s] for s in seqs]
    batch = B.make_batch(seqs, [K + 1] * N_SEQ)
    B.vs_draft(e.model, e.kv, seqs, [K] * N_SEQ, B.VS_GREEDY, 1.0, None, toks.data_ptr(), hL.data_ptr(),
               zd.data_ptr(), e.stream)
    B.vs_verify(e.model, e.kv, batch, CFG.exit_layer, toks.data_ptr(), hL.data_ptr(), zt.data_ptr(), e.stream)
    B.vs_accept(e.model, batch, B.VS_GREEDY, 1.0, toks.data_ptr(), zt.data_ptr(), None, None, res.data_ptr(),
                e.stream)
    B.vs_commit(e.model, e.kv, batch, res.data_ptr(), e.stream)
    torch.cuda.synchronize()
    got = G.result_rows(res, N_SEQ)
    P, pending, committed = e.state()
    t = toks.cpu().numpy()
    for i, s in enumerate(seqs):
        a, y = got[i][0], got[i][1]
        assert 0 <= a <= K and P[s] == P_before[i] + a + 1 and pending[s] == y and committed[s] == P[s] + 1
    zdh, zth = zd.cpu().numpy().astype(np.float64), zt.cpu().numpy().astype(np.float64)
    dec = G.oracle_decoder(CFG)
    decided_rows = 0
    for i in (0, 31, 63):
        r0 = i * (K + 1)
        cache = KVCache(CFG, 128)
        st, _ = spec.prefill(dec, cache, 0, ctx["prompts"][i])
        toks_o, zd_o, hL_o = spec.draft_chain(dec, cache, st, K)
        # drafts: equal while every earlier choice was decided
        j = 0
        while j < K:
            assert np.abs(zdh[r0 + j] - zd_o[j]).max() <= G.LOGIT_TOL
            if not _decided(zdh[r0 + j], zd_o[j]):
                break
            assert t[r0 + j + 1] == toks_o[j + 1], (i, j)
            j += 1
        decided_rows += j
        if j < K:
            continue  # later drafts differ legitimately; the verify rows see other inputs
        zt_o = spec.verify_chain(dec, cache, st, toks_o, hL_o)
        assert np.abs(zth[r0:r0 + K + 1] - zt_o).max() <= G.LOGIT_TOL
        a, y = spec.accept_greedy_chain(toks_o, zt_o)
        if all(_decided(zth[r0 + r], zt_o[r]) for r in range(a + 1)):
            assert (got[i][0], got[i][1]) == (a, y), (i, got[i][:2], a, y)
    assert decided_rows >= 8, decided_rows


def test_inputs_past_the_limits(ctx):
    e, seqs = ctx["e"], ctx["seqs"]
    toks = torch.zeros(B.VS_MAX_PASS_ROWS + 64, dtype=torch.int32, device="cuda")
    res = torch.zeros((N_SEQ + 1, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    # make room for a sequence with a small capacity
    B.vs_seq_close(e.kv, seqs[-1])
    keep = seqs[:-1]
    small = e.open(P0 + 4)
    B.vs_prefill(e.model, e.kv, small, G.i32(ctx["prompts"][1]).data_ptr(), P0, B.VS_GREEDY, 1.0, None, None,
                 e.stream)
    torch.cuda.synchronize()
    before = e.state()
    cases = [
        ([], [], B.VS_E_SHAPE),                                  # empty batch
        (keep + [small, keep[0]], [1] * (N_SEQ + 1), B.VS_E_SHAPE),  # 65 sequences
        (keep[:1], [K + 1], B.VS_E_INVAL),                       # k above 16
        (keep[:1], [-1], B.VS_E_INVAL),                          # negative k
        ([keep[0], keep[0]], [1, 1], B.VS_E_INVAL),              # a sequence twice
        ([small], [8], B.VS_E_NOKV),                             # capacity P0 + 4 cannot take 9 more slots
    ]
    for sq, ks, code in cases:
        with pytest.raises(B.VsError) as err:
            B.vs_step(e.model, e.kv, sq, ks, B.VS_GREEDY, 1.0, None, toks.data_ptr(), res.data_ptr(), e.stream)
        assert err.value.code == code, (sq[:2], ks[:2], err.value)
    torch.cuda.synchronize()
    after = e.state()
    for s in keep + [small]:
        assert [x[s] for x in after] == [x[s] for x in before]
    # the same context still takes a round that fits
    P_small = after[0][small]
    B.vs_step(e.model, e.kv, [small], [2], B.VS_GREEDY, 1.0, None, toks.data_ptr(), res.data_ptr(), e.stream)
    torch.cuda.synchronize()
    a = G.result_rows(res, 1)[0][0]
    assert e.state()[0][small] == P_small + a + 1
    B.vs_seq_close(e.kv, small)
    ctx["seqs"] = keep

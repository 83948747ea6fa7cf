"""Full-depth verify parity at the 7B shape (32 layers, d 4096, 32x128 heads,
FFN 11008, V 32000, bf16, draft = first 12 layers).  The verify runs layers
L..N-1 over the k+1 positions (or the tree's rows) and then the head
(self-speculative decoding page, m.lqnn.cn/news/278124, §4.3; "FlashSpec"
page, lnrk.cn/news/47842, §2.2 for the tree batch).

Three passes on one engine, each in the launch configuration the benchmark
times:
* the chain of the headline workload: context 1024, k = 5 greedy (6 rows);
* the stochastic batch: 8 requests at context 2048, k = 4 drafted by
  sampling at T = 1 (40 rows); request 0 is compared;
* the 64-row token tree at context 4096.
For each, the GPU's verify logits are compared with the float64 oracle
chained through the same 20 layers and the head, starting from the same
layer-12 rows (the GPU draft's) and the committed KV the GPU wrote: max-abs
<= 2e-2.  Also: a sequence's verify logits are bit-identical alone and in
passes with other sequences (every kernel's arithmetic is fixed per row),
and repeating a pass gives the same bits (the cross-workgroup combines of
attention and of the K-split GEMM)."""
import numpy as np
import pytest
import torch

from oracle import spec
from oracle.decoder import Decoder, KVCache, Row
from synth.workloads import LLAMA7B
from tests import gpu_common as G
from tests.test_gpu_tree import DEPTH, KEEP, R, T, TOPK, draft_tree
from verification_verify_step_amd import binding as B

pytestmark = pytest.mark.gpu

CFG = LLAMA7B
L, N = CFG.exit_layer, CFG.n_layers
P_CHAIN, K_CHAIN = 1024, 5
P_REQ, K_REQ, N_REQ = 2048, 4, 8
P_TREE = 4096


def _verify(e, seqs, rows, toks, hL, depth=None, mask=None):
    M = sum(rows)
    z = torch.empty((M, CFG.vocab), dtype=torch.float32, device="cuda")
    batch = B.make_batch(seqs, rows, depth, mask)
    B.vs_verify(e.model, e.kv, batch, L, toks.data_ptr(), hL.data_ptr(), z.data_ptr(), e.stream)
    torch.cuda.synchronize()
    return z


@pytest.fixture(scope="module")
def ctx():
    e = G.engine(CFG, max_rows=128, max_seqs=12, max_ctx=P_TREE + 160)
    st = e.stream
    out = {"e": e}
    # the chain
    a = e.open(P_CHAIN + 150)
    B.vs_prefill(e.model, e.kv, a, G.i32(G.prompt(CFG, P_CHAIN, req=0)).data_ptr(), P_CHAIN, B.VS_GREEDY, 1.0, None,
                 None, st)
    toks = torch.empty(K_CHAIN + 1, dtype=torch.int32, device="cuda")
    hL = torch.empty((K_CHAIN + 1, CFG.d_model), dtype=torch.float32, device="cuda")
    B.vs_draft(e.model, e.kv, [a], [K_CHAIN], B.VS_GREEDY, 1.0, None, toks.data_ptr(), hL.data_ptr(), None, st)
    out["chain"] = (a, toks, hL)
    # the stochastic batch: 8 requests, sampled drafts
    reqs = []
    for r in range(N_REQ):
        s = e.open(P_REQ + 150)
        B.vs_prefill(e.model, e.kv, s, G.i32(G.prompt(CFG, P_REQ, req=20 + r)).data_ptr(), P_REQ, B.VS_GREEDY, 1.0,
                     None, None, st)
        reqs.append(s)
    Mb = N_REQ * (K_REQ + 1)
    U = np.stack([G.uniforms(20 + r, 1) for r in range(N_REQ)])
    du = G.f64(U.reshape(-1))
    tb = torch.empty(Mb, dtype=torch.int32, device="cuda")
    hb = torch.empty((Mb, CFG.d_model), dtype=torch.float32, device="cuda")
    zd = torch.empty((Mb, CFG.vocab), dtype=torch.float32, device="cuda")
    B.vs_draft(e.model, e.kv, reqs, [K_REQ] * N_REQ, B.VS_SAMPLE, 1.0, du.data_ptr(), tb.data_ptr(), hb.data_ptr(),
               zd.data_ptr(), st)
    out["batch"] = (reqs, tb, hb)
    # the tree
    c = e.open(P_TREE + 150)
    B.vs_prefill(e.model, e.kv, c, G.i32(G.prompt(CFG, P_TREE, req=3)).data_ptr(), P_TREE, B.VS_GREEDY, 1.0, None,
                 None, st)
    torch.cuda.synchronize()
    out["tree"] = (c, draft_tree(e, c, CFG))
    torch.cuda.synchronize()
    yield out
    for s in [a, c] + reqs:
        B.vs_seq_close(e.kv, s)
    e.close()
    del out, e
    torch.cuda.empty_cache()


def _chain_rows(P, n):
    return spec.chain_rows(0, P, n)


def _tree_rows(tr, P):
    depth = tr["depth"].cpu().tolist()
    mask = tr["mask"].cpu().numpy().view(np.uint64)
    rows = []
    for r in range(R):
        vis = [P + j for j in range(R) if (int(mask[r]) >> j) & 1]
        rows.append(Row(0, P + depth[r], P + r, np.concatenate([np.arange(P), np.array(vis)])))
    return rows


def _oracle_verify(e, passes):
    """passes: (seq, oracle rows, layer-L rows float64).  Layers L..N-1 and
    the head in float64, each pass over the committed KV (slots 0..P-1) the
    GPU holds for its sequence."""
    dec = Decoder(CFG, G.LayerWeights(CFG))
    hs = [h.copy() for _, _, h in passes]
    P = e.state()[0]
    for l in range(L, N):
        for j, (seq, rows, _) in enumerate(passes):
            cache = KVCache(CFG, P[seq] + len(rows) + 1)
            k, v = G.kv_slots(e, seq, l, np.arange(P[seq]))
            Kc, Vc = cache.get(0, l)
            Kc[:, :P[seq]], Vc[:, :P[seq]] = k, v
            hs[j] = dec.layer(l, cache, rows, hs[j])
    return [dec.head(h) for h in hs]


def test_full_depth_logits_vs_oracle(ctx):
    """GPU verify logits of the chain, request 0 of the stochastic batch and
    the tree against the oracle's 20 verify layers + head: max-abs <= 2e-2."""
    e = ctx["e"]
    P = e.state()[0]
    a, ta, ha = ctx["chain"]
    reqs, tb, hb = ctx["batch"]
    c, tr = ctx["tree"]
    za = _verify(e, [a], [K_CHAIN + 1], ta, ha)
    zb = _verify(e, reqs, [K_REQ + 1] * N_REQ, tb, hb)[:K_REQ + 1]
    zc = _verify(e, [c], [R], tr["tok"], tr["hL"], tr["depth"].data_ptr(), tr["mask"].data_ptr())
    passes = [
        (a, _chain_rows(P[a], K_CHAIN + 1), ha.cpu().numpy().astype(np.float64)),
        (reqs[0], _chain_rows(P[reqs[0]], K_REQ + 1), hb[:K_REQ + 1].cpu().numpy().astype(np.float64)),
        (c, _tree_rows(tr, P[c]), tr["hL"].cpu().numpy().astype(np.float64)),
    ]
    zo = _oracle_verify(e, passes)
    for name, zg, z in (("chain", za, zo[0]), ("request", zb, zo[1]), ("tree", zc, zo[2])):
        err = np.abs(zg.cpu().numpy().astype(np.float64) - z).max()
        assert err <= G.LOGIT_TOL, (name, err)


def test_rows_invariant_to_batch(ctx):
    """A sequence's logits do not depend on the sequences beside it: the chain
    alone, with the 8 requests (the one-group attention kernel then runs
    several chunks per workgroup) and with the tree (a pass that runs both
    attention kernels), and the tree and the requests alone against the same
    passes: bit-identical."""
    e = ctx["e"]
    a, ta, ha = ctx["chain"]
    reqs, tb, hb = ctx["batch"]
    c, tr = ctx["tree"]
    za = _verify(e, [a], [K_CHAIN + 1], ta, ha)
    zb = _verify(e, reqs, [K_REQ + 1] * N_REQ, tb, hb)
    zc = _verify(e, [c], [R], tr["tok"], tr["hL"], tr["depth"].data_ptr(), tr["mask"].data_ptr())
    ma = K_CHAIN + 1
    # chain + 8 requests
    zab = _verify(e, [a] + reqs, [ma] + [K_REQ + 1] * N_REQ, torch.cat([ta, tb]), torch.cat([ha, hb]))
    assert torch.equal(zab[:ma], za)
    assert torch.equal(zab[ma:], zb)
    # chain + tree: chain masks (all bits up to the row) and depths for the chain rows
    depth = torch.cat([torch.arange(ma, dtype=torch.int32, device="cuda"), tr["depth"]])
    chain_mask = torch.tensor([(2 << i) - 1 for i in range(ma)], dtype=torch.int64, device="cuda")
    mask = torch.cat([chain_mask, tr["mask"]])
    zac = _verify(e, [a, c], [ma, R], torch.cat([ta, tr["tok"]]), torch.cat([ha, tr["hL"]]), depth.data_ptr(),
                  mask.data_ptr())
    assert torch.equal(zac[:ma], za)
    assert torch.equal(zac[ma:], zc)
    # request 3 alone
    r3 = slice(3 * (K_REQ + 1), 4 * (K_REQ + 1))
    z3 = _verify(e, [reqs[3]], [K_REQ + 1], tb[r3].contiguous(), hb[r3].contiguous())
    assert torch.equal(z3, zb[r3])


def test_repeated_passes_bit_identical(ctx):
    """The 40-row pass of the stochastic batch (the down projection splits K
    over workgroups; attention runs nine chunks per workgroup) and the
    64-row tree pass (grouped attention, 16 splits and the combine kernel),
    repeated: the same bits every time."""
    e = ctx["e"]
    reqs, tb, hb = ctx["batch"]
    c, tr = ctx["tree"]
    ref_b = _verify(e, reqs, [K_REQ + 1] * N_REQ, tb, hb)
    ref_c = _verify(e, [c], [R], tr["tok"], tr["hL"], tr["depth"].data_ptr(), tr["mask"].data_ptr())
    for _ in range(6):
        assert torch.equal(_verify(e, reqs, [K_REQ + 1] * N_REQ, tb, hb), ref_b)
        assert torch.equal(_verify(e, [c], [R], tr["tok"], tr["hL"], tr["depth"].data_ptr(), tr["mask"].data_ptr()),
                           ref_c)

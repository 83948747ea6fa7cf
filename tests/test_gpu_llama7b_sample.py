"""GPU parity for stochastic verification at the 7B shape: 8 independent
requests with 2048-token prompts, temperature 1, chain k = 4, so one verify
pass carries 40 rows.  The oracle checks sampled outputs: one verify layer of
two of the requests given the GPU's layer input and committed KV, the head on
the GPU's final hidden rows, the draft's samples and the accept decisions
under shared uniforms on identical logits.  The distribution of the GPU's
rejection sampling is checked by chi-square on a 16-id vocabulary."""
import numpy as np
import pytest
import torch

from oracle import spec
from oracle.decoder import Decoder, KVCache
from synth.model_weights import SynthWeights
from synth.workloads import LLAMA7B, ModelCfg
from tests import gpu_common as G
from verification_verify_step_amd import binding as B

pytestmark = pytest.mark.gpu

CFG = LLAMA7B
N_REQ, P0, K, T = 8, 2048, 4, 1.0
M = N_REQ * (K + 1)
CDF_BAND = 1e-9  # a draw this close (relative) to a CDF boundary may legitimately differ


@pytest.fixture(scope="module")
def ctx():
    e = G.engine(CFG, max_rows=64, max_seqs=N_REQ, max_ctx=P0 + 64)
    seqs = []
    for i in range(N_REQ):
        s = e.open(P0 + 48)
        du = G.f64(G.uniforms(i, 0))
        B.vs_prefill(e.model, e.kv, s, G.i32(G.prompt(CFG, P0, req=i)).data_ptr(), P0, B.VS_SAMPLE, T,
                     du.data_ptr(), None, e.stream)
        seqs.append(s)
    U = np.stack([G.uniforms(i, 1) for i in range(N_REQ)])
    du = G.f64(U.reshape(-1))
    toks = torch.empty(M, dtype=torch.int32, device="cuda")
    hL = torch.empty((M, CFG.d_model), dtype=torch.float32, device="cuda")
    zd = torch.empty((M, CFG.vocab), dtype=torch.float32, device="cuda")
    B.vs_draft(e.model, e.kv, seqs, [K] * N_REQ, B.VS_SAMPLE, T, du.data_ptr(), toks.data_ptr(), hL.data_ptr(),
               zd.data_ptr(), e.stream)
    torch.cuda.synchronize()
    yield {"e": e, "seqs": seqs, "U": U, "toks": toks, "hL": hL, "zd": zd,
           "batch": B.make_batch(seqs, [K + 1] * N_REQ)}
    for s in seqs:
        B.vs_seq_close(e.kv, s)


def _forward(e, batch, start, end, toks, hin):
    out = torch.empty((M, CFG.d_model), dtype=torch.float32, device="cuda")
    B.vs_forward_layers(e.model, e.kv, batch, start, end, toks.data_ptr(), hin.data_ptr() if hin is not None else None,
                        out.data_ptr(), e.stream)
    return out


def test_draft_samples_follow_the_draft_distribution(ctx):
    """Each drafted token is the inverse-CDF draw from softmax(z/T) of the
    draft logits that produced it, with uniform slot s of its request."""
    toks = ctx["toks"].cpu().numpy()
    zd = ctx["zd"].cpu().numpy().astype(np.float64)
    U = ctx["U"]
    checked = 0
    for i in range(N_REQ):
        for s in range(K):
            r = i * (K + 1) + s
            w = spec.probs(zd[r], T)
            C = np.cumsum(w)
            j = spec.sample_index(w, U[i][s])
            edge = np.min(np.abs(C - U[i][s] * C[-1])) < CDF_BAND * C[-1]
            if not edge:
                assert toks[r + 1] == j, (i, s, toks[r + 1], j)
                checked += 1
    assert checked >= N_REQ * K - 1


@pytest.mark.parametrize("layer", [12, 27])
def test_layer_parity_40_rows(ctx, layer):
    """One verify layer over all 40 rows on the GPU; requests 0 and 5
    recomputed by the oracle from the GPU's layer input and committed KV."""
    e, seqs, batch = ctx["e"], ctx["seqs"], ctx["batch"]
    X = ctx["hL"] if layer == CFG.exit_layer else _forward(e, batch, CFG.exit_layer, layer, ctx["toks"], ctx["hL"])
    Y = _forward(e, batch, layer, layer + 1, ctx["toks"], X)
    torch.cuda.synchronize()
    Xh, Yh = X.cpu().numpy().astype(np.float64), Y.cpu().numpy().astype(np.float64)
    dec = Decoder(CFG, SynthWeights(CFG, precision="bf16", cache=True))
    for i in (0, 5):
        s = seqs[i]
        P = e.state()[0][s]
        cache = KVCache(CFG, P + K + 2)
        k, v = G.kv_slots(e, s, layer, np.arange(P))
        Kc, Vc = cache.get(0, layer)
        Kc[:, :P], Vc[:, :P] = k, v
        rs = slice(i * (K + 1), (i + 1) * (K + 1))
        Yo = dec.layer(layer, cache, spec.chain_rows(0, P, K + 1), Xh[rs])
        scale = np.abs(Yo).max()
        err = np.abs(Yh[rs] - Yo).max()
        assert err <= 1e-3 * scale + 1e-4, (layer, i, err, scale)


def test_layer_rows_identical_alone_and_in_the_pass(ctx):
    """A request's rows of one verify layer carry the same bits alone (5
    rows: 32 attention units, one chunk per workgroup and the cross-workgroup
    combine; skinny GEMMs) as inside the 40-row pass (256 units: one
    workgroup per unit runs all 17 chunks; 40-row GEMM forms).  Both passes
    append the same in-round K/V, since the QKV rows do not depend on the
    pass either."""
    e, seqs, batch = ctx["e"], ctx["seqs"], ctx["batch"]
    layer = CFG.exit_layer
    X, toks = ctx["hL"], ctx["toks"]
    Y = _forward(e, batch, layer, layer + 1, toks, X)
    torch.cuda.synchronize()
    for i in (0, 5):
        rs = slice(i * (K + 1), (i + 1) * (K + 1))
        out = torch.empty((K + 1, CFG.d_model), dtype=torch.float32, device="cuda")
        B.vs_forward_layers(e.model, e.kv, B.make_batch([seqs[i]], [K + 1]), layer, layer + 1, toks[rs].data_ptr(),
                            X[rs].data_ptr(), out.data_ptr(), e.stream)
        torch.cuda.synchronize()
        assert torch.equal(out, Y[rs]), (i, (out - Y[rs]).abs().max().item())


def test_head_and_stochastic_accept(ctx):
    """Verify logits of sampled rows against the oracle head; accept decisions
    of all 8 requests on the GPU's own logits equal the oracle's
    accept_or_reject with the same uniforms, except flagged near-ties."""
    e, batch = ctx["e"], ctx["batch"]
    Y = _forward(e, batch, CFG.exit_layer, CFG.n_layers, ctx["toks"], ctx["hL"])
    z = torch.empty((M, CFG.vocab), dtype=torch.float32, device="cuda")
    B.vs_head(e.model, M, Y.data_ptr(), z.data_ptr(), e.stream)
    res = torch.zeros((N_REQ, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    du = G.f64(ctx["U"].reshape(-1))
    B.vs_accept(e.model, batch, B.VS_SAMPLE, T, ctx["toks"].data_ptr(), z.data_ptr(), ctx["zd"].data_ptr(),
                du.data_ptr(), res.data_ptr(), e.stream)
    torch.cuda.synchronize()
    zg = z.cpu().numpy().astype(np.float64)
    sample = [0, 7, 13, 22, 39]
    dec = Decoder(CFG, SynthWeights(CFG, precision="bf16", cache=True))
    zo = dec.head(Y.cpu().numpy().astype(np.float64)[sample])
    assert np.abs(zg[sample] - zo).max() <= G.LOGIT_TOL, np.abs(zg[sample] - zo).max()
    got = G.result_rows(res, N_REQ)
    toks = ctx["toks"].cpu().numpy()
    zd = ctx["zd"].cpu().numpy().astype(np.float64)
    flagged = 0
    for i in range(N_REQ):
        rs = slice(i * (K + 1), (i + 1) * (K + 1))
        pr = [spec.probs(r, T) for r in zg[rs]]
        qr = [spec.probs(r, T) for r in zd[rs]]
        a, y, flags = spec.accept_stochastic_chain(list(toks[rs]), pr, qr, ctx["U"][i])
        assert bool(got[i][2] & 1) == bool(flags), (i, got[i][2], flags)  # the same near-ties are flagged
        if flags:
            flagged += 1
            continue
        assert (got[i][0], got[i][1]) == (a, y), (i, got[i], a, y)
        assert got[i][3] == list(range(1, a + 1))
    assert flagged <= 2


def test_top_p_accept(ctx):
    """Accept with the target truncated to its top-0.9 set, on the verify
    logits of the 8 requests (full vocabulary) and the draft logits: the
    decisions equal the oracle's test against top_p_filter(p) with the same
    uniforms, except flagged near-ties (ratio within 1e-3 of u, or a row
    whose cumulative probability lies within 1e-9 of 0.9 at the boundary)."""
    e, batch = ctx["e"], ctx["batch"]
    Y = _forward(e, batch, CFG.exit_layer, CFG.n_layers, ctx["toks"], ctx["hL"])
    z = torch.empty((M, CFG.vocab), dtype=torch.float32, device="cuda")
    B.vs_head(e.model, M, Y.data_ptr(), z.data_ptr(), e.stream)
    res = torch.zeros((N_REQ, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    du = G.f64(ctx["U"].reshape(-1))
    top_p = 0.9
    B.vs_accept_top_p(e.model, batch, T, top_p, ctx["toks"].data_ptr(), z.data_ptr(), ctx["zd"].data_ptr(),
                      du.data_ptr(), res.data_ptr(), e.stream)
    torch.cuda.synchronize()
    got = G.result_rows(res, N_REQ)
    zg = z.cpu().numpy().astype(np.float64)
    zd = ctx["zd"].cpu().numpy().astype(np.float64)
    toks = ctx["toks"].cpu().numpy()
    flagged = 0
    for i in range(N_REQ):
        rs = slice(i * (K + 1), (i + 1) * (K + 1))
        pr_full = [spec.probs(r, T) for r in zg[rs]]
        if min(spec.top_p_margin(p, top_p) for p in pr_full) < 1e-9:
            flagged += 1
            continue
        pr = [spec.top_p_filter(p, top_p) for p in pr_full]
        qr = [spec.probs(r, T) for r in zd[rs]]
        a, y, flags = spec.accept_stochastic_chain(list(toks[rs]), pr, qr, ctx["U"][i])
        assert bool(got[i][2] & 1) == bool(flags), (i, got[i][2], flags)  # the same near-ties are flagged
        if flags:
            flagged += 1
            continue
        assert (got[i][0], got[i][1]) == (a, y), (i, got[i], a, y)
        assert pr[min(a, K)][y] > 0 or a < K  # the bonus comes from the truncated target
    assert flagged <= 2


@pytest.mark.parametrize("scale,top_p", [(1.0, 0.9), (4.0, 0.5), (8.0, 0.9), (8.0, 0.99)])
def test_top_p_set_at_full_vocabulary(ctx, scale, top_p):
    """The top-p set over 32000 ids, seen through the bonus draw of one-row
    chains (no drafts): y is the oracle's inverse-CDF draw from the truncated
    target with the same uniform.  Logits are seeded normals times a scale
    (flat to sharp distributions, nuclei from a few ids to most of the
    vocabulary).  Draws within 1e-9 (relative) of a CDF boundary and rows
    whose cumulative probability lies within 1e-9 of top_p at the set's edge
    are skipped."""
    e = ctx["e"]
    n = N_REQ
    rng = np.random.default_rng(int(scale * 100 + top_p * 10))
    zl = (rng.standard_normal((n, CFG.vocab)) * scale).astype(np.float32)
    z = torch.from_numpy(zl).cuda()
    U = rng.random((n, B.VS_N_UNIFORMS))
    batch = B.make_batch(ctx["seqs"], [1] * n)
    toks = G.i32(np.zeros(n, dtype=np.int32))
    res = torch.zeros((n, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    B.vs_accept_top_p(e.model, batch, 1.0, top_p, toks.data_ptr(), z.data_ptr(), z.data_ptr(),
                      G.f64(U.reshape(-1)).data_ptr(), res.data_ptr(), e.stream)
    torch.cuda.synchronize()
    got = G.result_rows(res, n)
    checked = 0
    for i in range(n):
        p = spec.probs(zl[i].astype(np.float64), 1.0)
        if spec.top_p_margin(p, top_p) < 1e-9:
            continue
        pt = spec.top_p_filter(p, top_p)
        C = np.cumsum(pt)
        if np.min(np.abs(C - U[i][spec.SLOT_RESAMPLE] * C[-1])) < CDF_BAND * C[-1]:
            continue
        assert got[i][0] == 0 and got[i][1] == spec.sample_index(pt, U[i][spec.SLOT_RESAMPLE]), (i, got[i])
        assert pt[got[i][1]] > 0
        checked += 1
    assert checked >= n - 2


def test_verify_confidence(ctx):
    """vs_confidence on the verify logits of the 8 requests (5 rows each, full
    vocabulary) equals the oracle's mean top-1 probability and mean top-1/top-2
    gap of the same logits, at T = 1 and T = 0.7."""
    e, batch = ctx["e"], ctx["batch"]
    Y = _forward(e, batch, CFG.exit_layer, CFG.n_layers, ctx["toks"], ctx["hL"])
    z = torch.empty((M, CFG.vocab), dtype=torch.float32, device="cuda")
    B.vs_head(e.model, M, Y.data_ptr(), z.data_ptr(), e.stream)
    conf = torch.zeros((N_REQ, 2), dtype=torch.float64, device="cuda")
    for temp in (1.0, 0.7):
        B.vs_confidence(e.model, batch, temp, z.data_ptr(), conf.data_ptr(), e.stream)
        torch.cuda.synchronize()
        got = conf.cpu().numpy()
        zg = z.cpu().numpy().astype(np.float64)
        for i in range(N_REQ):
            # the ABI takes the temperature as a float: the oracle divides by that value
            t1, g = spec.row_confidence(zg[i * (K + 1):(i + 1) * (K + 1)], float(np.float32(temp)))
            assert abs(got[i, 0] - t1) <= 1e-10 and abs(got[i, 1] - g) <= 1e-10, (temp, i, got[i], t1, g)


def test_rounds_keep_the_state_invariant(ctx):
    """Stochastic rounds through vs_step: every request advances by a + 1 and
    keeps committed == P + 1."""
    e, seqs = ctx["e"], ctx["seqs"]
    toks = torch.empty(64, dtype=torch.int32, device="cuda")
    res = torch.zeros((N_REQ, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    for rnd in range(2, 5):
        P_before = [e.state()[0][s] for s in seqs]
        du = G.f64(np.stack([G.uniforms(i, rnd) for i in range(N_REQ)]).reshape(-1))
        B.vs_step(e.model, e.kv, seqs, [K] * N_REQ, B.VS_SAMPLE, T, du.data_ptr(), toks.data_ptr(), res.data_ptr(),
                  e.stream)
        e.sync()
        P_after, pend, committed = e.state()
        for i, s in enumerate(seqs):
            a, y, _, path = G.result_rows(res, N_REQ)[i]
            assert 0 <= a <= K and 0 <= y < CFG.vocab
            assert P_after[s] == P_before[i] + a + 1
            assert committed[s] == P_after[s] + 1 and pend[s] == y


# ---------------------------------------------------------------------------
# Distribution of the GPU's rejection sampling (16-id vocabulary).

SMALL = ModelCfg(n_layers=1, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64, d_ffn=256, vocab=16, exit_layer=1)


def test_rejection_sampling_chi_square():
    """The first emitted token of a k = 1 round (the draft token if accepted,
    else the residual draw) is distributed as the target p, including ids
    where p or q is zero (1e5 seeded trials, 16 ids)."""
    _chi_square_first_token(None)


def test_rejection_sampling_top_p_chi_square():
    """The same with the target truncated to its top-0.8 set on the verify
    side (drafts still from the full q): the first token follows the
    truncated target, ids outside the set never appear."""
    _chi_square_first_token(0.8)


def _chi_square_first_token(top_p):
    from scipy.stats import chi2

    n_seq = 32  # 2 rows each: the 64-row limit of one pass
    e = G.engine(SMALL, force_host=True, max_rows=64, max_seqs=n_seq, max_ctx=64)
    seqs = [e.open(16) for _ in range(n_seq)]
    batch = B.make_batch(seqs, [2] * n_seq)
    V = SMALL.vocab
    zp = np.array([1.0, 0.5, -np.inf, 2.0, 0.0, -1.0, 1.5, -np.inf, 0.3, 0.8, -0.5, 1.2, -np.inf, 0.1, 2.2, 0.4],
                  dtype=np.float32)
    zq = np.array([0.2, 1.5, 1.0, 0.5, -np.inf, 0.7, 1.0, 0.0, -np.inf, 2.0, 0.1, 0.3, 0.9, -0.3, 0.5, 1.1],
                  dtype=np.float32)
    p = spec.probs(zp.astype(np.float64), 1.0)
    if top_p is not None:
        assert spec.top_p_margin(p, top_p) > 1e-6
        p = spec.top_p_filter(p, top_p)
    q = spec.probs(zq.astype(np.float64), 1.0)
    zt = torch.from_numpy(np.tile(zp, (2 * n_seq, 1))).cuda()
    zd = torch.from_numpy(np.tile(zq, (2 * n_seq, 1))).cuda()
    rng = np.random.default_rng(2024)
    res = torch.zeros((n_seq, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    counts = np.zeros(V, dtype=np.int64)
    accepted = 0
    n_calls = 3125  # 100000 trials
    for _ in range(n_calls):
        d1 = rng.choice(V, size=n_seq, p=q)
        toks = np.zeros(2 * n_seq, dtype=np.int32)
        toks[1::2] = d1
        U = rng.random((n_seq, B.VS_N_UNIFORMS))
        if top_p is None:
            B.vs_accept(e.model, batch, B.VS_SAMPLE, 1.0, G.i32(toks).data_ptr(), zt.data_ptr(), zd.data_ptr(),
                        G.f64(U.reshape(-1)).data_ptr(), res.data_ptr(), e.stream)
        else:
            B.vs_accept_top_p(e.model, batch, 1.0, top_p, G.i32(toks).data_ptr(), zt.data_ptr(), zd.data_ptr(),
                              G.f64(U.reshape(-1)).data_ptr(), res.data_ptr(), e.stream)
        r = res[:n_seq, :2].cpu().numpy()
        first = np.where(r[:, 0] >= 1, d1, r[:, 1])
        accepted += int((r[:, 0] >= 1).sum())
        np.add.at(counts, first, 1)
    n = n_calls * n_seq
    assert np.all(counts[p == 0] == 0), counts
    live = p > 0
    expect = p[live] * n
    stat = float(((counts[live] - expect) ** 2 / expect).sum())
    pval = float(chi2.sf(stat, df=int(live.sum()) - 1))
    assert pval > 1e-3, (stat, pval, counts, expect)
    rate = np.minimum(p, q).sum()
    sd = np.sqrt(n * rate * (1 - rate))
    assert abs(accepted - n * rate) < 4 * sd, (accepted, n * rate, sd)
    for s in seqs:
        B.vs_seq_close(e.kv, s)

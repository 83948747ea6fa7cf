"""GPU parity at the 70B shape on one GPU: 80 layers, d 8192, 64 query / 8 KV
heads x 128, FFN 28672, V 32000, bf16, paged KV (block 16), draft = first 24
layers; 32 requests with contexts uniform in [512, 8192] and draft lengths
uniform in [2, 16] (about 330 verify rows per pass).  The committed KV is
written straight into the cache by the seeded generator (N(0, 1) bf16)
instead of 32 prefills of up to 8192 tokens.  The oracle checks sampled
outputs: one verify layer of three requests (shortest, middle, longest
context) from the GPU's layer input and committed KV, the head on sampled
rows, and the greedy accept of every request on the GPU's logits; draft
tokens are the argmax of their draft logits, and the draft's first-L KV
and layer-L inputs are bit-identical to a batched first-L pass.  Rounds: the
confidence-scheduled draft length over several rounds of the whole batch
(starting from the drawn K_r), against plain greedy AR from the same
contexts, on this model and on a calibrated one (upper-layer W_o and W_down
zeroed so every draft is accepted, LM head x4 so the confidence is high)."""
import numpy as np
import pytest
import torch

import synth
from oracle import spec
from oracle.decoder import Decoder, KVCache
from synth.model_weights import SynthWeights
from synth.workloads import LLAMA70B, WORKLOADS, ragged_batch
from tests import gpu_common as G
from verification_verify_step_amd import binding as B

pytestmark = pytest.mark.gpu

CFG = LLAMA70B
W = WORKLOADS["llama70b_ragged_b32"]
CTX, KS, PEND = ragged_batch(W)
N = len(CTX)
ROWS = [k + 1 for k in KS]
M = sum(ROWS)
START = np.concatenate([[0], np.cumsum(ROWS)]).astype(int)
MAX_CTX = max(CTX) + 160
ROUNDS = 3


@pytest.fixture(scope="module")
def ctx():
    bps = (MAX_CTX + 15) // 16 + 2
    n_blocks = sum((c + 160 + 15) // 16 for c in CTX) + 16
    e = G.engine(CFG, max_rows=N * (B.VS_MAX_K + 1), max_seqs=N, max_ctx=MAX_CTX, n_blocks=n_blocks,
                 max_blocks_per_seq=bps)
    st = e.stream
    for layer in range(CFG.n_layers):
        K, V, _ = e.kv_layer(layer)
        synth.dev_normal_bf16(synth.SEED_KV, synth.stream_kv(layer, 0), K.numel(), K.data_ptr(), st, std=1.0)
        synth.dev_normal_bf16(synth.SEED_KV, synth.stream_kv(layer, 1), V.numel(), V.data_ptr(), st, std=1.0)
    seqs = []
    for i in range(N):
        s = e.open(CTX[i] + 150)
        B.vs_seq_assume(e.kv, s, CTX[i], PEND[i], st)
        seqs.append(s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(70)
    hL = torch.from_numpy(rng.standard_normal((M, CFG.d_model)).astype(np.float32)).cuda()
    toks = torch.from_numpy(rng.integers(0, CFG.vocab, M).astype(np.int32)).cuda()
    batch = B.make_batch(seqs, ROWS)
    yield {"e": e, "seqs": seqs, "hL": hL, "toks": toks, "batch": batch}
    for s in seqs:
        B.vs_seq_close(e.kv, s)


def _forward(e, batch, start, end, toks, hin):
    out = torch.empty((M, CFG.d_model), dtype=torch.float32, device="cuda")
    B.vs_forward_layers(e.model, e.kv, batch, start, end, toks.data_ptr(), hin.data_ptr() if hin is not None else None,
                        out.data_ptr(), e.stream)
    return out


def test_state_after_assume(ctx):
    P, pending, committed = ctx["e"].state()
    for i, s in enumerate(ctx["seqs"]):
        assert P[s] == CTX[i] and pending[s] == PEND[i] and committed[s] == CTX[i] + 1


@pytest.mark.parametrize("layer", [CFG.exit_layer, 50])
def test_verify_layer_parity_ragged(ctx, layer):
    e, seqs, batch = ctx["e"], ctx["seqs"], ctx["batch"]
    X = ctx["hL"] if layer == CFG.exit_layer else _forward(e, batch, CFG.exit_layer, layer, ctx["toks"], ctx["hL"])
    Y = _forward(e, batch, layer, layer + 1, ctx["toks"], X)
    torch.cuda.synchronize()
    Xh, Yh = X.cpu().numpy().astype(np.float64), Y.cpu().numpy().astype(np.float64)
    dec = Decoder(CFG, SynthWeights(CFG, precision="bf16", cache=True))
    order = np.argsort(CTX)
    for i in (int(order[0]), int(order[N // 2]), int(order[-1])):
        P = CTX[i]
        cache = KVCache(CFG, P + ROWS[i] + 1)
        k, v = G.kv_slots(e, seqs[i], layer, np.arange(P))
        Kc, Vc = cache.get(0, layer)
        Kc[:, :P], Vc[:, :P] = k, v
        rs = slice(START[i], START[i + 1])
        Yo = dec.layer(layer, cache, spec.chain_rows(0, P, ROWS[i]), Xh[rs])
        scale = np.abs(Yo).max()
        err = np.abs(Yh[rs] - Yo).max()
        assert err <= 1e-3 * scale + 1e-4, (layer, i, P, err, scale)


def test_slice_and_head_vs_oracle(ctx):
    """Four verify layers (24..27) and the head over all 327 rows; the oracle
    chains the same layers and the head from the same layer-24 rows and
    committed KV for the shortest, middle and longest context: logits within
    max-abs 2e-2.  The same pass repeated gives the same bits (grouped
    attention with up to 9 splits and its combine, row-tiled GEMMs)."""
    e, seqs, batch = ctx["e"], ctx["seqs"], ctx["batch"]
    n_l = 4
    Y = _forward(e, batch, CFG.exit_layer, CFG.exit_layer + n_l, ctx["toks"], ctx["hL"])
    z = torch.empty((M, CFG.vocab), dtype=torch.float32, device="cuda")
    B.vs_head(e.model, M, Y.data_ptr(), z.data_ptr(), e.stream)
    for _ in range(2):
        assert torch.equal(_forward(e, batch, CFG.exit_layer, CFG.exit_layer + n_l, ctx["toks"], ctx["hL"]), Y)
    torch.cuda.synchronize()
    zg = z.cpu().numpy().astype(np.float64)
    Xh = ctx["hL"].cpu().numpy().astype(np.float64)
    dec = Decoder(CFG, G.LayerWeights(CFG))
    P = e.state()[0]
    order = np.argsort(CTX)
    pick = [int(order[0]), int(order[N // 2]), int(order[-1])]
    hs = {i: Xh[START[i]:START[i + 1]].copy() for i in pick}
    for layer in range(CFG.exit_layer, CFG.exit_layer + n_l):
        for i in pick:
            Pi = P[seqs[i]]
            cache = KVCache(CFG, Pi + ROWS[i] + 1)
            k, v = G.kv_slots(e, seqs[i], layer, np.arange(Pi))
            Kc, Vc = cache.get(0, layer)
            Kc[:, :Pi], Vc[:, :Pi] = k, v
            hs[i] = dec.layer(layer, cache, spec.chain_rows(0, Pi, ROWS[i]), hs[i])
    for i in pick:
        err = np.abs(zg[START[i]:START[i + 1]] - dec.head(hs[i])).max()
        assert err <= G.LOGIT_TOL, (i, CTX[i], err)


def test_head_and_ragged_greedy_accept(ctx):
    """Verify over all rows; head of sampled rows vs the oracle; draft tokens
    set so that request i's first i % (K_i + 1) drafts match the target's
    argmax and the next one does not: the accepted lengths, bonus tokens and
    the committed state follow the oracle's greedy rule."""
    e, seqs, batch = ctx["e"], ctx["seqs"], ctx["batch"]
    Y = _forward(e, batch, CFG.exit_layer, CFG.n_layers, ctx["toks"], ctx["hL"])
    z = torch.empty((M, CFG.vocab), dtype=torch.float32, device="cuda")
    B.vs_head(e.model, M, Y.data_ptr(), z.data_ptr(), e.stream)
    torch.cuda.synchronize()
    zg = z.cpu().numpy()
    sample = [0, 5, M // 2, M - 1]
    dec = Decoder(CFG, SynthWeights(CFG, precision="bf16", cache=True))
    zo = dec.head(Y.cpu().numpy().astype(np.float64)[sample])
    assert np.abs(zg[sample].astype(np.float64) - zo).max() <= G.LOGIT_TOL
    # the whole pass ran the row-tiled GEMM; launches of 8 rows run the
    # skinny form: the same bits row for row
    for c0 in (0, 8, (M // 2) // 8 * 8, (M - 1) // 8 * 8):
        n = min(8, M - c0)
        zc = torch.empty((n, CFG.vocab), dtype=torch.float32, device="cuda")
        B.vs_head(e.model, n, Y[c0:c0 + n].contiguous().data_ptr(), zc.data_ptr(), e.stream)
        torch.cuda.synchronize()
        assert np.array_equal(zc.cpu().numpy(), zg[c0:c0 + n]), c0
    toks = ctx["toks"].cpu().numpy().copy()
    want = []
    for i in range(N):
        r0, k = START[i], KS[i]
        a = i % (k + 1)
        for j in range(1, k + 1):
            am = int(np.argmax(zg[r0 + j - 1]))
            toks[r0 + j] = am if j <= a else (am + 1) % CFG.vocab
        want.append(spec.accept_greedy_chain(list(toks[r0:r0 + k + 1]), zg[r0:r0 + k + 1]))
    dt = G.i32(toks)
    res = torch.zeros((N, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    P0 = [e.state()[0][s] for s in seqs]
    B.vs_accept(e.model, batch, B.VS_GREEDY, 1.0, dt.data_ptr(), z.data_ptr(), None, None, res.data_ptr(), e.stream)
    B.vs_commit(e.model, e.kv, batch, res.data_ptr(), e.stream)
    torch.cuda.synchronize()
    got = G.result_rows(res, N)
    P, pending, committed = e.state()
    for i, s in enumerate(seqs):
        a, y = want[i]
        assert (got[i][0], got[i][1]) == (a, y), (i, got[i][:2], a, y)
        assert a == i % (KS[i] + 1)
        assert P[s] == P0[i] + a + 1 and pending[s] == y and committed[s] == P[s] + 1


def test_ragged_draft(ctx):
    """A greedy draft with per-request lengths K_i: every draft token is the
    argmax of the draft logits that produced it, and the first-L KV it wrote
    is bit-identical to one batched first-L pass over the same rows (self-
    speculative decoding page, §2.3: the draft's first-L KV is what the
    verify reuses).  Late draft steps carry fewer requests and one row each,
    the batched pass K_i + 1 rows: the GEMMs give a row the same bits in
    every form, and attention cuts each sequence's keys at fixed positions
    from its own KV length, in the same (grouped, GQA) kernel class."""
    e, seqs = ctx["e"], ctx["seqs"]
    toks = torch.empty(M, dtype=torch.int32, device="cuda")
    hL = torch.empty((M, CFG.d_model), dtype=torch.float32, device="cuda")
    zd = torch.empty((M, CFG.vocab), dtype=torch.float32, device="cuda")
    B.vs_draft(e.model, e.kv, seqs, KS, B.VS_GREEDY, 1.0, None, toks.data_ptr(), hL.data_ptr(), zd.data_ptr(),
               e.stream)
    torch.cuda.synchronize()
    t = toks.cpu().numpy()
    zdh = zd.cpu().numpy()
    P, pending, _ = e.state()
    for i, s in enumerate(seqs):
        r0 = START[i]
        assert t[r0] == pending[s]
        for j in range(KS[i]):
            row = zdh[r0 + j]
            if not G.near_tie(row):
                assert t[r0 + j + 1] == int(np.argmax(row)), (i, j)
    layers = [0, CFG.exit_layer - 1]
    slots = {i: np.arange(P[s], P[s] + ROWS[i]) for i, s in enumerate(seqs)}
    pick = [0, N // 2, N - 1]
    before = {(i, l): G.kv_slots(e, seqs[i], l, slots[i]) for i in pick for l in layers}
    hL_draft = hL.cpu().numpy()
    batch = B.make_batch(seqs, ROWS)
    hL_batch = _forward(e, batch, 0, CFG.exit_layer, toks, None).cpu().numpy()
    for i in pick:
        for l in layers:
            k2, v2 = G.kv_slots(e, seqs[i], l, slots[i])
            k1, v1 = before[(i, l)]
            for x1, x2 in ((k1, k2), (v1, v2)):
                assert np.array_equal(x1, x2), (i, l, np.mean(x1 == x2), np.abs(x1 - x2).max())
    assert np.array_equal(hL_draft, hL_batch), (np.mean(hL_draft == hL_batch), np.abs(hL_draft - hL_batch).max())


def _reset(e, seqs):
    """Back to the drawn contexts: the committed KV below P was never written
    by the rounds, so rewinding P and the pending token restores the start."""
    for i, s in enumerate(seqs):
        B.vs_seq_rewind(e.kv, s, CTX[i], PEND[i], e.stream)
    torch.cuda.synchronize()


def _scheduled(e, seqs, rounds):
    cfg = B.sched_cfg()
    states = (B.vs_spec_state * N)()
    for i in range(N):
        states[i] = B.vs_sched_init(cfg, int(KS[i]))
    mirror = [spec.SchedState(int(KS[i])) for i in range(N)]
    toks = torch.zeros(N * (B.VS_MAX_K + 1), dtype=torch.int32, device="cuda")
    res = torch.zeros((N, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    out = [[int(PEND[i])] for i in range(N)]
    ks, accs = [], []
    for r in range(rounds):
        k_round = [states[i].k for i in range(N)]
        got, conf = B.vs_step_sched(e.model, e.kv, seqs, cfg, states, toks.data_ptr(), res.data_ptr(), e.stream)
        t = toks.cpu().numpy()
        P, pending, committed = e.state()
        r0 = 0
        for i, s in enumerate(seqs):
            a, y = got[i][0], got[i][1]
            out[i] += [int(x) for x in t[r0 + 1:r0 + a + 1]] + [y]
            r0 += k_round[i] + 1
            assert P[s] == CTX[i] + len(out[i]) - 1 and pending[s] == y and committed[s] == P[s] + 1
            nk, _ = spec.schedule_update(mirror[i], a, conf[i][0], conf[i][1])
            assert states[i].k == nk and states[i].ema == mirror[i].ema, (r, i)
        ks.append(k_round)
        accs.append([got[i][0] for i in range(N)])
    return out, ks, accs


def _greedy_ar(e, seqs, n_new):
    """Plain greedy AR of every request: the pending tokens through all layers
    as one batch of single rows per step.  Returns tokens and logits rows."""
    batch = B.make_batch(seqs, [1] * N)
    z = torch.empty((N, CFG.vocab), dtype=torch.float32, device="cuda")
    res = torch.zeros((N, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    out = [[int(PEND[i])] for i in range(N)]
    zs = [[] for _ in range(N)]
    for step in range(n_new):
        pend = G.i32([e.state()[1][s] for s in seqs])
        B.vs_verify(e.model, e.kv, batch, 0, pend.data_ptr(), None, z.data_ptr(), e.stream)
        B.vs_accept(e.model, batch, B.VS_GREEDY, 1.0, pend.data_ptr(), z.data_ptr(), None, None, res.data_ptr(),
                    e.stream)
        B.vs_commit(e.model, e.kv, batch, res.data_ptr(), e.stream)
        zh = z.cpu().numpy()
        for i, (a, y, _, _) in enumerate(G.result_rows(res, N)):
            out[i].append(y)
            zs[i].append(zh[i])
    return out, zs


def _compare_with_ar(e, seqs, out, head_scale=1.0):
    n_new = max(len(o) for o in out) - 1
    _reset(e, seqs)
    ar, zs = _greedy_ar(e, seqs, n_new)
    for i in range(N):
        tie = next((j for j in range(len(out[i]) - 1) if G.near_tie(zs[i][j], head_scale)), len(out[i]) - 1)
        assert out[i][:tie + 1] == ar[i][:tie + 1], (i, tie, out[i], ar[i])


def test_scheduled_rounds_equal_ar(ctx):
    """Three scheduled rounds of the 32 requests from their drawn K_r.  On
    this random-weight model the target's distributions are nearly flat and
    drafts are rejected, so k drops to 2 after the first round; the committed
    tokens equal greedy AR from the same contexts."""
    e, seqs = ctx["e"], ctx["seqs"]
    _reset(e, seqs)
    out, ks, accs = _scheduled(e, seqs, ROUNDS)
    assert ks[0] == [int(k) for k in KS]
    _compare_with_ar(e, seqs, out)


def test_scheduled_rounds_calibrated(ctx):
    """The calibrated model: W_o and W_down of the verify layers zeroed (the
    target equals the draft, every draft is accepted) and the LM head scaled
    by 4 (confident distributions): k climbs to the top of its range, and the
    committed tokens still equal greedy AR of the same model.  The last test
    of the module: it changes the weights."""
    import synth
    from synth import gpu_weights
    e, seqs = ctx["e"], ctx["seqs"]
    for l in range(CFG.exit_layer, CFG.n_layers):
        for t in (synth.T_WO, synth.T_W_DOWN):
            e.set_tensor(t, l, gpu_weights.device_bits(CFG, t, l, e.device, e.stream, eps=0.0))
    e.set_tensor(synth.T_HEAD, 0, gpu_weights.device_bits(CFG, synth.T_HEAD, 0, e.device, e.stream, head_scale=4.0))
    torch.cuda.synchronize()
    _reset(e, seqs)
    out, ks, accs = _scheduled(e, seqs, ROUNDS)
    for r in range(ROUNDS):
        assert accs[r] == ks[r], (r, accs[r], ks[r])  # target == draft: everything accepted
    assert max(ks[-1]) == B.VS_MAX_K and np.mean(ks[-1]) > np.mean(ks[0]), (ks[0], ks[-1])
    _compare_with_ar(e, seqs, out, head_scale=4.0)

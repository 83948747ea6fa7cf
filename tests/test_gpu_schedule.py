"""Draft-length policies over several rounds, through the C ABI, on the tiny
decoder.

The confidence schedule ("DSpark" page, §2.2-§2.3) over a ragged batch, with
W_o and W_down of the verify layers scaled by 0.5 (a synthetic model whose
drafts are sometimes accepted) and the LM head scaled by 16 (sharper output
distributions, the same argmax everywhere, so that the confidence, and with
it k, moves over its range).  Per round and request:
* the library's next k and acceptance average equal the oracle schedule fed
  the library's own (a, confidence), bit for bit;
* the confidences agree with the oracle's scheduled run while the two runs
  are in step;
* the committed tokens equal the oracle's greedy tokens (the method is
  lossless whatever k is) up to the first near-tie, and the k sequence equals
  the oracle's until a decision lands within reach of rounding.

The windowed dynamic k with its context-cost cut-off (self-speculative
decoding page, §3.2 and §5.3) over one request: the library's controller
against the oracle's on the GPU's accepted counts, and the tokens against the
oracle's greedy tokens, including the plain decoding steps it switches to."""
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
EPS = 0.5
HEAD = 16.0
N_REQ, ROUNDS, K0 = 4, 10, 4
CONF_TOL = 5e-2   # probabilities from logits that agree within HEAD x 2e-2
K_BAND = 0.15     # a schedule value this close to an integer may round either way


@pytest.fixture(scope="module")
def eng():
    return G.engine(CFG, eps=EPS, head_scale=HEAD, force_host=True, max_rows=80, max_seqs=8, max_ctx=512)


def test_scheduled_rounds(eng):
    e = eng
    prompts = [G.prompt(CFG, 40 + 8 * i, req=20 + i) for i in range(N_REQ)]
    seqs = []
    for p in prompts:
        s = e.open(480)
        t = G.i32(p)
        B.vs_prefill(e.model, e.kv, s, t.data_ptr(), len(p), B.VS_GREEDY, 1.0, None, None, e.stream)
        seqs.append(s)
    torch.cuda.synchronize()
    cfg = B.sched_cfg()
    states = (B.vs_spec_state * N_REQ)()
    for i in range(N_REQ):
        states[i] = B.vs_sched_init(cfg, K0)
    mirror = [spec.SchedState(K0) for _ in range(N_REQ)]
    toks = torch.zeros(N_REQ * (B.VS_MAX_K + 1), dtype=torch.int32, device="cuda")
    res = torch.zeros((N_REQ, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    out = [[e.state()[1][s]] for s in seqs]
    ks = [[] for _ in range(N_REQ)]
    a_gpu = [[] for _ in range(N_REQ)]
    confs = [[] for _ in range(N_REQ)]
    for r in range(ROUNDS):
        k_round = [states[i].k for i in range(N_REQ)]
        P0 = [e.state()[0][s] for s in seqs]
        got, conf = B.vs_step_sched(e.model, e.kv, seqs, cfg, states, toks.data_ptr(), res.data_ptr(), e.stream)
        t = toks.cpu().numpy()
        P, pending, committed = e.state()
        r0 = 0
        for i, s in enumerate(seqs):
            k = k_round[i]
            a, y = got[i][0], got[i][1]
            assert 0 <= a <= k
            out[i] += [int(x) for x in t[r0 + 1:r0 + a + 1]] + [y]
            r0 += k + 1
            assert P[s] == P0[i] + a + 1 and pending[s] == y and committed[s] == P[s] + 1
            # the library's schedule is the oracle's schedule on the same inputs
            nk, _ = spec.schedule_update(mirror[i], a, conf[i][0], conf[i][1])
            assert states[i].k == nk and states[i].ema == mirror[i].ema, (r, i)
            assert states[i].rounds == r + 1 and states[i].last_a == a
            ks[i].append(k)
            a_gpu[i].append(a)
            confs[i].append(conf[i])
    # the oracle's own scheduled run of each request
    dec = G.oracle_decoder(CFG, eps=EPS, head_scale=HEAD)
    varied = False
    compared = 0
    for i in range(N_REQ):
        n_new = len(out[i])
        cache = KVCache(CFG, 512)
        ref, ref_ks, ref_conf, _ = spec.generate_scheduled(dec, cache, i, prompts[i], n_new, K0)
        varied |= len(set(ks[i])) > 2
        # tokens: equal up to the oracle's first near-tie (checked on the oracle's AR logits)
        cache2 = KVCache(CFG, 512)
        st, z0 = spec.prefill(dec, cache2, 0, prompts[i])
        zs = [z0]
        while len(zs) < n_new:
            zs.append(spec.ar_step(dec, cache2, st)[1])
        tie = next((j for j in range(n_new) if G.near_tie(zs[j], HEAD)), n_new)
        assert out[i][:tie] == ref[:tie], (i, tie)
        # k sequences: equal while the runs are in step (same accepted counts,
        # no target near-tie among the tokens so far) and no decision is marginal
        done = 0
        for r in range(min(len(ks[i]), len(ref_ks))):
            assert ks[i][r] == ref_ks[r], (i, r, ks[i], ref_ks)
            compared += 1
            t1, g, C, a_ref = ref_conf[r]
            if a_gpu[i][r] != a_ref:
                break  # a draft-side near-tie: the committed tokens still agree
            done += a_ref + 1
            if done >= tie:
                break
            assert abs(confs[i][r][0] - t1) <= CONF_TOL and abs(confs[i][r][1] - g) <= CONF_TOL, (i, r)
            x = spec.next_k_real(C)
            if a_ref != 0 and 2 < x < 16 and abs(x - round(x)) < K_BAND:
                break
    assert varied, f"k took fewer than three values in every request: {ks}"
    print(f"k decisions compared with the oracle's own run: {compared} of {N_REQ * ROUNDS}; k: {ks}")
    assert compared >= 2 * N_REQ
    for s in seqs:
        B.vs_seq_close(e.kv, s)


@pytest.mark.parametrize("eps", [0.0, None])
def test_dynamic_k_rounds(eps):
    """Twelve rounds of one request with the windowed dynamic k and the
    context-cost cut-off at c = L/N = 0.5 (the draft's share of the layers):
    each next k equals the oracle controller fed the GPU's accepted counts; a
    round with k = 0 is a plain decoding step.  With every draft accepted
    (eps = 0) k climbs to 8; on the random model (drafts rejected) drafting
    switches off.  The tokens equal the oracle's greedy tokens throughout."""
    e = G.engine(CFG, eps=eps, force_host=True, max_rows=64, max_seqs=2, max_ctx=512)
    p = G.prompt(CFG, 48, req=30)
    seq = e.open(480)
    t = G.i32(p)
    B.vs_prefill(e.model, e.kv, seq, t.data_ptr(), len(p), B.VS_GREEDY, 1.0, None, None, e.stream)
    torch.cuda.synchronize()
    c_draft = CFG.exit_layer / CFG.n_layers
    cfg = B.dynk_cfg()
    lib = B.vs_dynk_init(cfg, 4)
    ora = spec.DynKState(4)
    toks = torch.zeros(B.VS_MAX_K + 1, dtype=torch.int32, device="cuda")
    res = torch.zeros((1, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    z = torch.empty((1, CFG.vocab), dtype=torch.float32, device="cuda")
    batch1 = B.make_batch([seq], [1])
    pend_ptr = B.vs_kv_state(e.kv)[1] + 4 * seq
    out = [e.state()[1][seq]]
    k_next, ks = 4, []
    for r in range(12):
        ks.append(k_next)
        if k_next > 0:
            B.vs_step(e.model, e.kv, [seq], [k_next], B.VS_GREEDY, 1.0, None, toks.data_ptr(), res.data_ptr(),
                      e.stream)
            a, y, _, _ = G.result_rows(res, 1)[0]
            out += [int(x) for x in toks[1:a + 1].cpu().tolist()] + [y]
            k_used = k_next
        else:
            B.vs_verify(e.model, e.kv, batch1, 0, pend_ptr, None, z.data_ptr(), e.stream)
            B.vs_accept(e.model, batch1, B.VS_GREEDY, 1.0, pend_ptr, z.data_ptr(), None, None, res.data_ptr(),
                        e.stream)
            B.vs_commit(e.model, e.kv, batch1, res.data_ptr(), e.stream)
            a, y, _, _ = G.result_rows(res, 1)[0]
            out.append(y)
            k_used = 0
        P, pending, committed = e.state()
        assert P[seq] == len(p) + len(out) - 1 and pending[seq] == y and committed[seq] == P[seq] + 1
        k_next = B.vs_dynk_update(cfg, lib, a, k_used, c_draft)
        assert k_next == spec.dynk_update(ora, a, k_used, c_draft) and lib.k == ora.k and lib.alpha == ora.alpha
    if eps == 0.0:
        assert max(ks) == 8 and ks[:5] == [4, 5, 6, 7, 8], ks
    else:
        assert 0 in ks, ks
    dec = G.oracle_decoder(CFG, eps=eps)
    cache = KVCache(CFG, 512)
    st, z0 = spec.prefill(dec, cache, 0, p)
    ref, zs = [st.pending], [z0]
    while len(ref) < len(out):
        y, zz = spec.ar_step(dec, cache, st)
        ref.append(y)
        zs.append(zz)
    tie = next((j for j in range(len(out)) if G.near_tie(zs[j])), len(out))
    assert out[:tie + 1] == ref[:tie + 1], (tie, out, ref)
    B.vs_seq_close(e.kv, seq)

"""GPU tree drafting on the tiny decoder against the oracle: the tree the
GPU builds equals the oracle's level-synchronous selection on the GPU's own
level logits (integers bit-exact, near-ties at the kept cutoff excepted);
the level logits and the final rows' layer-L inputs match the oracle's
float64 decoder; a whole tree round (draft, verify, accept, commit) keeps
the oracle's greedy walk and the state invariant."""
import numpy as np
import pytest
import torch

from oracle import spec, tree
from oracle.decoder import KVCache
from synth.workloads import TINY
from tests import gpu_common as G
from tests.tree_replay import replay
from verification_verify_step_amd import binding as B

pytestmark = pytest.mark.gpu

CFG = TINY
TOPK, DEPTH, KEEP, T = 5, 4, 63, 1.0
R = 1 + KEEP


@pytest.fixture(scope="module")
def eng():
    return G.engine(CFG, force_host=True, max_rows=64, max_seqs=8, max_ctx=512)


@pytest.fixture(scope="module")
def dec():
    return G.oracle_decoder(CFG)


def draft_tree(e, seq, cfg=CFG):
    out = {
        "tok": torch.empty(R, dtype=torch.int32, device="cuda"),
        "depth": torch.empty(R, dtype=torch.int32, device="cuda"),
        "mask": torch.empty(R, dtype=torch.int64, device="cuda"),
        "parent": torch.empty(R, dtype=torch.int32, device="cuda"),
        "hL": torch.empty((R, cfg.d_model), dtype=torch.float32, device="cuda"),
        "lz": torch.empty((DEPTH, R, cfg.vocab), dtype=torch.float32, device="cuda"),
    }
    B.vs_draft_tree(e.model, e.kv, seq, TOPK, DEPTH, KEEP, T, out["tok"].data_ptr(), out["depth"].data_ptr(),
                    out["mask"].data_ptr(), out["parent"].data_ptr(), out["hL"].data_ptr(), out["lz"].data_ptr(),
                    e.stream)
    torch.cuda.synchronize()
    return out


def check_layout(out, nodes, order):
    assert out["tok"].cpu().tolist() == [nodes[n].token for n in order]
    assert out["depth"].cpu().tolist() == [nodes[n].depth for n in order]
    masks = np.array(tree.masks_of_rows(nodes, order), dtype=np.uint64)
    assert np.array_equal(out["mask"].cpu().numpy().view(np.uint64), masks)
    assert out["parent"].cpu().tolist() == tree.parents_of_rows(nodes, order)


def _prefill(e, p):
    seq = e.open(480)
    B.vs_prefill(e.model, e.kv, seq, G.i32(p).data_ptr(), len(p), B.VS_GREEDY, 1.0, None, None, e.stream)
    torch.cuda.synchronize()
    return seq


@pytest.mark.parametrize("req", [6, 9])
def test_tree_selection_equals_oracle(eng, req):
    seq = _prefill(eng, G.prompt(CFG, 48, req=req))
    out = draft_tree(eng, seq)
    root = eng.state()[1][seq]
    nodes, order, _, near = replay(out["lz"].cpu().numpy(), root, T, TOPK, DEPTH, KEEP)
    B.vs_seq_close(eng.kv, seq)
    if near:
        pytest.skip("near-tie at the kept cutoff")
    check_layout(out, nodes, order)


def test_tree_level_logits_and_hidden_match_oracle(eng, dec):
    p = G.prompt(CFG, 48, req=6)
    seq = _prefill(eng, p)
    out = draft_tree(eng, seq)
    cache = KVCache(CFG, 512)
    st, _ = spec.prefill(dec, cache, 0, p)
    assert st.pending == eng.state()[1][seq]
    lz = out["lz"].cpu().numpy().astype(np.float64)
    nodes, order, layouts, _ = replay(lz, st.pending, T, TOPK, DEPTH, KEEP)
    L = CFG.exit_layer
    for d, lay in enumerate(layouts):  # level passes: the root and the kept nodes of that level
        rows = tree.tree_rows(nodes, lay, 0, st.P)
        h = dec.forward_layers(cache, rows, dec.embed([nodes[n].token for n in lay]), 0, L)
        zo = dec.head(h)
        assert np.abs(lz[d][:len(lay)] - zo).max() <= G.LOGIT_TOL, (d, np.abs(lz[d][:len(lay)] - zo).max())
    rows = tree.tree_rows(nodes, order, 0, st.P)
    toks = out["tok"].cpu().tolist()
    hLo = dec.forward_layers(cache, rows, dec.embed(toks), 0, L)
    hg = out["hL"].cpu().numpy().astype(np.float64)
    assert np.abs(hg - hLo).max() <= 1e-3 * np.abs(hLo).max() + 1e-4
    B.vs_seq_close(eng.kv, seq)


def test_tree_round(eng, dec):
    """draft_tree -> verify(L) -> greedy walk -> compaction, twice."""
    p = G.prompt(CFG, 48, req=11)
    seq = _prefill(eng, p)
    for _ in range(2):
        P0 = eng.state()[0][seq]
        out = draft_tree(eng, seq)
        batch = B.make_batch([seq], [R], out["depth"].data_ptr(), out["mask"].data_ptr())
        z = torch.empty((R, CFG.vocab), dtype=torch.float32, device="cuda")
        B.vs_verify(eng.model, eng.kv, batch, CFG.exit_layer, out["tok"].data_ptr(), out["hL"].data_ptr(),
                    z.data_ptr(), eng.stream)
        res = torch.zeros((8, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
        B.vs_accept(eng.model, batch, B.VS_GREEDY, 1.0, out["tok"].data_ptr(), z.data_ptr(), None, None,
                    res.data_ptr(), eng.stream)
        B.vs_commit(eng.model, eng.kv, batch, res.data_ptr(), eng.stream)
        torch.cuda.synchronize()
        a, y, _, path = G.result_rows(res, 1)[0]
        toks = out["tok"].cpu().tolist()
        oa, opath, oy = tree.accept_greedy_tree(toks, out["parent"].cpu().tolist(), z.cpu().numpy())
        assert (a, path, y) == (oa, opath, oy)
        P, pending, committed = eng.state()
        assert P[seq] == P0 + a + 1 and pending[seq] == y and committed[seq] == P[seq] + 1
    B.vs_seq_close(eng.kv, seq)


def test_tree_draft_rejects_bad_arguments(eng):
    seq = _prefill(eng, G.prompt(CFG, 16, req=3))
    out = {k: torch.empty(128, dtype=torch.int64, device="cuda") for k in ("a", "b", "c", "d")}
    hL = torch.empty((64, CFG.d_model), dtype=torch.float32, device="cuda")
    for topk, depth, keep in [(0, 4, 63), (9, 4, 63), (5, 0, 63), (5, 9, 63), (5, 4, 64), (8, 8, 63)]:
        with pytest.raises(B.VsError):
            B.vs_draft_tree(eng.model, eng.kv, seq, topk, depth, keep, 1.0, out["a"].data_ptr(), out["b"].data_ptr(),
                            out["c"].data_ptr(), out["d"].data_ptr(), hL.data_ptr(), None, eng.stream)
    B.vs_seq_close(eng.kv, seq)

"""GPU parity for tree verification at the 7B shape with a 4096-token
context: a top-5, depth-4 draft tree pruned to 63 nodes (64 verify rows with
ancestor masks and positions P + depth).  The tree the GPU drafts equals the
oracle's selection on the GPU's own level logits; verify layers over all 64
rows match the float64 oracle given the GPU's layer input and committed KV;
head logits of sampled rows match; the greedy walk on the GPU's logits and
the compaction commit equal the oracle's."""
import numpy as np
import pytest
import torch

from oracle import tree
from oracle.decoder import Decoder, KVCache, Row
from synth.model_weights import SynthWeights
from synth.workloads import LLAMA7B
from tests import gpu_common as G
from tests.test_gpu_tree import DEPTH, KEEP, R, T, TOPK, check_layout, draft_tree
from tests.tree_replay import replay
from verification_verify_step_amd import binding as B

pytestmark = pytest.mark.gpu

CFG = LLAMA7B
P0 = 4096


@pytest.fixture(scope="module")
def ctx():
    e = G.engine(CFG, max_rows=64, max_seqs=2, max_ctx=P0 + 160)
    seq = e.open(P0 + 150)
    B.vs_prefill(e.model, e.kv, seq, G.i32(G.prompt(CFG, P0, req=3)).data_ptr(), P0, B.VS_GREEDY, 1.0, None, None,
                 e.stream)
    torch.cuda.synchronize()
    out = draft_tree(e, seq, CFG)
    batch = B.make_batch([seq], [R], out["depth"].data_ptr(), out["mask"].data_ptr())
    yield {"e": e, "seq": seq, "out": out, "batch": batch}
    B.vs_seq_close(e.kv, seq)


def _rows(out, P):
    depth = out["depth"].cpu().tolist()
    mask = out["mask"].cpu().numpy().view(np.uint64)
    rows = []
    for r in range(R):
        vis = [P + j for j in range(R) if (int(mask[r]) >> j) & 1]
        rows.append(Row(0, P + depth[r], P + r, np.concatenate([np.arange(P), np.array(vis)])))
    return rows


def _forward(e, batch, start, end, toks, hin):
    y = torch.empty((R, CFG.d_model), dtype=torch.float32, device="cuda")
    B.vs_forward_layers(e.model, e.kv, batch, start, end, toks.data_ptr(), hin.data_ptr(), y.data_ptr(), e.stream)
    return y


def test_tree_selection_equals_oracle(ctx):
    e, out = ctx["e"], ctx["out"]
    root = e.state()[1][ctx["seq"]]
    nodes, order, _, near = replay(out["lz"].cpu().numpy(), root, T, TOPK, DEPTH, KEEP)
    if near:
        pytest.skip("near-tie at the kept cutoff")
    check_layout(out, nodes, order)


@pytest.mark.parametrize("layer", [12, 22])
def test_verify_layer_parity_64_tree_rows(ctx, layer):
    e, seq, out, batch = ctx["e"], ctx["seq"], ctx["out"], ctx["batch"]
    P = e.state()[0][seq]
    X = out["hL"] if layer == CFG.exit_layer else _forward(e, batch, CFG.exit_layer, layer, out["tok"], out["hL"])
    Y = _forward(e, batch, layer, layer + 1, out["tok"], X)
    torch.cuda.synchronize()
    dec = Decoder(CFG, SynthWeights(CFG, precision="bf16", cache=True))
    cache = KVCache(CFG, P + R + 1)
    k, v = G.kv_slots(e, seq, layer, np.arange(P))
    Kc, Vc = cache.get(0, layer)
    Kc[:, :P], Vc[:, :P] = k, v
    Yo = dec.layer(layer, cache, _rows(out, P), X.cpu().numpy().astype(np.float64))
    Yg = Y.cpu().numpy().astype(np.float64)
    scale = np.abs(Yo).max()
    assert np.abs(Yg - Yo).max() <= 1e-3 * scale + 1e-4, (layer, np.abs(Yg - Yo).max(), scale)


def test_head_walk_and_compaction(ctx):
    e, seq, out, batch = ctx["e"], ctx["seq"], ctx["out"], ctx["batch"]
    P0_ = e.state()[0][seq]
    z = torch.empty((R, CFG.vocab), dtype=torch.float32, device="cuda")
    B.vs_verify(e.model, e.kv, batch, CFG.exit_layer, out["tok"].data_ptr(), out["hL"].data_ptr(), z.data_ptr(),
                e.stream)
    Y = _forward(e, batch, CFG.exit_layer, CFG.n_layers, out["tok"], out["hL"])
    torch.cuda.synchronize()
    sample = [0, 1, 6, 31, 63]
    dec = Decoder(CFG, SynthWeights(CFG, precision="bf16", cache=True))
    zo = dec.head(Y.cpu().numpy().astype(np.float64)[sample])
    zg = z.cpu().numpy().astype(np.float64)
    assert np.abs(zg[sample] - zo).max() <= G.LOGIT_TOL, np.abs(zg[sample] - zo).max()
    res = torch.zeros((2, B.VS_RESULT_INTS), dtype=torch.int32, device="cuda")
    B.vs_accept(e.model, batch, B.VS_GREEDY, 1.0, out["tok"].data_ptr(), z.data_ptr(), None, None, res.data_ptr(),
                e.stream)
    a, y, _, path = G.result_rows(res, 1)[0]
    toks = out["tok"].cpu().tolist()
    parents = out["parent"].cpu().tolist()
    oa, opath, oy = tree.accept_greedy_tree(toks, parents, z.cpu().numpy())
    assert (a, path, y) == (oa, opath, oy)
    # compaction of a forced depth-3 path: every layer's KV of the path rows moves to P+1..P+3
    leaf = max(r for r in range(R) if out["depth"][r].item() == 3)
    forced = [leaf]
    while parents[forced[-1]] > 0:
        forced.append(parents[forced[-1]])
    forced = forced[::-1]
    layers = [0, CFG.exit_layer - 1, CFG.exit_layer, CFG.n_layers - 1]
    before = [G.kv_slots(e, seq, l, [P0_ + r for r in forced]) for l in layers]
    r = torch.zeros((2, B.VS_RESULT_INTS), dtype=torch.int32)
    r[0, 0], r[0, 1], r[0, 3] = len(forced), 11, len(forced)
    r[0, 4:4 + len(forced)] = torch.tensor(forced)
    B.vs_commit(e.model, e.kv, batch, r.cuda().data_ptr(), e.stream)
    torch.cuda.synchronize()
    for l, (k1, v1) in zip(layers, before):
        k2, v2 = G.kv_slots(e, seq, l, [P0_ + 1 + i for i in range(len(forced))])
        assert np.array_equal(k2, k1) and np.array_equal(v2, v1)
    P, pending, committed = e.state()
    assert P[seq] == P0_ + len(forced) + 1 and pending[seq] == 11 and committed[seq] == P[seq] + 1

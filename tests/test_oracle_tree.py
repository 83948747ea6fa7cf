"""Pins of the oracle's tree draft / tree verify / tree walk ("FlashSpec"
page, lnrk.cn/news/47842, §2.2, §3.2, §5.2): level-synchronous selection equals
brute-force enumeration of the whole top-5 depth-4 tree; a node's logits equal
a chain verify of its root path; the greedy walk equals the longest accepted
root-to-leaf path found by brute force; masked (padding) slots never leak."""

import numpy as np

import synth
from oracle import spec, tree
from oracle.decoder import Decoder, KVCache, Row
from synth.model_weights import SynthWeights
from synth.workloads import TINY


def _hash_q(path, V=8):
    """A fixed pseudo-random distribution for each root path (stand-in model)."""
    key = 1469598103934665603
    for t in path:
        key = (key * 1099511628211 + t + 1) & ((1 << 64) - 1)
    u = synth.uniforms(key, 0, V)
    w = np.exp(3.0 * u)
    return w / w.sum()


def _path(nodes, i):
    out = []
    while i >= 0:
        out.append(nodes[i].token)
        i = nodes[i].parent
    return out[::-1]


def test_level_synchronous_equals_brute_force():
    for root in range(6):
        def expand(frontier, nodes):
            return [_hash_q(_path(nodes, i)) for i in frontier]
        nodes, order = tree.build_tree(expand, root, topk=5, depth=4, keep=63)
        got = sorted(tuple(_path(nodes, i)) for i in order[1:])
        # brute force: every node of the full tree with its score
        full = []

        def rec(path, score, depth):
            if depth == 4:
                return
            for r, (tok, p) in enumerate(tree.top_children(_hash_q(path), 5)):
                full.append((score * p, depth + 1, tuple(path + [tok])))
                rec(path + [tok], score * p, depth + 1)
        rec([root], 1.0, 0)
        assert len(full) == 5 + 25 + 125 + 625
        full.sort(key=lambda x: (-x[0], x[1]))
        want = sorted(x[2] for x in full[:63])
        assert got == want
        # ancestor-closed, at most 4 levels, 64 rows, level order
        paths = set(got)
        for p in got:
            assert len(p) <= 5 and (len(p) == 2 or p[:-1] in paths)
        depths = [nodes[i].depth for i in order]
        assert len(order) == 64 and depths == sorted(depths)


def _tiny(eps=0.3):
    from tests.test_oracle_spec import UpperScaled
    return Decoder(TINY, UpperScaled(SynthWeights(TINY, "bf16"), TINY.exit_layer, eps))


def test_tree_logits_equal_chain_of_root_path():
    dec = _tiny()
    prompt = synth.tokens(synth.SEED_PROMPTS, synth.stream_prompt(1), TINY.vocab, 40)
    cache = KVCache(TINY, 256)
    st, _ = spec.prefill(dec, cache, 0, prompt)
    nodes, order, toks, hL = tree.draft_tree(dec, cache, st)
    rows = tree.tree_rows(nodes, order, 0, st.P)
    z = spec.verify_rows(dec, cache, rows, hL, TINY.exit_layer)
    parents = tree.parents_of_rows(nodes, order)
    for r in (0, 1, 7, 20, 63):
        path_rows = []
        x = r
        while x >= 0:
            path_rows.append(x)
            x = parents[x]
        path_rows = path_rows[::-1]
        c2 = KVCache(TINY, 256)
        spec.prefill(dec, c2, 0, prompt)
        ptoks = [toks[x] for x in path_rows]
        crow = spec.chain_rows(0, st.P, len(ptoks))
        zc = spec.verify_rows(dec, c2, crow, ptoks, 0)
        np.testing.assert_allclose(z[r], zc[-1], rtol=1e-9, atol=1e-9)


def test_masks_and_positions():
    dec = _tiny()
    cache = KVCache(TINY, 256)
    st, _ = spec.prefill(dec, cache, 0, synth.tokens(synth.SEED_PROMPTS, synth.stream_prompt(2), TINY.vocab, 16))
    nodes, order, toks, _ = tree.draft_tree(dec, cache, st)
    masks = tree.masks_of_rows(nodes, order)
    parents = tree.parents_of_rows(nodes, order)
    rows = tree.tree_rows(nodes, order, 0, st.P)
    for r in range(64):
        # own bit set, parent's mask contained in this row's, position = parent's + 1
        assert masks[r] >> r & 1
        if r:
            assert masks[parents[r]] & masks[r] == masks[parents[r]]
            assert rows[r].pos == rows[parents[r]].pos + 1
            assert parents[r] < r
        assert rows[r].pos == st.P + nodes[order[r]].depth
    # a chain-shaped tree gives the causal chain masks
    assert [(1 << (i + 1)) - 1 for i in range(5)] == [sum(1 << j for j in range(i + 1)) for i in range(5)]


def test_greedy_walk_equals_longest_path_brute_force():
    rng = np.random.default_rng(9)
    for _ in range(300):
        n = 12
        parents = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        toks = [0] + [int(rng.integers(0, 4)) for _ in range(1, n)]
        # siblings carry distinct tokens, as top-k children do
        seen = set()
        for i in range(1, n):
            while (parents[i], toks[i]) in seen:
                toks[i] = (toks[i] + 1) % 7
            seen.add((parents[i], toks[i]))
        logits = rng.standard_normal((n, 7))
        a, path, y = tree.accept_greedy_tree(toks, parents, logits)
        best = 0
        for leaf in range(n):
            chain = []
            x = leaf
            while x > 0:
                chain.append(x)
                x = parents[x]
            chain = chain[::-1]
            ok = 0
            prev = 0
            for c in chain:
                if toks[c] != int(np.argmax(logits[prev])):
                    break
                ok += 1
                prev = c
            best = max(best, ok)
        assert a == best
        last = path[-1] if path else 0
        assert y == int(np.argmax(logits[last]))


def test_tree_commit_equals_chain_of_accepted_path():
    dec = _tiny(eps=0.0)  # target == draft: the walk accepts a full path
    prompt = synth.tokens(synth.SEED_PROMPTS, synth.stream_prompt(4), TINY.vocab, 24)
    cache = KVCache(TINY, 256)
    st, _ = spec.prefill(dec, cache, 0, prompt)
    P0 = st.P
    nodes, order, toks, hL = tree.draft_tree(dec, cache, st)
    rows = tree.tree_rows(nodes, order, 0, st.P)
    z = spec.verify_rows(dec, cache, rows, hL, TINY.exit_layer)
    a, path, y = tree.accept_greedy_tree(toks, tree.parents_of_rows(nodes, order), z)
    # target == draft: the walk follows the top-1 children as deep as the kept tree goes
    assert a >= 2 and all(nodes[order[r]].rank == 0 for r in path)
    top1_depth = max(nodes[n].depth for n in order if all(nodes[m].rank == 0 for m in tree.ancestors_or_self(nodes, n)[:-1]))
    assert a == top1_depth
    tree.commit_tree(cache, st, toks, path, y)
    c2 = KVCache(TINY, 256)
    spec.prefill(dec, c2, 0, prompt)
    ptoks = [toks[0]] + [toks[r] for r in path]
    spec.verify_rows(dec, c2, spec.chain_rows(0, P0, len(ptoks)), ptoks, 0)
    for l in range(TINY.n_layers):
        np.testing.assert_allclose(cache.get(0, l)[0][:, :P0 + a + 1], c2.get(0, l)[0][:, :P0 + a + 1], atol=1e-9)
        np.testing.assert_allclose(cache.get(0, l)[1][:, :P0 + a + 1], c2.get(0, l)[1][:, :P0 + a + 1], atol=1e-9)


def test_masked_slots_never_leak():
    """Garbage (NaN) in slots a row does not see leaves its output finite."""
    dec = _tiny()
    cache = KVCache(TINY, 64)
    rows = [Row(0, i, i, np.arange(i + 1)) for i in range(8)]
    h = dec.forward_layers(cache, rows, dec.embed(list(range(8))), 0, TINY.n_layers)
    assert np.isfinite(h).all()
    # slots 8.. are NaN-initialised and invisible; a row that saw one would be NaN
    bad = [Row(0, 8, 8, np.arange(10))]
    hb = dec.forward_layers(cache, bad, dec.embed([3]), 0, 1)
    assert np.isnan(hb).all()

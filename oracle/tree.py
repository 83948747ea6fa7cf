"""Tree drafting, tree verification and the greedy tree walk (oracle).

TEST INFRASTRUCTURE: see ``oracle/__init__.py``.

From the "FlashSpec" page (lnrk.cn/news/47842): the candidates form a tree
that is verified in one forward pass, laid out in level order with a mask that
tells each node which earlier nodes are its ancestors (§2.2); a node's
position id is its parent's plus one (§3.2); padding must never be visible
(§5.2); the result is the longest acceptable root-to-leaf path (§1.2, §4.1).

Readings where the page is silent or garbled (listed in the design doc):
* Shape: top-k children per node (k=5) to depth 4, and the kept set is the
  global top-63 non-root nodes by path score (product of the draft
  probabilities along the path), ties by (depth, discovery order).  Built
  level by level, expanding at depth d only nodes in the current top-63 of all
  nodes found so far; this equals the global selection because a child never
  scores above its parent.
* Layout: row 0 is the root (the pending token); rows 1..63 in level order
  (depth, then parent's row, then child rank).  Position = P + depth,
  KV slot = P + row.
* Level passes write their first-L KV at scratch slots P + 64 + forward index;
  a final first-L pass over the 64 kept rows writes slots P + row and gives
  verify its inputs.
* Greedy acceptance walks from the root to the child whose token equals the
  target argmax at the current node; siblings are distinct ids, so the path
  is unique.  Commit copies the accepted nodes' KV (all layers) to slots
  P+1..P+a.
"""
from dataclasses import dataclass

import numpy as np

from .decoder import Row
from .spec import argmax, probs

SCRATCH = 64  # level-pass scratch slots start at P + 64


@dataclass
class Node:
    token: int
    parent: int  # node index, -1 for the root
    depth: int
    score: float
    rank: int  # child rank under its parent (0 = most probable)
    disc: int  # discovery order


def top_children(q, topk):
    """The topk ids of q by probability, ties to the lower id."""
    order = np.lexsort((np.arange(len(q)), -np.asarray(q)))
    return [(int(i), float(q[i])) for i in order[:topk]]


def _top_keep(nodes, keep):
    cand = [i for i in range(1, len(nodes))]
    cand.sort(key=lambda i: (-nodes[i].score, nodes[i].depth, nodes[i].disc))
    return set(cand[:keep])


def build_tree(expand, root_token, topk=5, depth=4, keep=63):
    """Level-synchronous construction of the kept tree.

    expand(list of node indices, nodes) -> list of q rows, one per node.
    Returns (nodes, order) where order lists node indices in level order,
    root first.
    """
    nodes = [Node(int(root_token), -1, 0, 1.0, 0, 0)]

    def add_children(i, q):
        for r, (tok, p) in enumerate(top_children(q, topk)):
            nodes.append(Node(tok, i, nodes[i].depth + 1, nodes[i].score * p, r, len(nodes)))

    frontier = [0]
    for d in range(depth):
        qs = expand(frontier, nodes)
        for i, q in zip(frontier, qs):
            add_children(i, q)
        if d + 1 == depth:
            break
        kept = _top_keep(nodes, keep)
        frontier = sorted((i for i in kept if nodes[i].depth == d + 1), key=lambda i: nodes[i].disc)
        if not frontier:
            break
    kept = _top_keep(nodes, keep)
    return nodes, level_order(nodes, kept, depth)


def level_order(nodes, kept, depth):
    """The root, then the kept nodes in level order: depth, then the
    parent's row, then child rank."""
    row_of = {0: 0}
    order = [0]
    for d in range(1, depth + 1):
        level = [i for i in kept if nodes[i].depth == d]
        level.sort(key=lambda i: (row_of[nodes[i].parent], nodes[i].rank))
        for i in level:
            row_of[i] = len(order)
            order.append(i)
    return order


def ancestors_or_self(nodes, i):
    out = []
    while i >= 0:
        out.append(i)
        i = nodes[i].parent
    return out


def tree_rows(nodes, order, sid, P):
    """Verify rows: position P + depth, slot P + row, visible = committed
    context plus the slots of the node's ancestors and itself."""
    row_of = {n: r for r, n in enumerate(order)}
    rows = []
    for r, n in enumerate(order):
        anc = sorted(P + row_of[a] for a in ancestors_or_self(nodes, n))
        rows.append(Row(sid, P + nodes[n].depth, P + r, np.concatenate([np.arange(P), np.array(anc)])))
    return rows


def parents_of_rows(nodes, order):
    row_of = {n: r for r, n in enumerate(order)}
    return [-1 if nodes[n].parent < 0 else row_of[nodes[n].parent] for n in order]


def masks_of_rows(nodes, order):
    """uint64 ancestor-or-self bit masks over row indices."""
    row_of = {n: r for r, n in enumerate(order)}
    out = []
    for n in order:
        m = 0
        for a in ancestors_or_self(nodes, n):
            m |= 1 << row_of[a]
        out.append(m)
    return out


def draft_tree(dec, cache, st, topk=5, depth=4, keep=63, T=1.0):
    """Tree draft on the decoder: level passes (first L layers + head) to grow
    the tree, then a final first-L pass over the kept rows.

    Returns (nodes, order, tokens per row, hidden_L [rows][d])."""
    L = dec.cfg.exit_layer
    fwd = {}

    def expand(frontier, nodes):
        rows = []
        for i in frontier:
            fwd[i] = len(fwd)
            anc = [st.P + SCRATCH + fwd[a] for a in ancestors_or_self(nodes, i)]
            rows.append(Row(st.sid, st.P + nodes[i].depth, st.P + SCRATCH + fwd[i],
                            np.concatenate([np.arange(st.P), np.array(sorted(anc))])))
        h = dec.forward_layers(cache, rows, dec.embed([nodes[i].token for i in frontier]), 0, L)
        z = dec.head(h)
        return [probs(zz, T) for zz in z]

    nodes, order = build_tree(expand, st.pending, topk, depth, keep)
    toks = [nodes[n].token for n in order]
    rows = tree_rows(nodes, order, st.sid, st.P)
    hL = dec.forward_layers(cache, rows, dec.embed(toks), 0, L)
    return nodes, order, toks, hL


def accept_greedy_tree(toks, parents, logits):
    """Walk from the root; at each node follow the child whose token equals the
    target argmax there.  Returns (a, path rows, y)."""
    cur, path = 0, []
    while True:
        t = argmax(logits[cur])
        nxt = [c for c in range(len(toks)) if parents[c] == cur and toks[c] == t]
        if not nxt:
            return len(path), path, t
        cur = nxt[0]
        path.append(cur)


def commit_tree(cache, st, toks, path, y):
    """Move the accepted nodes' KV to slots P+1..P+a, then advance as a chain."""
    for i, r in enumerate(path):
        cache.copy_slot(st.sid, st.P + r, st.P + 1 + i)
    st.tokens += [int(toks[r]) for r in path] + [int(y)]
    st.P += len(path) + 1
    st.pending = int(y)
    st.rounds.append(len(path))
    cache.poison(st.sid, st.P)
    st.check()

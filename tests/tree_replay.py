"""Replays the tree selection in the oracle on the GPU's own level logits,
so that every integer decision (top-k children, the kept cutoff, the level
order) is taken in the same precision on both sides."""
import numpy as np

from oracle import spec, tree

CUTOFF_BAND = 1e-12  # relative score gap at the kept cutoff below which the choice is a near-tie


def _near_cutoff(nodes, keep):
    s = sorted((nodes[i].score for i in range(1, len(nodes))), reverse=True)
    if len(s) <= keep:
        return False
    return abs(s[keep - 1] - s[keep]) <= CUTOFF_BAND * s[keep - 1]


def replay(level_logits, root_token, T=1.0, topk=5, depth=4, keep=63):
    """Returns (nodes, final order, per-level row orders, near_tie)."""
    layouts = []
    near = [False]

    def expand(frontier, nodes):
        d = nodes[frontier[0]].depth
        kept = set() if d == 0 else tree._top_keep(nodes, keep)
        if d > 0:
            near[0] |= _near_cutoff(nodes, keep)
        order = tree.level_order(nodes, kept, depth)
        layouts.append(order)
        row_of = {n: r for r, n in enumerate(order)}
        return [spec.probs(np.asarray(level_logits[d][row_of[i]], dtype=np.float64), T) for i in frontier]

    nodes, order = tree.build_tree(expand, root_token, topk, depth, keep)
    near[0] |= _near_cutoff(nodes, keep)
    return nodes, order, layouts, near[0]

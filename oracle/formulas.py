"""Closed-form reporting formulas of the pages (oracle).

TEST INFRASTRUCTURE: see ``oracle/__init__.py``.
"""


def expected_tokens(alpha, k):
    """E(k) = (1 - alpha^(k+1)) / (1 - alpha): mean tokens per round with k
    drafts and per-position acceptance alpha (self-speculative decoding page,
    m.lqnn.cn/news/278124, §3.2)."""
    if alpha == 1.0:
        return float(k + 1)
    return (1.0 - alpha ** (k + 1)) / (1.0 - alpha)


def speedup_layer_skip(alpha, k, c):
    """E(k) / (c*k + 1), c = draft cost relative to one full forward (same
    page, §3.2; c is about L/N by §2.3)."""
    return expected_tokens(alpha, k) / (c * k + 1.0)


def speedup_block(a, K, t_over_T):
    """a*T / (T + K*t): accepted tokens a per round, K draft forwards of cost t
    each, one target forward of cost T ("DSpark" page, §2.4)."""
    return a / (1.0 + K * t_over_T)


def confidence(avg_top1, avg_gap, ema_acc):
    """C = 0.4*avg_top1 + 0.3*min(5*avg_gap, 1) + 0.3*EMA(acceptance)
    ("DSpark" page, §2.2)."""
    return 0.4 * avg_top1 + 0.3 * min(avg_gap * 5.0, 1.0) + 0.3 * ema_acc


def next_k(C, min_k, max_k, low, high):
    """Linear map of confidence to the next draft length, clamped ("DSpark"
    page, §2.3)."""
    k = int(min_k + (max_k - min_k) * (C - low) / (high - low))
    return max(min_k, min(max_k, k))

"""Self-speculative decoding round on the float64 decoder (oracle).

TEST INFRASTRUCTURE: see ``oracle/__init__.py``.

Round structure (self-speculative decoding page, m.lqnn.cn/news/278124):
* State: committed tokens; KV valid for positions 0..P-1; the last committed
  token ("pending") sits at position P without KV.  Invariant P ==
  len(tokens) - 1 (the page's §3.3 assert, restated for this convention).
* Draft (§2.1, §4.2): k serial steps of layers 0..L-1 at position P+s,
  writing KV at slot P+s, then final norm + LM head (§3.1: the norm must not be
  skipped), then argmax or a sample from q = softmax(z/T).  Reading: a
  finishing first-L pass over the last draft token gives verify its k+1 rows,
  so verify only runs layers L..N-1 (KV reuse, §2.1 and §2.3).
* Verify (§4.3): layers L..N-1 over rows [x, d_1..d_k] at P..P+k, then the
  head: k+1 distributions; row i judges d_{i+1}, row k is the bonus.
* Accept: greedy = longest prefix where the draft token equals the target's
  argmax, then the target's argmax at the first mismatch ("DSpark" page §2.1;
  greedy is its own branch, self-speculative page §2.4); stochastic = the
  page's accept_or_reject (§4.3) with min(1, p/q), residual max(0, p-q),
  fall back to p when the residual sums to <= 0, bonus from p_k.
* Rollback (§3.3, §4.3): keep x, d_1..d_a, so P <- P + a + 1.  The page's
  "seq_len + i" would drop d_a's KV under its own convention; this is the
  reading listed in the design doc.
"""
from dataclasses import dataclass, field

import numpy as np

from . import formulas
from .decoder import Row, softmax

FLAG_BAND = 1e-3  # |p/q - u| below this marks an acceptance decision as a near-tie
SLOT_ACCEPT = 16  # uniform slots: 0..k-1 draft samples, 16.. accept tests, 32 residual/bonus
SLOT_RESAMPLE = 32
N_UNIFORMS = 48


@dataclass
class SeqState:
    sid: int
    tokens: list
    P: int
    pending: int
    rounds: list = field(default_factory=list)  # accepted count per round

    def check(self):
        assert self.P == len(self.tokens) - 1, (self.P, len(self.tokens))
        assert self.tokens[-1] == self.pending


def argmax(z):
    """Index of the largest value; ties go to the lowest index."""
    return int(np.argmax(z))


def probs(z, T):
    """softmax(z / T) in float64."""
    return softmax(np.asarray(z, dtype=np.float64) / T)


def sample_index(w, u):
    """Inverse-CDF draw from non-negative weights w with a uniform u in [0, 1).

    S = sum(w) and the running sums C_j are taken in float64 in id order; the
    draw is the smallest j with u*S < C_j, else the largest j with w_j > 0.
    A zero-weight id is never returned.
    """
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w)
    S = C[-1]
    j = int(np.searchsorted(C, u * S, side="right"))
    if j >= len(w):
        j = int(np.nonzero(w > 0)[0][-1])
    return j


def top_p_filter(p, top_p):
    """The target truncated to its top-p set and renormalised there
    ("self-speculative" page, §3.4): ids ordered by probability, highest
    first, lower id first among equals; keep the shortest prefix whose
    cumulative probability reaches top_p; zero elsewhere."""
    p = np.asarray(p, dtype=np.float64)
    order = sorted(range(len(p)), key=lambda j: (-p[j], j))
    kept, c = [], 0.0
    for j in order:
        kept.append(j)
        c += p[j]
        if c >= top_p:
            break
    out = np.zeros_like(p)
    out[kept] = p[kept]
    return out / out.sum()


def top_p_margin(p, top_p):
    """How far the cumulative probabilities around the top-p boundary lie from
    top_p (a boundary this close may fall one token either way under another
    summation order)."""
    p = np.asarray(p, dtype=np.float64)
    order = sorted(range(len(p)), key=lambda j: (-p[j], j))
    c = np.cumsum(p[order])
    n = int(np.searchsorted(c >= top_p, True))
    lo = abs(c[n - 1] - top_p) if n > 0 else np.inf
    return min(lo, abs(c[n] - top_p))


def chain_rows(sid, P, n, first=0):
    """Rows first..first+n-1 of a chain at P: position = slot = P+i; row i sees
    slots 0..P+i (committed context plus itself and earlier rows)."""
    return [Row(sid, P + i, P + i, np.arange(P + i + 1)) for i in range(first, first + n)]


def prefill(dec, cache, sid, prompt, mode="greedy", T=1.0, u=None):
    """Run the prompt through all layers; the first generated token is the
    argmax (or a sample with uniform slot 32) of the last row's logits."""
    n = len(prompt)
    rows = [Row(sid, i, i, np.arange(i + 1)) for i in range(n)]
    h = dec.forward_layers(cache, rows, dec.embed(prompt), 0, dec.cfg.n_layers)
    z = dec.head(h[-1:])[0]
    y = argmax(z) if mode == "greedy" else sample_index(probs(z, T), u[SLOT_RESAMPLE])
    st = SeqState(sid, list(int(t) for t in prompt) + [y], n, y)
    st.check()
    return st, z


def draft_chain(dec, cache, st, k, mode="greedy", T=1.0, u=None, exit_layer=None):
    """k draft steps plus the finishing pass.

    Returns (tokens [x, d_1..d_k], draft logits [k][V], hidden_L [k+1][d]).
    """
    L = dec.cfg.exit_layer if exit_layer is None else exit_layer
    toks, zs, hs = [st.pending], [], []
    for s in range(k + 1):
        row = chain_rows(st.sid, st.P, 1, first=s)
        h = dec.forward_layers(cache, row, dec.embed([toks[s]]), 0, L)
        hs.append(h[0])
        if s < k:
            z = dec.head(h)[0]
            zs.append(z)
            toks.append(argmax(z) if mode == "greedy" else sample_index(probs(z, T), u[s]))
    zs = np.array(zs) if zs else np.zeros((0, dec.cfg.vocab))
    return toks, zs, np.array(hs)


def verify_rows(dec, cache, rows, h_or_tokens, start):
    """Layers start..N-1 over the rows, then final norm + head.  With start ==
    0 the rows' inputs are token ids (plain full-depth forward)."""
    h = dec.embed(h_or_tokens) if start == 0 else np.asarray(h_or_tokens, dtype=np.float64)
    h = dec.forward_layers(cache, rows, h, start, dec.cfg.n_layers)
    return dec.head(h)


def verify_chain(dec, cache, st, toks, hidden_L, exit_layer=None):
    L = dec.cfg.exit_layer if exit_layer is None else exit_layer
    rows = chain_rows(st.sid, st.P, len(toks))
    return verify_rows(dec, cache, rows, toks if L == 0 else hidden_L, L)


def accept_greedy_chain(toks, logits):
    """a = longest prefix of drafts matching the target argmax; y = argmax of row a."""
    k = len(toks) - 1
    a = 0
    while a < k and toks[a + 1] == argmax(logits[a]):
        a += 1
    return a, argmax(logits[a])


def accept_stochastic_chain(toks, p_rows, q_rows, u):
    """Stochastic verification of a chain under shared uniforms
    (self-speculative decoding page, m.lqnn.cn/news/278124, §2.4; "推测解码"
    page, §2.2).

    Draft d_{i+1} = toks[i+1] is kept when u[16+i] < min(1, p_i(d)/q_i(d)),
    the ratio being 0 where q_i(d) = 0; a is the number of leading drafts
    kept.  After a rejection at row a the emitted token is drawn with u[32]
    from normalize(max(0, p_a - q_a)), or from p_a when that has no mass;
    when every draft is kept it is drawn from p_k (the bonus row).
    p_rows has k+1 rows, q_rows at least k.  Returns (a, y, flags), flags
    listing the tested rows (0..min(a, k-1)) whose |ratio - u| < 1e-3.
    """
    k = len(toks) - 1
    d = [int(t) for t in toks[1:]]
    ratio = np.array([p_rows[i][d[i]] / q_rows[i][d[i]] if q_rows[i][d[i]] > 0 else 0.0 for i in range(k)],
                     dtype=np.float64)
    ut = np.asarray(u[SLOT_ACCEPT:SLOT_ACCEPT + k], dtype=np.float64)
    kept = ut < np.minimum(1.0, ratio)
    a = k if bool(kept.all()) else int(np.argmin(kept))  # the first rejected row
    flags = [i for i in range(min(a + 1, k)) if abs(ratio[i] - ut[i]) < FLAG_BAND]
    if a == k:
        return k, sample_index(p_rows[k], u[SLOT_RESAMPLE]), flags
    p_a, q_a = np.asarray(p_rows[a], dtype=np.float64), np.asarray(q_rows[a], dtype=np.float64)
    resid = np.maximum(p_a - q_a, 0.0)
    return a, sample_index(resid if resid.sum() > 0 else p_a, u[SLOT_RESAMPLE]), flags


def commit_chain(cache, st, toks, a, y):
    """Keep x, d_1..d_a and append y: P <- P + a + 1; later slots are garbage."""
    st.tokens += [int(t) for t in toks[1:a + 1]] + [int(y)]
    st.P += a + 1
    st.pending = int(y)
    st.rounds.append(a)
    cache.poison(st.sid, st.P)  # a stale read of a rolled-back slot turns into NaN
    st.check()


def spec_round(dec, cache, st, k, mode="greedy", T=1.0, u=None, exit_layer=None):
    """One round: draft, verify, accept, commit.  Returns (a, y, logits, flags)."""
    L = dec.cfg.exit_layer if exit_layer is None else exit_layer
    toks, zd, hL = draft_chain(dec, cache, st, k, mode, T, u, L)
    zt = verify_chain(dec, cache, st, toks, hL, L)
    if mode == "greedy":
        a, y = accept_greedy_chain(toks, zt)
        flags = []
    else:
        p_rows = [probs(z, T) for z in zt]
        q_rows = [probs(z, T) for z in zd]
        a, y, flags = accept_stochastic_chain(toks, p_rows, q_rows, u)
    commit_chain(cache, st, toks, a, y)
    return a, y, zt, flags


def ar_step(dec, cache, st):
    """Plain greedy autoregressive step: the pending token through all layers."""
    z = verify_rows(dec, cache, chain_rows(st.sid, st.P, 1), [st.pending], 0)[0]
    y = argmax(z)
    commit_chain(cache, st, [st.pending], 0, y)
    return y, z


def generate_ar(dec, cache, sid, prompt, n_new):
    st, _ = prefill(dec, cache, sid, prompt)
    while len(st.tokens) - len(prompt) < n_new:
        ar_step(dec, cache, st)
    return st.tokens[len(prompt):len(prompt) + n_new], st


def generate_spec(dec, cache, sid, prompt, n_new, k, exit_layer=None):
    st, _ = prefill(dec, cache, sid, prompt)
    while len(st.tokens) - len(prompt) < n_new:
        spec_round(dec, cache, st, k, exit_layer=exit_layer)
    return st.tokens[len(prompt):len(prompt) + n_new], st


def row_confidence(z_rows, T=1.0):
    """Confidence of the target over a verify block ("DSpark" page, §2.2): the
    mean over the rows of the top-1 probability and of the top-1 minus top-2
    probability, p = softmax(z/T) in float64."""
    top1, gap = [], []
    for z in z_rows:
        p = np.sort(probs(z, T))[::-1]
        top1.append(p[0])
        gap.append(p[0] - p[1])
    return float(np.mean(top1)), float(np.mean(gap))


@dataclass
class SchedState:
    """Per-request draft-length state ("DSpark" page, §2.2-§2.3, and the
    per-request state it asks the scheduler to keep): the draft length of the
    next round and the moving average of the acceptance rate (starts at 0.5)."""
    k: int
    ema: float = 0.5


SCHED = dict(min_k=2, max_k=16, low=0.3, high=0.7)


def schedule_update(state, a, avg_top1, avg_gap, min_k=2, max_k=16, low=0.3, high=0.7):
    """After a round with a accepted of state.k drafts: fold the round's
    acceptance a/k into the average (weight 0.2), form the confidence C from
    the target's mean top-1 probability, its mean top-1/top-2 gap and the
    average, map C linearly onto [min_k, max_k]; a first-draft reject sends K
    straight back to min_k (the page raises K only after a round that kept at
    least one draft and lowers it at once after a first-token reject)."""
    state.ema = 0.2 * (a / state.k) + 0.8 * state.ema
    C = formulas.confidence(avg_top1, avg_gap, state.ema)
    k = formulas.next_k(C, min_k, max_k, low, high)
    state.k = min_k if a == 0 else k
    return state.k, C


def next_k_real(C, min_k=2, max_k=16, low=0.3, high=0.7):
    """The unclamped, untruncated value that next_k truncates (for checks that
    must know how close a decision was to the next integer)."""
    return min_k + (max_k - min_k) * (C - low) / (high - low)


def generate_scheduled(dec, cache, sid, prompt, n_new, k0, **sched):
    """Greedy speculative decoding with the confidence-scheduled draft length:
    each round drafts state.k tokens, verifies, accepts, commits, then updates
    the state from the verify rows' confidence.  Returns (new tokens, the k of
    every round, the (top1, gap, C) of every round, the state)."""
    cfg = dict(SCHED, **sched)
    st, _ = prefill(dec, cache, sid, prompt)
    state = SchedState(max(cfg["min_k"], min(cfg["max_k"], k0)))
    ks, confs = [], []
    while len(st.tokens) - len(prompt) < n_new:
        k = state.k
        a, y, zt, _ = spec_round(dec, cache, st, k)
        top1, gap = row_confidence(zt)
        _, C = schedule_update(state, a, top1, gap, **cfg)
        ks.append(k)
        confs.append((top1, gap, C, a))
    return st.tokens[len(prompt):len(prompt) + n_new], ks, confs, state


@dataclass
class DynKState:
    """Windowed dynamic draft length (self-speculative decoding page, §3.2):
    the controller's k and the (accepted, drafted) counts of recent rounds."""
    k: int
    window: list = field(default_factory=list)
    alpha: float = 1.0


DYNK = dict(window=64, min_k=2, max_k=8, up=0.85, down=0.7)


def dynk_update(state, a, k_used, c_draft=0.0, window=64, min_k=2, max_k=8, up=0.85, down=0.7):
    """After a round that drafted k_used tokens and kept a of them: the
    window's acceptance alpha = accepted / drafted over the last `window`
    rounds; alpha above `up` adds one to k, below `down` takes one away, k
    stays in [min_k, max_k] (§3.2; read as a check every round, like additive
    increase / decrease).  With a draft cost c_draft > 0 (one draft step over
    one full forward, §3.2 and §5.3), the next round drafts at most the k that
    maximises E(k) / (c k + 1); if that k is below min_k, or no k beats plain
    decoding, the next round is a plain decoding step (returns 0, §5.3).  A
    round without drafts leaves the window as it is."""
    if k_used > 0:
        state.window = (state.window + [(a, k_used)])[-window:]
        state.alpha = sum(x for x, _ in state.window) / sum(y for _, y in state.window)
        if state.alpha > up:
            state.k = min(max_k, state.k + 1)
        elif state.alpha < down:
            state.k = max(min_k, state.k - 1)
    k_next = state.k
    if c_draft > 0:
        sp = {k: formulas.speedup_layer_skip(state.alpha, k, c_draft) for k in range(1, max_k + 1)}
        best = max(sp, key=lambda k: (sp[k], -k))
        k_next = 0 if (sp[best] <= 1.0 or best < min_k) else min(k_next, best)
    return k_next


def ngram_propose(history, search_len, min_ngram, max_ngram, k_max):
    """Prompt-copy drafting ("self-speculative" page, §2.2: the next tokens
    are assumed to have appeared already): the longest suffix of the history
    (max_ngram down to min_ngram tokens) that occurs earlier, at its latest
    earlier occurrence whose continuation starts inside the first search_len
    tokens; the proposal is that continuation, at most k_max tokens and not
    past search_len."""
    n = len(history)
    limit = min(n, search_len)
    for g in range(min(max_ngram, n - 1), min_ngram - 1, -1):
        suffix = list(history[n - g:])
        starts = [i for i in range(0, limit - g) if list(history[i:i + g]) == suffix]
        if starts:
            i = max(starts)
            return [int(t) for t in history[i + g:min(i + g + k_max, limit)]]
    return []


def ngram_round(dec, cache, st, k_max, search_len=None, min_ngram=1, max_ngram=3):
    """One greedy round with an n-gram draft and a full-depth verify (start
    layer 0: no first-L KV to reuse); no proposal is a plain decoding step."""
    sl = len(st.tokens) if search_len is None else search_len
    d = ngram_propose(st.tokens, sl, min_ngram, max_ngram, k_max)
    toks = [st.pending] + d
    z = verify_rows(dec, cache, chain_rows(st.sid, st.P, len(toks)), toks, 0)
    a, y = accept_greedy_chain(toks, z)
    commit_chain(cache, st, toks, a, y)
    return d, a, y, z

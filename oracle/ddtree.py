"""Prefix-conditional draft-tree construction (DDTree top-D), in float64
(test infrastructure).

"On the SPOT: Enhancing Speculative Decoding for Diffusion Language Models
via Commit-Order Prediction" (SPOT), Sec. 4.2 ("Inference", Eq. 3) and
App. C.2 (Algorithm 2):

* Drafting starts from the current state x_t with masked positions M(x_t)
  and the stale target conditionals p^_s (one logit row per position).
* Token hypotheses H(s) per masked position, from p^_s alone: at T = 0 the
  argmax of p^_s, plus the runner-up when the top-1 probability is below 0.6;
  at T > 0 the coupled stale draw of Eq. 4, argmax_v [(1/T) log p^_s(v) +
  G[a(s), v]] with the Gumbel row of the position.
* An order model gives q(s | y) over s in M(y) for every hypothetical state
  y; a calibration temperature tau is applied to it before the search.
* A child z = y (+) (s, v) has prefix mass m(z) = m(y) q(s | y) p^_s(v),
  m(x_t) = 1 (Eq. 3).  Every factor lies in [0, 1], so a child's mass never
  exceeds its parent's.
* The tree holds the root and the D states of highest prefix mass.  DDTree
  reaches them level by level; sequential best-first search is the plain
  definition, and both give the same set by the monotonicity above.

Readings (where the pages are silent):
* p^_s(v) in the mass and the 0.6 test is the stale conditional itself, the
  softmax of the stale logits at temperature 1 (the pages write p^, not the
  temperature-adjusted pi^_T, in Eq. 3).
* The order model is an input: a function from a state (its path of (s, v)
  edges from the root) to logits over the block positions; q(s | y) =
  softmax over s in M(y) of logits / tau, zero elsewhere.  The library
  accepts either such rows for each frontier state, level by level, or a
  first-order table whose row is chosen by the last committed position
  (row L for the root), see ``table_order``.
* Ties in mass: the order is mass descending, then depth ascending (a child
  after its parent on equal mass), then the path lexicographically by its
  (position, token) edges.  The set is closed under taking parents.
* Level-batched reading of Algorithm 2: at each level the children of the
  states admitted at the previous level are merged with the tree and the D
  highest kept (earlier states may be displaced); the search stops when no
  new state is admitted.  This is the reading under which the procedure
  gives the best-first set, the property the pages state; filling the
  remaining budget with the next level only would not.
* The prefix-mass floor gamma (SPOT Sec. 4.2, "Adaptive budget"): candidates
  with m(z) < gamma are discarded; gamma = 0 keeps every state.
* The runner-up at T = 0 is the largest logit other than the argmax (lowest
  id on ties); at T = 0 H(s) never holds more than these two tokens, at T > 0
  exactly one.
* A stale row of a root-masked position that is not a distribution (NaN,
  +inf, all -inf), a Gumbel score row that is not one (T > 0), or the order
  row of an expanded state that is not one over M(y), is an error of the
  sequence (the row's status bits); its tree is then not defined.  The
  states expanded are those of the level-batched procedure: every state
  admitted at some level.
"""

import heapq

import numpy as np

from .rows import STATUS_ERROR_MASK, row_status, argmax_lowest

RUNNER_UP_BELOW = 0.6


def stale_softmax(x):
    """p^_s: softmax of one stale logit row at temperature 1."""
    z = np.asarray(x, np.float64)
    w = np.exp(z - np.max(z))
    return w / w.sum()


def hypotheses(row, temperature, gumbel_row=None, runner_up_below=RUNNER_UP_BELOW):
    """H(s) of one masked position as a list of (token, p^_s(token)), with
    the decision margins: ``top1_margin`` = |p^(v0) - runner_up_below| (T = 0)
    and ``pick_margin`` = gap between the two best Gumbel scores (T > 0)."""
    x = np.asarray(row, np.float64)
    p = stale_softmax(x)
    if temperature == 0.0:
        v0 = argmax_lowest(x)
        hyp = [(v0, float(p[v0]))]
        top1_margin = abs(float(p[v0]) - runner_up_below)
        if p[v0] < runner_up_below and x.size > 1:
            rest = x.copy()
            rest[v0] = -np.inf
            v1 = argmax_lowest(rest)
            hyp.append((v1, float(p[v1])))
        return dict(hyp=hyp, top1_margin=top1_margin, pick_margin=np.inf)
    g = np.asarray(gumbel_row, np.float64)
    with np.errstate(divide="ignore"):
        score = np.log(p) / float(temperature) + g
    v = argmax_lowest(score)
    s = np.sort(score)
    gap = float(s[-1] - s[-2]) if s.size > 1 else np.inf
    return dict(hyp=[(v, float(p[v]))], top1_margin=np.inf, pick_margin=gap)


def order_distribution(logits, masked_positions, tau):
    """q(s | y) over the masked positions of y (zeros elsewhere): softmax of
    the order logits / tau restricted to M(y).  None when the restricted row
    is not a distribution."""
    z = np.asarray(logits, np.float64)
    q = np.zeros(z.size)
    ms = list(masked_positions)
    if not ms:
        return q
    sub = z[ms] / float(tau)
    if row_status(sub):
        return None
    w = np.exp(sub - np.max(sub))
    q[ms] = w / w.sum()
    return q


def table_order(table):
    """The first-order table order model: the order logits of state y in
    sequence b are table[b, c], c the position committed by the last edge of
    y's path, or c = L for the root."""
    table = np.asarray(table, np.float64)

    def fn(b, path):
        L = table.shape[-1]
        return table[b, path[-1][0] if path else L]
    return fn


def rank_key(mass, path):
    """Sort key of a state: mass descending, depth ascending, then the path."""
    return (-mass, len(path), tuple(path))


class _Search:
    """Children of a state under one sequence's hypotheses and order model."""

    def __init__(self, masked, hyps, order_fn, b, tau, gamma):
        self.root_masked = [s for s in range(len(masked)) if masked[s]]
        self.hyps = hyps
        self.order_fn = order_fn
        self.b = b
        self.tau = tau
        self.gamma = gamma
        self.status = 0

    def masked_of(self, path):
        done = {s for s, _ in path}
        return [s for s in self.root_masked if s not in done]

    def children(self, path, mass):
        ms = self.masked_of(path)
        if not ms:
            return []
        z = np.asarray(self.order_fn(self.b, tuple(path)), np.float64)
        q = order_distribution(z, ms, self.tau)
        if q is None:
            self.status |= row_status(z[ms])
            return []
        out = []
        for s in ms:
            for v, pv in self.hyps[s]:
                m = mass * q[s] * pv
                if m >= self.gamma:
                    out.append((tuple(path) + ((s, v),), m))
        return out


def best_first(masked, hyps, order_fn, D, tau=1.0, gamma=0.0, b=0):
    """The D states of highest prefix mass by sequential best-first search:
    take the best candidate, add its children to the candidates, repeat.
    Returns ([(path, mass)] in rank order, status bits of bad order rows)."""
    srch = _Search(masked, hyps, order_fn, b, tau, gamma)
    if D <= 0:
        return [], 0
    heap = [(rank_key(m, p), p, m) for p, m in srch.children((), 1.0)]
    heapq.heapify(heap)
    chosen = []
    while len(chosen) < D and heap:
        _, p, m = heapq.heappop(heap)
        chosen.append((p, m))
        for c in srch.children(p, m):
            heapq.heappush(heap, (rank_key(c[1], c[0]), c[0], c[1]))
    return chosen, srch.status


def level_batched(masked, hyps, order_fn, D, tau=1.0, gamma=0.0, b=0):
    """SPOT Algorithm 2 under the level-batched reading: expand the states
    admitted last, keep the D best of the tree and the new candidates,
    repeat until nothing new is admitted.  Returns ([(path, mass)] in rank
    order, status bits of bad order rows, levels run)."""
    srch = _Search(masked, hyps, order_fn, b, tau, gamma)
    tree = []
    frontier = [((), 1.0)]
    levels = 0
    while frontier and D > 0:
        cand = []
        for p, m in frontier:
            cand.extend(srch.children(p, m))
        levels += 1
        pool = sorted(tree + cand, key=lambda e: rank_key(e[1], e[0]))[:D]
        old = {p for p, _ in tree}
        frontier = [e for e in pool if e[0] not in old]
        tree = pool
    return tree, srch.status, levels


def tree_arrays(chosen, masked):
    """Node arrays of a chosen set in rank order (node 0 the root): parent,
    edge position, edge token, mass, depth and the masked positions of each
    state (the layout the tree verifier reads)."""
    L = len(masked)
    n = len(chosen) + 1
    index = {(): 0}
    parent = np.full(n, -1, np.int64)
    pos = np.full(n, -1, np.int64)
    tok = np.full(n, -1, np.int64)
    mass = np.zeros(n)
    depth = np.zeros(n, np.int64)
    mk = np.zeros((n, L), np.uint8)
    mass[0] = 1.0
    mk[0] = np.asarray(masked, np.uint8)
    for z, (p, m) in enumerate(chosen, start=1):
        index[p] = z
        y = index[p[:-1]]
        parent[z] = y
        pos[z], tok[z] = p[-1]
        mass[z] = m
        depth[z] = len(p)
        mk[z] = mk[y]
        mk[z, p[-1][0]] = 0
    return dict(parent=parent, pos=pos, tok=tok, mass=mass, depth=depth, masked=mk)


def build_ddtree(stale, masked, order_fn, D, temperature, tau=1.0, gamma=0.0, gumbel=None,
                 runner_up_below=RUNNER_UP_BELOW):
    """Hypotheses and the top-D tree of every sequence.

    stale [B, L, V] stale logits (rows at masked positions are read),
    masked [B, L] the masked positions of the current state, order_fn(b,
    path) -> [L] order logits, gumbel [B, L, V] (T > 0).  Returns per
    sequence: ``hyp_tok`` / ``hyp_prob`` [B, L, 2] (-1 / 0 where absent),
    the margins, ``hyp_status`` (rows of the hypotheses), ``status`` (with
    the order rows of the search) and ``trees`` (a list of ``tree_arrays`` dicts,
    None for a sequence in error)."""
    stale = np.asarray(stale)
    B, L, V = stale.shape
    masked = np.asarray(masked).astype(bool)
    out = dict(hyp_tok=np.full((B, L, 2), -1, np.int64), hyp_prob=np.zeros((B, L, 2)),
               top1_margin=np.full((B, L), np.inf), pick_margin=np.full((B, L), np.inf),
               status=np.zeros(B, np.int64), hyp_status=np.zeros(B, np.int64), trees=[None] * B,
               chosen=[None] * B)
    for b in range(B):
        st = 0
        for s in range(L):
            if masked[b, s]:
                st |= row_status(stale[b, s])
        if st & STATUS_ERROR_MASK:
            out["status"][b] = out["hyp_status"][b] = st
            continue
        hyps = []
        for s in range(L):
            if not masked[b, s]:
                hyps.append([])
                continue
            h = hypotheses(stale[b, s], temperature, None if gumbel is None else gumbel[b, s],
                           runner_up_below)
            if temperature > 0.0:
                with np.errstate(divide="ignore"):
                    st |= row_status(np.log(stale_softmax(stale[b, s])) / temperature
                                     + np.asarray(gumbel[b, s], np.float64))
            hyps.append(h["hyp"])
            out["top1_margin"][b, s] = h["top1_margin"]
            out["pick_margin"][b, s] = h["pick_margin"]
            for k, (v, pv) in enumerate(h["hyp"]):
                out["hyp_tok"][b, s, k] = v
                out["hyp_prob"][b, s, k] = pv
        out["hyp_status"][b] = st
        if st & STATUS_ERROR_MASK:
            out["status"][b] = st
            continue
        chosen, ost, _ = level_batched(masked[b], hyps, order_fn, D, tau, gamma, b)
        st |= ost
        out["status"][b] = st
        if not st & STATUS_ERROR_MASK:
            out["chosen"][b] = chosen
            out["trees"][b] = tree_arrays(chosen, masked[b])
    return out

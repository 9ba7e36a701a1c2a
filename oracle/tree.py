"""Coupled shared-Gumbel state-equality verification of a draft tree.

Test infrastructure (see the package docstring).  Follows SPOT, Sec. 4.1
and 4.3 and App. A.1:

* a state y of the active block has masked positions M(y);
* s*(y) = argmax over s in M(y) of max_v p_s(v | y), ties to the lowest
  position ("fixed deterministic tie-breaking rule");
* at T > 0 the target's draw is v*_G(y) = argmax_v [(1/T) log p_{s*}(v) +
  G[a(s*), v]] with a Gumbel table shared by drafter and verifier and indexed
  by absolute position; at T = 0 it is the argmax of p_{s*};
* Phi(y) = y (+) (s*(y), v*(y)); an edge (y, z) is accepted exactly when z
  equals Phi(y).  Walking from the root, the verifier follows the child equal
  to Phi(y_j); when none exists it commits Phi(y_j) itself and stops; a
  terminal state (no masked position) makes no transition.

Tree layout (one row per sequence b, nodes 0..S-1, node 0 the root):
``parent[b, z] < z`` (``parent[b, 0] = -1``); the edge into z commits
``edge_tok[b, z]`` at block position ``edge_pos[b, z]``; ``masked[b, z, s]``
marks the masked positions of state z; ``logits[b, z, s, :]`` is the target's
conditional at position s of state z; ``gumbel[b, s, :]`` is the Gumbel row of
the absolute position of block position s.

In the fixed-position mode the position of every state's transition is
given (``next_pos[b, z]``, -1 for a state that makes no transition) and only
the token is drawn there; this is the chain / autoregressive special case.
"""

import numpy as np

from .rows import (
    STATUS_BAD_INPUT, STATUS_ERROR_MASK, row_status,
    max_probability, argmax_lowest,
)

TREE_STATE_EQUALITY = 0
TREE_FIXED_POSITION = 1


def _log_tempered_softmax(x, temperature):
    a = np.asarray(x, dtype=np.float64) / float(temperature)
    m = np.max(a)
    return a - m - np.log(np.sum(np.exp(a - m)))


def _top2_gap(values):
    """Gap between the largest and second-largest entry (inf if < 2)."""
    v = np.sort(np.asarray(values, dtype=np.float64))
    if v.size < 2:
        return np.inf
    return float(v[-1] - v[-2])


def state_transition(rows, masked_positions, gumbel, temperature, fixed_pos=None):
    """Phi(y) for one state.

    ``rows[s]`` is the logit row at block position s, ``masked_positions`` the
    ordered list M(y) (ignored when ``fixed_pos`` is given), ``gumbel[s]`` the
    Gumbel row of position s (unused at T = 0).

    Returns dict(pos, tok, conf, pos_margin, tok_margin, status); pos = -1
    for a terminal state.
    """
    res = dict(pos=-1, tok=-1, conf=np.nan, pos_margin=np.inf,
               tok_margin=np.inf, status=0)
    if fixed_pos is None:
        if len(masked_positions) == 0:
            return res
        status = 0
        for s in masked_positions:
            status |= row_status(rows[s])
        if status & STATUS_ERROR_MASK:
            res["status"] = status
            return res
        conf = [max_probability(rows[s]) for s in masked_positions]
        best = max(conf)
        s_star = min(s for s, c in zip(masked_positions, conf) if c == best)
        res["pos_margin"] = _top2_gap(conf) / best
        res["conf"] = best
    else:
        if fixed_pos < 0:
            return res
        s_star = int(fixed_pos)
        status = row_status(rows[s_star])
        if status & STATUS_ERROR_MASK:
            res["status"] = status
            return res
        res["conf"] = max_probability(rows[s_star])

    x = rows[s_star]
    if temperature > 0.0:
        g = np.asarray(gumbel[s_star], dtype=np.float64)
        with np.errstate(invalid="ignore"):
            score = _log_tempered_softmax(x, temperature) + g
        # The score row obeys the logit-row rule: NaN / +inf (from the
        # Gumbel row) is an error, -inf is a zero-weight entry.
        st = row_status(score)
        if st:
            res["status"] = st
            return res
        tok = argmax_lowest(score)
        res["tok_margin"] = _top2_gap(score)
    else:
        tok = argmax_lowest(x)
    res["pos"] = int(s_star)
    res["tok"] = int(tok)
    return res


def walk(parent, edge_pos, edge_tok, ns, pos, tok):
    """State-equality walk from the root (SPOT, App. A.1, state-equality
    verifier): follow the child equal to Phi(y) (lowest node index if there
    are several), else commit Phi(y) and stop; a state with pos = -1 makes no
    transition.  ``pos[y], tok[y]`` is Phi(y).  Returns (path, commits)."""
    y = 0
    path = [0]
    commits = []
    while pos[y] >= 0:
        match = [z for z in range(1, ns) if parent[z] == y
                 and edge_pos[z] == pos[y] and edge_tok[z] == tok[y]]
        if not match:
            commits.append((int(pos[y]), int(tok[y])))
            break
        y = match[0]
        path.append(y)
        commits.append((int(edge_pos[y]), int(edge_tok[y])))
    return path, commits


def verify_gumbel_tree(logits, masked, parent, edge_pos, edge_tok,
                       num_states=None, gumbel=None, temperature=1.0,
                       mode=TREE_STATE_EQUALITY, next_pos=None):
    """State-equality verification of one draft tree per sequence.

    Returns per-state selections (sel_pos, sel_tok, sel_conf), the accepted
    path (path_len = number of accepted edges, path_nodes starting at the
    root), the commitments (accepted edges, then Phi of the last accepted
    state unless it is terminal) and the status.
    """
    logits = np.asarray(logits)
    B, S, L, V = logits.shape
    parent = np.asarray(parent).reshape(B, S)
    edge_pos = np.asarray(edge_pos).reshape(B, S)
    edge_tok = np.asarray(edge_tok).reshape(B, S)
    fixed = mode == TREE_FIXED_POSITION

    out = dict(
        sel_pos=np.full((B, S), -1, np.int32), sel_tok=np.full((B, S), -1, np.int32),
        sel_conf=np.full((B, S), np.nan), pos_margin=np.full((B, S), np.inf),
        tok_margin=np.full((B, S), np.inf),
        path_len=np.full(B, -1, np.int32), path_nodes=np.full((B, S), -1, np.int32),
        commit_pos=np.full((B, S), -1, np.int32), commit_tok=np.full((B, S), -1, np.int32),
        num_commits=np.zeros(B, np.int32), status=np.zeros(B, np.int32),
    )
    for b in range(B):
        ns = S if num_states is None else int(np.asarray(num_states)[b])
        status = 0
        if ns < 1 or ns > S:
            out["status"][b] = STATUS_BAD_INPUT
            continue
        if parent[b, 0] != -1:
            status |= STATUS_BAD_INPUT
        for z in range(1, ns):
            if not (0 <= parent[b, z] < z):
                status |= STATUS_BAD_INPUT
            if not (0 <= edge_pos[b, z] < L) or not (0 <= edge_tok[b, z] < V):
                status |= STATUS_BAD_INPUT
            if fixed and not (-1 <= int(np.asarray(next_pos)[b, z]) < L):
                status |= STATUS_BAD_INPUT
        if fixed and not (-1 <= int(np.asarray(next_pos)[b, 0]) < L):
            status |= STATUS_BAD_INPUT
        if status & STATUS_ERROR_MASK:
            out["status"][b] = status
            continue

        trans = []
        for z in range(ns):
            if fixed:
                t = state_transition(logits[b, z], None,
                                     None if gumbel is None else gumbel[b],
                                     temperature, fixed_pos=int(np.asarray(next_pos)[b, z]))
            else:
                mpos = [s for s in range(L) if masked[b, z, s]]
                t = state_transition(logits[b, z], mpos,
                                     None if gumbel is None else gumbel[b],
                                     temperature)
            status |= t["status"]
            trans.append(t)
        out["status"][b] = status
        if status & STATUS_ERROR_MASK:
            continue
        for z, t in enumerate(trans):
            out["sel_pos"][b, z] = t["pos"]
            out["sel_tok"][b, z] = t["tok"]
            out["sel_conf"][b, z] = t["conf"]
            out["pos_margin"][b, z] = t["pos_margin"]
            out["tok_margin"][b, z] = t["tok_margin"]

        path, commits = walk(parent[b], edge_pos[b], edge_tok[b], ns,
                             [t["pos"] for t in trans], [t["tok"] for t in trans])
        out["path_len"][b] = len(path) - 1
        out["path_nodes"][b, :len(path)] = path
        for k, (s, v) in enumerate(commits):
            out["commit_pos"][b, k] = s
            out["commit_tok"][b, k] = v
        out["num_commits"][b] = len(commits)
    return out

"""Chain verification on the joint (position, token) space, in float64 (test
infrastructure).

"On the SPOT: Enhancing Speculative Decoding for Diffusion Language Models
via Commit-Order Prediction", App. B (rejection sampling as an alternative
verifier), Eq. 10-14 and Proposition 3, and the regime law of its Table 22
discussion (a confidence-gated hybrid of coupled-noise match and rejection
sampling on chains).

One link k of a drafted chain sits at a verified state y_k.  The target
commits at one position, s*_k = s*(y_k), with token law pi_T (Eq. 10):
    pi_k(s, v) = 1{s = s*_k} p_k(v),   p_k = tempered target row at s*_k.
The drafter proposed z~_k = (s~_k, v~_k) from (Eq. 12)
    q_k(s, v) = q_pos_k(s) qhat_{k,s}(v),
qhat the drafter's stale tempered token conditional.  Rejection sampling
(Eq. 13-14): accept with min{1, pi_k(z~) / q_k(z~)}; on rejection draw from
normalize((pi_k - q_k)_+) over the joint space.  Off s*_k, pi_k = 0, so a
proposal elsewhere is rejected and the residual lives on s*_k alone:
    r_k(v) = [p_k(v) - c_k qhat_{k,s*}(v)]_+,   c_k = q_pos_k(s*_k).
Coupled-noise match (SPOT Sec. 4.1, App. A.1): with the shared Gumbel row g
of position s*_k, the target's commit is (s*_k, argmax_v [(1/T) log p(v) +
g(v)]) and the proposal is accepted exactly when it equals that pair.

Inputs per sequence (K = drafted links, n <= K valid):
  tgt  [K+1, V]  target logits at (y_k, s*_k), k = 0..K (row n: the bonus)
  drf  [K, V]    drafter logits at (k, s*_k)
  pos_star [K+1], prop_pos [K], prop_tok [K], q_pos_star [K] = c_k
  u_accept [K], u_resample [K+1], gumbel [K+1, V] (optional).

Readings (where the pages are silent):
* The committed position of every link is s*_k (accepted links propose it;
  a rejected link commits there), so positions are not an output.
* The hybrid's stale confidence of link k is max_v qhat_{k,s*}(v), the
  drafter's confidence at the position the link commits.  Where the
  proposal sits elsewhere the link rejects under either verifier, and the
  gate only picks how the forced commit is drawn; p_k is its law either
  way.  Match is used when a Gumbel row is given and the confidence is at
  least tau, rejection sampling otherwise.
* The bonus after n accepted links is the target's commit at y_n: the
  Gumbel argmax of row n when Gumbel rows are given, else an inverse-CDF
  draw from p_n.
* With Gumbel rows given every row 0..n is read with its Gumbel row (their
  score rows obey the logit-row rule).  c_k must lie in [0, 1], pos_star_k
  must be >= 0 for k <= n, and v~_k must lie in [0, V).
* c_k qhat(v~) = 0 at a proposal on s*_k: the ratio is read as +inf when
  p(v~) > 0 (accept, flagged) and 0 otherwise, as in the token chain.
"""

import numpy as np

from .rows import (
    STATUS_BAD_INPUT, STATUS_ERROR_MASK, STATUS_Q_ZERO, STATUS_Z_ZERO,
    row_status, tempered_softmax, argmax_lowest, inverse_cdf, stopping_index,
)

MODE_RS = 0
MODE_MATCH = 1


def _gumbel_scores(x, g, temperature):
    """(1/T) log pi_T(v) + g(v) for one row (SPOT Sec. 4.1)."""
    a = np.asarray(x, np.float64) / float(temperature)
    m = np.max(a)
    with np.errstate(invalid="ignore"):
        return a - m - np.log(np.sum(np.exp(a - m))) + np.asarray(g, np.float64)


def _top2_gap(values):
    v = np.sort(np.asarray(values, np.float64))
    return np.inf if v.size < 2 else float(v[-1] - v[-2])


def rs_link(u, p, qhat, c, on_star, tok):
    """The rejection-sampling test of one link (SPOT Eq. 13).

    q(z~) = c qhat(v~) when the proposal sits on s*, and pi(z~) = 0
    otherwise.  Returns (accepted, alpha, margin, q_zero_flag).
    """
    if not on_star:
        return False, 0.0, np.inf, False
    pz = float(p[tok])
    qz = float(c) * float(qhat[tok])
    if qz > 0.0:
        alpha = min(1.0, pz / qz)
    else:
        alpha = 1.0 if pz > 0.0 else 0.0
    return bool(u < alpha), alpha, abs(u - alpha), bool(qz == 0.0 and pz > 0.0)


def rs_residual(p, qhat, c):
    """(pi_k - q_k)_+ restricted to s*_k (SPOT Eq. 14): [p - c qhat]_+."""
    return np.maximum(np.asarray(p, np.float64) - float(c) * np.asarray(qhat, np.float64), 0.0)


def verify_spot_chain(tgt, drf, pos_star, prop_pos, prop_tok, q_pos_star, draft_len,
                      t_target, t_draft, u_accept, u_resample, gumbel=None, tau=0.6,
                      eos_id=-1, len_budget=None):
    """Chain verification on the joint space for B sequences: rejection
    sampling per link (gumbel=None), or the confidence-gated hybrid of
    match (stale confidence >= tau) and rejection sampling.

    Returns accept_len (h), num_out, out_tokens (C = v~_0..v~_{h-1}, c after
    the ending condition), status, per-link p_draft, q_draft (= c qhat(v~)),
    alpha, mode, conf, accept_margin, and per-sequence residual_mass,
    draw_margin, draw_row, draw_kind.
    """
    tgt = np.asarray(tgt)
    B, K1, V = tgt.shape
    K = K1 - 1
    drf = np.asarray(drf)
    ps = np.asarray(pos_star).reshape(B, K + 1)
    pp = np.asarray(prop_pos).reshape(B, K) if K > 0 else np.zeros((B, 0), np.int64)
    pt = np.asarray(prop_tok).reshape(B, K) if K > 0 else np.zeros((B, 0), np.int64)
    cs = np.asarray(q_pos_star, np.float64).reshape(B, K) if K > 0 else np.zeros((B, 0))
    ua = np.asarray(u_accept, np.float64).reshape(B, K) if K > 0 else np.zeros((B, 0))
    ur = np.asarray(u_resample, np.float64).reshape(B, K + 1)
    G = None if gumbel is None else np.asarray(gumbel)
    lens = [K] * B if draft_len is None else [int(v) for v in np.asarray(draft_len).reshape(-1)]

    out = dict(
        accept_len=np.full(B, -1, np.int32), num_out=np.zeros(B, np.int32),
        out_tokens=np.full((B, K + 1), -1, np.int32), status=np.zeros(B, np.int32),
        p_draft=np.zeros((B, K)), q_draft=np.zeros((B, K)), alpha=np.zeros((B, K)),
        mode=np.zeros((B, K), np.int32), conf=np.zeros((B, K)),
        accept_bits=np.zeros((B, K), bool), accept_margin=np.full((B, K), np.inf),
        gate_margin=np.full((B, K), np.inf),
        residual_mass=np.zeros(B), draw_margin=np.full(B, np.inf),
        draw_row=np.full(B, -1, np.int32), draw_kind=[None] * B,
    )
    for b in range(B):
        n = lens[b]
        status = 0
        budget = None if len_budget is None else int(np.asarray(len_budget)[b])
        rows_read = n + 1
        if n < 0 or n > K:
            status |= STATUS_BAD_INPUT
            n, rows_read = 0, 0
        if budget is not None and budget < 0:
            status |= STATUS_BAD_INPUT
        d = [int(t) for t in pt[b, :n]]
        if any(t < 0 or t >= V for t in d):
            status |= STATUS_BAD_INPUT
        if any(int(s) < 0 for s in ps[b, :rows_read]):
            status |= STATUS_BAD_INPUT
        if any(not (0.0 <= c <= 1.0) for c in cs[b, :n]):
            status |= STATUS_BAD_INPUT
        for i in range(rows_read):
            status |= row_status(tgt[b, i])
        for i in range(n):
            status |= row_status(drf[b, i])
        scores = []
        if G is not None:
            for i in range(rows_read):
                with np.errstate(invalid="ignore", over="ignore"):
                    s = _gumbel_scores(tgt[b, i], G[b, i], t_target)
                status |= row_status(s)
                scores.append(s)
        if status & STATUS_ERROR_MASK:
            out["status"][b] = status
            continue

        p = [tempered_softmax(tgt[b, i], t_target) for i in range(n + 1)]
        qh = [tempered_softmax(drf[b, i], t_draft) for i in range(n)]
        gtok = [argmax_lowest(s) for s in scores]
        for i in range(n):
            on_star = int(pp[b, i]) == int(ps[b, i])
            conf = float(np.max(qh[i]))
            mode = MODE_MATCH if (G is not None and conf >= tau) else MODE_RS
            out["conf"][b, i] = conf
            out["mode"][b, i] = mode
            out["gate_margin"][b, i] = abs(conf - tau)
            out["p_draft"][b, i] = p[i][d[i]]
            out["q_draft"][b, i] = cs[b, i] * qh[i][d[i]]
            if mode == MODE_RS:
                acc, alpha, margin, qz = rs_link(ua[b, i], p[i], qh[i], cs[b, i], on_star, d[i])
                if qz:
                    status |= STATUS_Q_ZERO
            else:
                acc = on_star and d[i] == gtok[i]
                alpha = 1.0 if acc else 0.0
                margin = _top2_gap(scores[i])
            out["alpha"][b, i] = alpha
            out["accept_bits"][b, i] = acc
            out["accept_margin"][b, i] = margin
        h = 0
        while h < n and out["accept_bits"][b, h]:
            h += 1

        if h < n and out["mode"][b, h] == MODE_RS:
            r = rs_residual(p[h], qh[h], cs[b, h])
            if np.sum(r) > 0.0:
                c, margin, Z = inverse_cdf(r, ur[b, h])
                kind = "residual"
            else:
                status |= STATUS_Z_ZERO
                c, margin, _ = inverse_cdf(p[h], ur[b, h])
                Z = 0.0
                kind = "residual_fallback"
            out["residual_mass"][b] = Z
        elif h < n:
            c, margin, kind = gtok[h], _top2_gap(scores[h]), "match"
        elif G is not None:
            c, margin, kind = gtok[n], _top2_gap(scores[n]), "match_bonus"
        else:
            c, margin, _ = inverse_cdf(p[n], ur[b, n])
            kind = "bonus"
        out["draw_margin"][b] = margin
        out["draw_row"][b] = h
        out["draw_kind"][b] = kind

        C = d[:h] + [c]
        a = stopping_index(C, h + 1, eos_id, budget)
        out["status"][b] = status
        out["accept_len"][b] = h
        out["num_out"][b] = a
        out["out_tokens"][b, :a] = C[:a]
    return out

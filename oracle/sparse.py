"""Verification against a stored sparse drafter distribution, in float64
(test infrastructure).

"One Call Ahead: Packed Self-Speculative Decoding with Diffusion Drafting",
Sec. 3.2: each draft token is stored with the distribution Q it was sampled
from, and with top-k or top-p truncation only Q's nonzero entries need to be
stored.  Verification is the lossless rule of App. B.2 (Algorithm 2) with
that Q: accept d with min{1, p(d) / Q(d)}, correct a rejection from
normalize([p - Q]_+), draw the bonus from p.  A token outside the stored
support has Q = 0, so the residual there is p itself.

Layout per sequence: q_idx [K, kmax] token ids, q_prob [K, kmax] their
probabilities, q_nnz [K] entries in use (the first q_nnz of each row).

Readings (where the page is silent):
* Q is used as stored: the entries are not renormalised.  The indices of one
  row are distinct (a caller contract; not checked).
* Entries beyond q_nnz are never read.  Bad input: q_nnz outside [0, kmax],
  an index outside [0, V), or a probability that is negative or not finite,
  in a row that the call reads (rows 0..n-1).
"""

import numpy as np

from .rows import (
    STATUS_BAD_INPUT, STATUS_ERROR_MASK, STATUS_Q_ZERO, STATUS_Z_ZERO,
    row_status, tempered_softmax, acceptance_test, inverse_cdf, residual_weights, stopping_index,
)


def dense_q(idx, prob, nnz, V):
    """The stored distribution as a length-V vector (zeros off its support)."""
    q = np.zeros(V)
    k = int(nnz)
    q[np.asarray(idx[:k], np.int64)] = np.asarray(prob[:k], np.float64)
    return q


def sparse_row_ok(idx, prob, nnz, kmax, V):
    k = int(nnz)
    if k < 0 or k > kmax:
        return False
    i = np.asarray(idx[:k], np.int64)
    p = np.asarray(prob[:k], np.float64)
    return bool(((i >= 0) & (i < V)).all() and np.isfinite(p).all() and (p >= 0).all())


def verify_sparse(tgt, q_idx, q_prob, q_nnz, draft_tokens, draft_len, t_target, u_accept,
                  u_resample, eos_id=-1, len_budget=None):
    """Lossless verification of B drafted chains against sparse stored Q.

    Returns accept_len, num_out, out_tokens, status, per-draft p_draft,
    q_draft, alpha, accept margins, and per-sequence residual_mass,
    draw_margin, draw_row, draw_kind (as the token-chain verifiers).
    """
    tgt = np.asarray(tgt)
    B, K1, V = tgt.shape
    K = K1 - 1
    kmax = np.asarray(q_idx).shape[-1] if K > 0 else 0
    qi = np.asarray(q_idx).reshape(B, K, kmax) if K > 0 else np.zeros((B, 0, 0), np.int64)
    qp = np.asarray(q_prob, np.float64).reshape(B, K, kmax) if K > 0 else np.zeros((B, 0, 0))
    qn = np.asarray(q_nnz).reshape(B, K) if K > 0 else np.zeros((B, 0), np.int64)
    d_all = np.asarray(draft_tokens).reshape(B, K) if K > 0 else np.zeros((B, 0), np.int64)
    ua = np.asarray(u_accept, np.float64).reshape(B, K) if K > 0 else np.zeros((B, 0))
    ur = np.asarray(u_resample, np.float64).reshape(B, K + 1)
    lens = [K] * B if draft_len is None else [int(v) for v in np.asarray(draft_len).reshape(-1)]

    out = dict(
        accept_len=np.full(B, -1, np.int32), num_out=np.zeros(B, np.int32),
        out_tokens=np.full((B, K + 1), -1, np.int32), status=np.zeros(B, np.int32),
        p_draft=np.zeros((B, K)), q_draft=np.zeros((B, K)), alpha=np.zeros((B, K)),
        accept_bits=np.zeros((B, K), bool), accept_margin=np.full((B, K), np.inf),
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
        d = [int(t) for t in d_all[b, :n]]
        if any(t < 0 or t >= V for t in d):
            status |= STATUS_BAD_INPUT
        if not all(sparse_row_ok(qi[b, i], qp[b, i], qn[b, i], kmax, V) for i in range(n)):
            status |= STATUS_BAD_INPUT
        for i in range(rows_read):
            status |= row_status(tgt[b, i])
        if status & STATUS_ERROR_MASK:
            out["status"][b] = status
            continue
        p = [tempered_softmax(tgt[b, i], t_target) for i in range(n + 1)]
        Q = [dense_q(qi[b, i], qp[b, i], qn[b, i], V) for i in range(n)]
        for i in range(n):
            acc, alpha, margin, qz = acceptance_test(ua[b, i], p[i][d[i]], Q[i][d[i]])
            out["p_draft"][b, i] = p[i][d[i]]
            out["q_draft"][b, i] = Q[i][d[i]]
            out["alpha"][b, i] = alpha
            out["accept_bits"][b, i] = acc
            out["accept_margin"][b, i] = margin
            if qz:
                status |= STATUS_Q_ZERO
        h = 0
        while h < n and out["accept_bits"][b, h]:
            h += 1
        if h < n:
            r = residual_weights(p[h], Q[h])
            if np.sum(r) > 0.0:
                c, margin, Z = inverse_cdf(r, ur[b, h])
                kind = "residual"
            else:
                status |= STATUS_Z_ZERO
                c, margin, _ = inverse_cdf(p[h], ur[b, h])
                Z = 0.0
                kind = "residual_fallback"
            out["residual_mass"][b] = Z
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

"""Per-sequence verification of a drafted chain (test infrastructure).

Layouts follow the library's calling convention:

* ``tgt``  [B, K+1, V]: target logits; row i (0-based) is the verifier's
  conditional at draft position i+1, row n_b is the bonus row.
* ``drf``  [B, K, V]  : the logits of the distribution each draft token was
  sampled from (Packed-SS, Sec. 3.2: the stored proposal Q).
* ``draft_tokens`` [B, K], ``draft_len`` [B] (n_b <= K; None means K).
* ``draft_rows`` [B, W, V] (greedy only): the drafter rows of the same call
  whose argmax forms the next draft (Packed-SS, Eq. 3-4).

Outputs are dicts of numpy arrays, with -1 in unused slots, plus per-row
decision details (alpha, margins) used by the parity checker.
"""

import numpy as np

from .rows import (
    STATUS_BAD_INPUT, STATUS_ERROR_MASK, STATUS_Q_ZERO, STATUS_Z_ZERO,
    row_status, tempered_softmax, argmax_lowest, acceptance_test,
    inverse_cdf, residual_weights, stopping_index,
)
from .cactus import cactus_acceptance, cactus_residual


def _lengths(draft_len, B, K):
    if draft_len is None:
        return [K] * B
    return [int(v) for v in np.asarray(draft_len).reshape(-1)]


def _budget(len_budget, b):
    return None if len_budget is None else int(np.asarray(len_budget)[b])


def verify_greedy(tgt, draft_tokens, draft_len=None, draft_rows=None,
                  eos_id=-1, len_budget=None):
    """Greedy (temperature 0) verification and next-draft retention.

    Packed-SS, Sec. 3.1 and Algorithm 1:
      v_i = argmax p(. | P, d_<i) for i = 1..|D|+1              (Eq. 1)
      h   = max{h <= |D| : d_i = v_i for all i <= h}             (Eq. 2)
      C   = (d_1..d_h, v_{h+1}),  A = h + 1
      a   = ending condition (EOS / length), C pruned to a
      z_j = argmax q^(j)(. | P) for j = 1..W                     (Eq. 3)
      D'  = (z_{a+1}, ..., z_W)                                  (Eq. 4)
    """
    tgt = np.asarray(tgt)
    B, K1, V = tgt.shape
    K = K1 - 1
    d_all = np.asarray(draft_tokens).reshape(B, K) if K > 0 else np.zeros((B, 0), np.int64)
    W = 0 if draft_rows is None else np.asarray(draft_rows).shape[1]
    lens = _lengths(draft_len, B, K)

    out = dict(
        accept_len=np.full(B, -1, np.int32), num_out=np.zeros(B, np.int32),
        out_tokens=np.full((B, K + 1), -1, np.int32),
        next_draft=np.full((B, W), -1, np.int32), next_len=np.zeros(B, np.int32),
        status=np.zeros(B, np.int32), verify_argmax=[], draft_argmax=[],
    )
    for b in range(B):
        n = lens[b]
        status = 0
        budget = _budget(len_budget, b)
        rows_read = n + 1
        if n < 0 or n > K:
            # No valid draft length: there are no verifier positions, so no
            # verifier row is read.
            status |= STATUS_BAD_INPUT
            n, rows_read = 0, 0
        if budget is not None and budget < 0:
            status |= STATUS_BAD_INPUT
        d = [int(t) for t in d_all[b, :n]]
        if any(t < 0 or t >= V for t in d):
            status |= STATUS_BAD_INPUT
        for i in range(rows_read):
            status |= row_status(tgt[b, i])
        for j in range(W):
            status |= row_status(draft_rows[b, j])
        out["status"][b] = status
        if status & STATUS_ERROR_MASK:
            out["verify_argmax"].append(None)
            out["draft_argmax"].append(None)
            continue

        v = [argmax_lowest(tgt[b, i]) for i in range(n + 1)]
        h = 0
        while h < n and d[h] == v[h]:
            h += 1
        C = d[:h] + [v[h]]
        a = stopping_index(C, h + 1, eos_id, budget)
        out["accept_len"][b] = h
        out["num_out"][b] = a
        out["out_tokens"][b, :a] = C[:a]
        z = [argmax_lowest(draft_rows[b, j]) for j in range(W)]
        keep = z[a:]
        out["next_draft"][b, :len(keep)] = keep
        out["next_len"][b] = max(0, W - a)
        out["verify_argmax"].append(v)
        out["draft_argmax"].append(z)
    return out


def _sampling_verify(tgt, drf, draft_tokens, draft_len, t_target, t_draft,
                     lam, u_accept, u_resample, eos_id, len_budget, delta=None):
    """Rejection-sampling verification of a chain; lam = 0 is lossless.
    With ``delta`` set, the modified Cactus rule (oracle.cactus) replaces
    the linear one: each drafted token's target is p~ with p~(d) = gamma.

    Packed-SS, Algorithm 2 (and Two Tradeoffs, Algorithm 1 for lam > 0):
      p_i = target distributions, i = 1..|D|+1
      alpha_i = min{1, p~_i(d_i) / q_i(d_i)} tested with u_i, i = 1..|D|
      h = max{h : u_i < alpha_i for all i <= h}
      c ~ [p~_{h+1} - q_{h+1}]_+ normalised   if h < |D|
      c ~ p_{|D|+1}                            if h = |D|   (the bonus uses
                                                  p, not p~)
      C = (d_1..d_h, c), then the ending condition.
    The draw uses u_resample[b, h] through ``inverse_cdf``.  A residual with
    zero mass (p~ = q in floating point) is never reached in exact
    arithmetic; it is read as a draw from p with the same uniform and
    flagged.
    """
    tgt = np.asarray(tgt)
    B, K1, V = tgt.shape
    K = K1 - 1
    drf = np.asarray(drf)
    d_all = np.asarray(draft_tokens).reshape(B, K) if K > 0 else np.zeros((B, 0), np.int64)
    ua = np.asarray(u_accept, np.float64).reshape(B, K) if K > 0 else np.zeros((B, 0))
    ur = np.asarray(u_resample, np.float64).reshape(B, K + 1)
    lens = _lengths(draft_len, B, K)

    out = dict(
        accept_len=np.full(B, -1, np.int32), num_out=np.zeros(B, np.int32),
        out_tokens=np.full((B, K + 1), -1, np.int32),
        status=np.zeros(B, np.int32),
        p_draft=np.zeros((B, K)), q_draft=np.zeros((B, K)), alpha=np.zeros((B, K)),
        gamma=np.zeros((B, K)),
        accept_bits=np.zeros((B, K), bool), accept_margin=np.full((B, K), np.inf),
        residual_mass=np.zeros(B), draw_margin=np.full(B, np.inf),
        draw_row=np.full(B, -1, np.int32), draw_kind=[None] * B,
    )
    for b in range(B):
        n = lens[b]
        status = 0
        budget = _budget(len_budget, b)
        rows_read = n + 1
        if n < 0 or n > K:
            # No valid draft length: no verifier or drafter row is read.
            status |= STATUS_BAD_INPUT
            n, rows_read = 0, 0
        if budget is not None and budget < 0:
            status |= STATUS_BAD_INPUT
        d = [int(t) for t in d_all[b, :n]]
        if any(t < 0 or t >= V for t in d):
            status |= STATUS_BAD_INPUT
        for i in range(rows_read):
            status |= row_status(tgt[b, i])
        for i in range(n):
            status |= row_status(drf[b, i])
        if status & STATUS_ERROR_MASK:
            out["status"][b] = status
            continue

        p = [tempered_softmax(tgt[b, i], t_target) for i in range(n + 1)]
        q = [tempered_softmax(drf[b, i], t_draft) for i in range(n)]
        for i in range(n):
            if delta is None:
                acc, alpha, margin, qz = acceptance_test(ua[b, i], p[i][d[i]], q[i][d[i]], lam)
                gamma = (1.0 - lam) * p[i][d[i]] + lam * q[i][d[i]]
            else:
                acc, alpha, margin, qz, gamma = cactus_acceptance(ua[b, i], p[i][d[i]], q[i][d[i]], delta)
            out["gamma"][b, i] = gamma
            out["p_draft"][b, i] = p[i][d[i]]
            out["q_draft"][b, i] = q[i][d[i]]
            out["alpha"][b, i] = alpha
            out["accept_bits"][b, i] = acc
            out["accept_margin"][b, i] = margin
            if qz:
                status |= STATUS_Q_ZERO
        h = 0
        while h < n and out["accept_bits"][b, h]:
            h += 1

        if h < n:
            if delta is None:
                r = residual_weights(p[h], q[h], lam)
            else:
                r = cactus_residual(p[h], q[h], d[h], out["gamma"][b, h])
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


def verify_rejection(tgt, drf, draft_tokens, draft_len, t_target, t_draft,
                     u_accept, u_resample, eos_id=-1, len_budget=None):
    """Lossless speculative-sampling verification (Packed-SS, Algorithm 2;
    Two Tradeoffs, Sec. 2 'Lossless Speculative Decoding')."""
    return _sampling_verify(tgt, drf, draft_tokens, draft_len, t_target,
                            t_draft, 0.0, u_accept, u_resample, eos_id,
                            len_budget)


def verify_lenient(tgt, drf, draft_tokens, draft_len, t_target, t_draft, lam,
                   u_accept, u_resample, eos_id=-1, len_budget=None):
    """Linear lenient verification, p~ = (1 - lam) p + lam q
    (Two Tradeoffs, Theorem 1 Eq. 5 and Algorithm 1)."""
    if not (0.0 <= lam <= 1.0):
        raise ValueError("lam must lie in [0, 1]")
    return _sampling_verify(tgt, drf, draft_tokens, draft_len, t_target,
                            t_draft, float(lam), u_accept, u_resample, eos_id,
                            len_budget)


def verify_cactus(tgt, drf, draft_tokens, draft_len, t_target, t_draft, delta,
                  u_accept, u_resample, eos_id=-1, len_budget=None):
    """Verification with the modified Cactus rule (Two Tradeoffs, App. E):
    gamma solves Phi(gamma) = delta exactly, accept with min{1, gamma/q(d)},
    correct from normalize([p~ - q]_+), bonus from p.  delta = 0 is the
    lossless rule."""
    if not (delta >= 0.0 and np.isfinite(delta)):
        raise ValueError("delta must be finite and >= 0")
    return _sampling_verify(tgt, drf, draft_tokens, draft_len, t_target,
                            t_draft, 0.0, u_accept, u_resample, eos_id,
                            len_budget, delta=float(delta))

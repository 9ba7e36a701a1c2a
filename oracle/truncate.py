"""Top-k / top-p truncation of a drafter distribution into stored sparse
form, in float64 (test infrastructure).

"One Call Ahead: Packed Self-Speculative Decoding with Diffusion Drafting",
Sec. 3.2: with top-k truncation (Fan et al.) or top-p truncation (Holtzman
et al.) only the nonzero entries of each stored drafter distribution Q need
to be kept; the page quotes top-k = 20 on a 151,936-token vocabulary and
top-p = 0.9.

For one logit row x at temperature T:
  q      = softmax(x / T)
  top-k  : the k tokens of largest q (equal values: the lower token id
           first); the rest get zero
  top-p  : within those, sorted by q descending (then by id), the shortest
           prefix whose mass is at least p of the top-k mass
  Q      = the kept q renormalised to sum 1
Entries are stored in that sorted order.

Readings (where the page is silent):
* Top-k is applied first and top-p to the renormalised top-k distribution
  (the order the cited samplers use together); top_p = 1 keeps all k.
* k must lie in [1, kmax]; p in (0, 1].
* A row that is not a distribution (NaN or +inf, or all -inf; the
  logit-row rule of the verifiers) is stored with q_nnz = -1, which the
  sparse verifier reports as bad input for any draft that uses it.
"""

import numpy as np

from .rows import row_status


def truncate_row(x, temperature, top_k, top_p):
    """Returns (idx, prob) of the kept tokens, sorted by probability
    descending then token id ascending."""
    x = np.asarray(x, np.float64)
    V = x.size
    k = min(int(top_k), V)
    a = x / float(temperature)
    q = np.exp(a - np.max(a))
    q /= q.sum()
    # q is increasing in x for T > 0: rank by the logits (no underflow ties)
    order = sorted(range(V), key=lambda v: (-x[v], v))[:k]
    mass = np.array([q[v] for v in order])
    mass = mass / mass.sum()
    keep = k
    if top_p < 1.0:
        run = 0.0
        for i in range(k):
            run += mass[i]
            if run >= top_p:
                keep = i + 1
                break
    kept = np.array(order[:keep], np.int64)
    prob = mass[:keep] / mass[:keep].sum()
    return kept, prob


def truncate_rows(rows, temperature, top_k, top_p, kmax, lengths=None):
    """Truncation of rows [B, K, V] into (q_idx [B, K, kmax], q_prob [B, K,
    kmax], q_nnz [B, K]); rows at i >= lengths[b] are not read (nnz 0)."""
    rows = np.asarray(rows)
    B, K, V = rows.shape
    if not (1 <= top_k <= kmax) or not (0.0 < top_p <= 1.0):
        raise ValueError("top_k must lie in [1, kmax] and top_p in (0, 1]")
    qi = np.zeros((B, K, kmax), np.int64)
    qp = np.zeros((B, K, kmax))
    qn = np.zeros((B, K), np.int64)
    for b in range(B):
        n = K if lengths is None else int(np.asarray(lengths)[b])
        for i in range(max(0, min(n, K))):
            if row_status(rows[b, i]):
                qn[b, i] = -1
                continue
            idx, prob = truncate_row(rows[b, i], temperature, top_k, top_p)
            qi[b, i, :idx.size] = idx
            qp[b, i, :idx.size] = prob
            qn[b, i] = idx.size
    return qi, qp, qn

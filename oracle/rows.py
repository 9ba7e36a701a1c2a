"""Per-row definitions of the verification step, in float64.

Test infrastructure: see the package docstring.  Each function states the
passage of the pages it writes out.
"""

import numpy as np

# Per-sequence status bits.  The first three are data errors: the sequence's
# outputs become sentinels.  The last two only annotate a decision that was
# still taken by the stated rule.
STATUS_BAD_INPUT = 1    # token / length / tree index out of range
STATUS_NONFINITE = 2    # a row that is read holds NaN or +inf
STATUS_EMPTY_ROW = 4    # a row that is read is entirely -inf (no mass)
STATUS_Q_ZERO = 8       # q(d) == 0 while p~(d) > 0 (accepted, flagged)
STATUS_Z_ZERO = 16      # residual mass is zero; draw fell back to p
STATUS_ERROR_MASK = STATUS_BAD_INPUT | STATUS_NONFINITE | STATUS_EMPTY_ROW

# A decision whose margin is below this is "near-margin": float32 and
# float64 evaluations may legitimately disagree on it.
NEAR_MARGIN = 1e-5


def row_status(x):
    """Status bits of one logit row that the verifier reads.

    ``-inf`` is a legal logit meaning zero probability (Packed-SS, Lemma B.3:
    neither distribution needs full support).  NaN and ``+inf`` are errors,
    and so is a row with no finite entry, which defines no distribution.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or np.isposinf(x).any():
        return STATUS_NONFINITE
    if np.isneginf(x).all():
        return STATUS_EMPTY_ROW
    return 0


def tempered_softmax(x, temperature):
    """Temperature-adjusted distribution of one logit row.

    SPOT, Sec. 4.1 Eq. 2: pi_T(v) = p(v)^(1/T) / sum_u p(u)^(1/T), which for
    logits z is softmax(z / T); T = 1 gives the model's own distribution
    (Packed-SS, Sec. 2.2).  Requires a row with ``row_status == 0``.
    """
    a = np.asarray(x, dtype=np.float64) / float(temperature)
    m = np.max(a)
    w = np.exp(a - m)
    return w / np.sum(w)


def max_probability(x):
    """Confidence of one masked position: max_v of the untempered softmax.

    SPOT, Sec. 4.1 / App. A.1 (position selection uses max_v p(v | x, C)).
    Equal to 1 / sum_v exp(z_v - max z).
    """
    z = np.asarray(x, dtype=np.float64)
    return 1.0 / np.sum(np.exp(z - np.max(z)))


def argmax_lowest(x):
    """Index of the largest entry; equal values resolve to the lowest index.

    Packed-SS, Sec. 3.1 Eq. 1 and Eq. 3 take argmax over the vocabulary, and
    App. B.2 ("Greedy decoding") fixes that each model puts its mass on the
    argmax "chosen by its fixed tie-breaking rule".  The rule fixed here is
    the lowest vocabulary index, applied to the raw logits.
    """
    x = np.asarray(x, dtype=np.float64)
    best = np.max(x)
    return int(np.flatnonzero(x == best)[0])


def acceptance_test(u, p_d, q_d, lam=0.0):
    """One rejection-sampling test of a drafted token d.

    Lossless (lam = 0): Packed-SS, Algorithm 2, acceptance tests --
    alpha = min{1, p(d) / Q(d)}, accepted when u < alpha.
    Lenient: Two Tradeoffs, Theorem 1 Eq. 5 replaces p by the interpolated
    target p~ = (1 - lam) p + lam q, chosen before d is drawn, and tests
    u against min{1, p~(d) / q(d)}.
    When q(d) == 0 (never for a token drawn from q, Lemma B.3) the ratio is
    read as +inf if p~(d) > 0 (accept) and 0 otherwise.

    Returns (accepted, alpha, margin, q_zero_flag).
    """
    pt_d = (1.0 - lam) * p_d + lam * q_d
    if q_d > 0.0:
        alpha = min(1.0, pt_d / q_d)
    else:
        alpha = 1.0 if pt_d > 0.0 else 0.0
    accepted = bool(u < alpha)
    q_zero = bool(q_d == 0.0 and pt_d > 0.0)
    return accepted, alpha, abs(u - alpha), q_zero


def inverse_cdf(w, u):
    """Draw an index from the non-negative weights w with the uniform u.

    Returns the smallest index c with F(c) > u * Z, where F is the running
    sum of w in vocabulary order and Z = F(last).  A zero-weight index is
    never returned.  The margin is the distance of u*Z to the nearer edge of
    c's interval, relative to Z.  Requires Z > 0.

    Returns (index, margin, Z).
    """
    w = np.asarray(w, dtype=np.float64)
    F = np.cumsum(w)
    Z = float(F[-1])
    t = u * Z
    hits = np.flatnonzero(F > t)
    if hits.size:
        c = int(hits[0])
    else:  # unreachable for u < 1; kept as the last positive weight
        c = int(np.flatnonzero(w > 0)[-1])
    lo = float(F[c - 1]) if c > 0 else 0.0
    margin = min(t - lo, float(F[c]) - t) / Z
    return c, margin, Z


def total_variation(p, q):
    """TV(p, q) = 1/2 sum_v |p(v) - q(v)| of two distributions on one
    vocabulary.  Two Tradeoffs, Sec. 2 (Eq. 1-2): the lossless verifier
    accepts a draft from q with probability 1 - TV(p, q), its diagnostic
    quantity per row."""
    return 0.5 * float(np.sum(np.abs(np.asarray(p, np.float64) - np.asarray(q, np.float64))))


def residual_weights(p, q, lam=0.0):
    """Unnormalised correction law [p~ - q]_+ at a rejected position.

    Packed-SS, Algorithm 2, correction draw (R proportional to [p - Q]_+);
    Two Tradeoffs, Algorithm 1 (Normalize([p~_k - q_k]_+) for k <= B).
    """
    pt = (1.0 - lam) * np.asarray(p, np.float64) + lam * np.asarray(q, np.float64)
    return np.maximum(pt - np.asarray(q, np.float64), 0.0)


def stopping_index(C, A, eos_id=-1, budget=None):
    """Number of emitted tokens kept after the ending condition.

    Packed-SS, Algorithm 1 / Algorithm 2, ending condition:
    a = min({A, remaining length} union {i <= A : C_i = EOS}) with 1-based
    i, after which C is pruned to its first a tokens.  ``eos_id < 0`` and
    ``budget is None`` disable the respective terms.
    """
    a = A
    if budget is not None:
        a = min(a, int(budget))
    if eos_id >= 0:
        for i in range(1, A + 1):
            if C[i - 1] == eos_id:
                a = min(a, i)
                break
    return a

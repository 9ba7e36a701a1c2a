"""The modified Cactus acceptance rule, in float64 (test infrastructure).

"Speculative Diffusion is a Tale of Two Tradeoffs", App. E (Modified
Cactus): for a drafted token y with verifier probability p = p(y) and
drafter probability q(y), the target is modified after y is seen.  The new
target p~ puts the largest mass gamma on y that keeps KL(p~ || p) <= delta,
and rescales every other token by (1 - gamma) / (1 - p), which keeps p~ a
distribution.  With that rescaling the KL is the Bernoulli divergence

    Phi(gamma) = gamma log(gamma / p) + (1 - gamma) log((1 - gamma) / (1 - p))

(App. E, Eq. 17).  The page solves Phi(gamma) = delta exactly (Newton's
method) rather than through the second-order Taylor form of Eq. 18.  Here
the root is found by bisection -- a different method, chosen so that the
checks do not share the GPU's iteration.  The draft is accepted with
probability min{1, gamma / q(y)}; a rejected position draws from
normalize([p~ - q]_+) as in any speculative sampler with target p~.

Readings (where App. E is silent):
* gamma is the largest value in [p, 1] with Phi(gamma) <= delta: gamma = 1
  when Phi(1) = -log p <= delta, gamma = p when delta = 0, gamma = 0 when
  p = 0 (Phi is +inf for any gamma > 0 then).
* The bonus after full acceptance is drawn from p, as for the linear rule
  (Two Tradeoffs, Algorithm 1).
"""

import math

import numpy as np


def cactus_divergence(gamma, p):
    """Phi(gamma) of App. E, Eq. 17, with 0 log 0 = 0."""
    def term(a, b):
        if a == 0.0:
            return 0.0
        if b == 0.0:
            return math.inf
        return a * math.log(a / b)
    return term(gamma, p) + term(1.0 - gamma, 1.0 - p)


def cactus_gamma(p, delta, iters=200):
    """Largest gamma in [p, 1] with Phi(gamma) <= delta, by bisection.

    Phi(p) = 0 and Phi is increasing on [p, 1] (its derivative
    log(gamma (1 - p) / (p (1 - gamma))) is positive there), so the feasible
    set is an interval [p, gamma*].
    """
    p = float(p)
    delta = float(delta)
    if delta < 0.0 or not math.isfinite(delta):
        raise ValueError("delta must be finite and >= 0")
    if p <= 0.0:
        return 0.0
    if p >= 1.0:
        return 1.0
    if delta == 0.0:
        return p
    if cactus_divergence(1.0, p) <= delta:
        return 1.0
    lo, hi = p, 1.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if cactus_divergence(mid, p) <= delta:
            lo = mid
        else:
            hi = mid
    return lo


def cactus_target(p, y, gamma):
    """The modified target p~ of App. E for drafted token y: p~(y) = gamma,
    p~(v) = (1 - gamma) / (1 - p(y)) p(v) otherwise."""
    p = np.asarray(p, np.float64)
    py = float(p[y])
    if py >= 1.0:
        pt = p.copy()
    else:
        pt = (1.0 - gamma) / (1.0 - py) * p
    pt[y] = gamma
    return pt


def cactus_acceptance(u, p_y, q_y, delta):
    """The Cactus test of one drafted token: gamma from the budget, accepted
    when u < alpha = min{1, gamma / q(y)}.  q(y) = 0 reads the ratio as +inf
    when gamma > 0 (accept, flagged) and 0 otherwise.

    Returns (accepted, alpha, margin, q_zero_flag, gamma).
    """
    gamma = cactus_gamma(p_y, delta)
    if q_y > 0.0:
        alpha = min(1.0, gamma / q_y)
    else:
        alpha = 1.0 if gamma > 0.0 else 0.0
    accepted = bool(u < alpha)
    return accepted, alpha, abs(u - alpha), bool(q_y == 0.0 and gamma > 0.0), gamma


def cactus_residual(p, q, y, gamma):
    """Unnormalised correction law [p~ - q]_+ at a rejected position."""
    return np.maximum(cactus_target(p, y, gamma) - np.asarray(q, np.float64), 0.0)

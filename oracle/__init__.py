"""Plain CPU oracle for draft-block verification (test infrastructure only).

This package is the slow, obviously-correct reference that the HIP path is
checked against.  It is NOT part of the product: only the test-suite, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code, constant tables or helpers
with the HIP library; both sides only consume the same seeded inputs.

Everything is computed in float64 with explicit per-row / per-sequence loops,
following the pages' definitions in their own order:

* ``rows``   -- per-row quantities: tempered softmax, lowest-index argmax,
  the acceptance test, inverse-CDF draws, the residual ``[p~ - q]_+``.
* ``chain``  -- per-sequence verification of a drafted chain: greedy match,
  lossless rejection, the linear lenient rule and the modified Cactus rule,
  with the stopping rule and next-draft retention.
* ``cactus`` -- the modified Cactus budget: gamma from the Bernoulli KL
  budget, the modified target p~ and its residual.
* ``anyorder`` -- one any-order greedy verification call (Packed-SS App. C,
  Algorithm 3): a chosen order over the active positions, missing drafts,
  the ending position and retention by position.
* ``tree``   -- coupled shared-Gumbel state-equality verification of a draft
  tree (and its T=0 greedy special case).
* ``sparse`` -- lossless verification against a stored sparse (top-k /
  top-p) drafter distribution.
* ``truncate`` -- top-k / top-p truncation of drafter rows into that stored
  sparse form.
* ``spot``   -- chain verification on the joint (position, token) space:
  rejection sampling per link (SPOT App. B) and the confidence-gated hybrid
  of coupled-noise match and rejection sampling.
* ``loop``   -- multi-iteration Packed-SS decoding with greedy verification
  (Packed-SS Sec. 3.1, Algorithm 1) over a model given as a function.
* ``ddtree`` -- prefix-conditional draft-tree construction: token hypotheses
  from the stale conditionals, prefix masses and the top-D tree (SPOT
  Sec. 4.2 Eq. 3, App. C.2 Algorithm 2).

Sources (pages by title):
* "One Call Ahead: Packed Self-Speculative Decoding with Diffusion Drafting"
  (Packed-SS): Sec. 2.2, Sec. 3.1 Eq. 1-4 and Algorithm 1, Sec. 3.2,
  Sec. 3.2 (stored sparse Q), App. B.2 Algorithm 2 and Lemma B.3, App. C
  Algorithm 3 and Prop. C.1,
  App. D.1.
* "On the SPOT: Enhancing Speculative Decoding for Diffusion Language Models
  via Commit-Order Prediction" (SPOT): Sec. 4.1, Sec. 4.2 Eq. 3, Sec. 4.3
  Eq. 4, App. A.1, A.3 Eq. 5-7, App. B Eq. 10-14, App. C.2 Algorithm 2.
* "Speculative Diffusion is a Tale of Two Tradeoffs" (Two Tradeoffs): Sec. 2
  Eq. 1-5 and Theorem 1, Sec. 3.2 Algorithm 1, App. C Proposition 1,
  App. E (modified Cactus, Eq. 17-18).
"""

from .rows import (  # noqa: F401
    STATUS_BAD_INPUT, STATUS_NONFINITE, STATUS_EMPTY_ROW, STATUS_Q_ZERO,
    STATUS_Z_ZERO, STATUS_ERROR_MASK, NEAR_MARGIN,
    row_status, tempered_softmax, argmax_lowest, acceptance_test,
    inverse_cdf, residual_weights, stopping_index, total_variation,
)
from .chain import verify_greedy, verify_rejection, verify_lenient, verify_cactus  # noqa: F401
from .cactus import (  # noqa: F401
    cactus_divergence, cactus_gamma, cactus_target, cactus_acceptance, cactus_residual,
)
from .anyorder import NO_END, verify_greedy_any_order  # noqa: F401
from .sparse import dense_q, verify_sparse  # noqa: F401
from .truncate import truncate_row, truncate_rows  # noqa: F401
from .spot import MODE_RS, MODE_MATCH, rs_link, rs_residual, verify_spot_chain  # noqa: F401
from .tree import (  # noqa: F401
    TREE_STATE_EQUALITY, TREE_FIXED_POSITION, state_transition, walk,
    verify_gumbel_tree,
)
from .ddtree import (  # noqa: F401
    RUNNER_UP_BELOW, hypotheses, order_distribution, table_order, best_first,
    level_batched, tree_arrays, build_ddtree,
)
from .loop import packed_ss_greedy  # noqa: F401

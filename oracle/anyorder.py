"""Any-order greedy verification of one Packed-SS call, in float64 (test
infrastructure).

"One Call Ahead: Packed Self-Speculative Decoding with Diffusion Drafting",
App. C (Any-Order Extension), Algorithm 3, the verification part of one
iteration t.  Per sequence the call sees the u unresolved
output positions of its active window, in textual order ("slots"
j = 0..u-1, output positions pos[j]), an order pi over them chosen before
the call (order[r] = the slot checked at rank r), the available draft tokens
(by slot; -1 where a position has no draft yet), the verifier rows in rank
order (row r is the verifier at pi(r) given the drafts at earlier ranks,
Eq. 8) and the drafter rows by slot.

  kappa = leading ranks whose position has a draft
  v_r   = argmax of verifier row r, r < min(kappa + 1, u)   (Eq. 8)
  z_j   = argmax of drafter row j, j < u
  h     = leading ranks r < kappa with d(pi(r)) = v_r
  A     = min(h + 1, u);  C = ((pos[pi(r)], v_r))_{r < A}
  E'    = min({E} U {position of an EOS in C})
  C'    = the pairs of C at positions <= E'
  next draft: z_j for the slots j not in C with pos[j] <= E'

Readings (where the page is silent):
* The verifier rows arrive in rank order (the order in which the packed call
  feeds the positions); rows at ranks >= min(kappa + 1, u) are not read.
* A draft token of -1 marks a missing draft; any other value outside
  [0, V) is bad input, as are an order that is not a permutation of
  0..u-1 and slot positions that do not increase.
* Argmax ties go to the lowest index (Packed-SS App. B.2, fixed rule).
"""

import numpy as np

from .rows import STATUS_BAD_INPUT, STATUS_ERROR_MASK, argmax_lowest, row_status

# The last position to generate when no end is given (E = L unbounded).
NO_END = 2 ** 31 - 1


def verify_greedy_any_order(tgt, order, num_active, positions, draft_tokens,
                            draft_rows=None, eos_id=-1, end_pos=None):
    """One any-order greedy verification call for B sequences.

    tgt [B, U, V] verifier rows by rank; order [B, U]; num_active [B] or
    None (= U); positions [B, U] or None (slot j at position j);
    draft_tokens [B, U] by slot (-1 = missing); draft_rows [B, U, V] by slot
    or None; eos_id (-1 disables); end_pos [B] or None (no limit, NO_END).
    Returns accept_len (h), kappa, num_accepted (|C'|), acc_pos / acc_tok
    (C' in rank order, -1 after), new_end (E'), next_draft (by slot, -1 where
    no draft is kept) and status.
    """
    tgt = np.asarray(tgt)
    B, U, V = tgt.shape
    order = np.asarray(order).reshape(B, U)
    drafts = np.asarray(draft_tokens).reshape(B, U)
    out = dict(
        accept_len=np.full(B, -1, np.int32), kappa=np.zeros(B, np.int32),
        num_accepted=np.zeros(B, np.int32),
        acc_pos=np.full((B, U), -1, np.int32), acc_tok=np.full((B, U), -1, np.int32),
        new_end=np.zeros(B, np.int64), next_draft=np.full((B, U), -1, np.int32),
        status=np.zeros(B, np.int32),
    )
    for b in range(B):
        u = U if num_active is None else int(np.asarray(num_active)[b])
        E = NO_END if end_pos is None else int(np.asarray(end_pos)[b])
        out["new_end"][b] = E
        status = 0
        if u < 0 or u > U:
            out["status"][b] = STATUS_BAD_INPUT
            continue
        pos = list(range(u)) if positions is None else [int(v) for v in np.asarray(positions)[b, :u]]
        pi = [int(v) for v in order[b, :u]]
        d = [int(v) for v in drafts[b, :u]]
        if sorted(pi) != list(range(u)):
            status |= STATUS_BAD_INPUT
        if any(pos[j] >= pos[j + 1] for j in range(u - 1)):
            status |= STATUS_BAD_INPUT
        if any(t < -1 or t >= V for t in d):
            status |= STATUS_BAD_INPUT
        if status:
            out["status"][b] = status
            continue
        kappa = 0
        while kappa < u and d[pi[kappa]] >= 0:
            kappa += 1
        nver = min(kappa + 1, u)
        for r in range(nver):
            status |= row_status(tgt[b, r])
        W = 0 if draft_rows is None else u
        for j in range(W):
            status |= row_status(draft_rows[b, j])
        out["kappa"][b] = kappa
        out["status"][b] = status
        if status & STATUS_ERROR_MASK:
            continue
        v = [argmax_lowest(tgt[b, r]) for r in range(nver)]
        h = 0
        while h < kappa and d[pi[h]] == v[h]:
            h += 1
        A = min(h + 1, u)
        C = [(pos[pi[r]], v[r]) for r in range(A)]
        if eos_id >= 0:
            for p_, t_ in C:
                if t_ == eos_id:
                    E = min(E, p_)
        kept = [(p_, t_) for p_, t_ in C if p_ <= E]
        out["accept_len"][b] = h
        out["num_accepted"][b] = len(kept)
        for k, (p_, t_) in enumerate(kept):
            out["acc_pos"][b, k] = p_
            out["acc_tok"][b, k] = t_
        out["new_end"][b] = E
        if draft_rows is not None:
            accepted = {pi[r] for r in range(A)}
            for j in range(u):
                if j not in accepted and pos[j] <= E:
                    out["next_draft"][b, j] = argmax_lowest(draft_rows[b, j])
    return out

"""Multi-iteration Packed-SS decoding with left-to-right greedy verification
(test infrastructure).

"One Call Ahead: Packed Self-Speculative Decoding with Diffusion Drafting",
Sec. 3.1 and Algorithm 1: start from the prompt with an empty draft; call t
evaluates, in one model call, the verifier rows of the previous draft plus
one (Eq. 1) and W draft rows conditioned on the previous prefix (Eq. 3);
h_t leading matches (Eq. 2), A_t = h_t + 1 tokens accepted, cut at the first
accepted EOS or at L new tokens; the draft rows after the first A_t become
the next draft (Eq. 4).

The model is an input: model(plen, d, n, t) returns the packed rows of call
t, [B, 2W, V] -- verify rows 0..W-1 (row r: the token after the prefix and r
draft tokens), then draft rows W..2W-1 -- for prefix lengths plen [B],
drafts d [B, W-1] (-1 past n) and draft lengths n [B].

Readings (where the page is silent):
* A draft holds at most W - 1 tokens (W - A_t with A_t >= 1), so a call
  verifies at most W - 1 draft tokens and reads W verify rows.
* A sequence that has stopped (EOS accepted or L tokens) stays in the batch
  with an empty draft and a length budget of 0, so it accepts nothing.
"""

import numpy as np

from .chain import verify_greedy


def packed_ss_greedy(model, B, W, L, calls, eos_id=-1):
    """Runs up to `calls` model calls.  Returns (tokens: list of B lists,
    per_call: list of dicts with num_out [B], accept_len [B], draft_len [B])."""
    plen = np.zeros(B, np.int64)
    d = np.full((B, W - 1), -1, np.int64)
    n = np.zeros(B, np.int64)
    done = np.zeros(B, bool)
    tokens = [[] for _ in range(B)]
    per_call = []
    for t in range(calls):
        if done.all():
            break
        packed = np.asarray(model(plen.copy(), d.copy(), n.copy(), t))
        budget = np.where(done, 0, L - plen)
        o = verify_greedy(packed[:, :W], d, n, packed[:, W:], eos_id, budget)
        per_call.append(dict(num_out=o["num_out"].copy(), accept_len=o["accept_len"].copy(),
                             draft_len=n.copy(), status=o["status"].copy()))
        for b in range(B):
            if done[b]:
                continue
            a = int(o["num_out"][b])
            out = [int(v) for v in o["out_tokens"][b, :a]]
            tokens[b].extend(out)
            plen[b] += a
            if (eos_id >= 0 and eos_id in out) or plen[b] >= L:
                done[b] = True
            d[b] = -1
            if done[b]:
                n[b] = 0
                continue
            nl = int(o["next_len"][b])
            d[b, :nl] = o["next_draft"][b, :nl]
            n[b] = nl
    return tokens, per_call

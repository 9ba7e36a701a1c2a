"""Multi-iteration Packed-SS decoding with greedy verification on the GPU
("One Call Ahead: Packed Self-Speculative Decoding with Diffusion Drafting",
Sec. 3.1 and Algorithm 1).

One verify_greedy call per model call verifies the previous draft and keeps
the next one; between calls only device-side bookkeeping happens here
(appending the committed tokens, the next draft and its length, the stop
flags), in torch tensors on the model's device, with no host round trip.
"""

import torch

from . import verify_greedy


def packed_ss_greedy_loop(model, B, W, L, calls, device, eos_id=-1, stop_when_done=True):
    """Runs up to `calls` model calls of batch B with speculative width W
    and L new tokens per sequence.

    model(plen, d, n, t) -> packed rows [B, 2W, V] on `device`: verify rows
    0..W-1 (row r: the token after the prefix and r draft tokens), then the
    W draft rows, for prefix lengths plen [B], drafts d [B, W-1] (-1 past n)
    and draft lengths n [B] (int32 device tensors).  A stopped sequence (an
    accepted EOS or L tokens) keeps an empty draft and a zero length budget.

    Returns dict(tokens [B, L] int32 (-1 past a sequence's length), length
    [B], num_out / accept_len / draft_len / status [calls run, B], calls).
    With stop_when_done the loop checks after each call whether every
    sequence has stopped (one host synchronisation per call)."""
    i32 = torch.int32
    plen = torch.zeros(B, dtype=i32, device=device)
    d = torch.full((B, W - 1), -1, dtype=i32, device=device)
    n = torch.zeros(B, dtype=i32, device=device)
    done = torch.zeros(B, dtype=torch.bool, device=device)
    dump = L + W                                   # column for masked-out writes
    tokens = torch.full((B, L + W + 1), -1, dtype=i32, device=device)
    j = torch.arange(W, device=device)
    recs = {"num_out": [], "accept_len": [], "draft_len": [], "status": []}
    t = 0
    for t in range(calls):
        if stop_when_done and bool(done.all()):
            break
        packed = model(plen, d, n, t)
        budget = torch.where(done, torch.zeros_like(plen), L - plen)
        r = verify_greedy(packed[:, :W], d, n, packed[:, W:], eos_id=eos_id, len_budget=budget)
        a = r["num_out"]
        keep = j[None, :] < a[:, None]
        idx = torch.where(keep, plen[:, None] + j[None, :], torch.full_like(keep, dump, dtype=i32))
        tokens.scatter_(1, idx.long(), r["out_tokens"][:, :W])
        recs["num_out"].append(a)
        recs["accept_len"].append(r["accept_len"])
        recs["draft_len"].append(n.clone())
        recs["status"].append(r["status"])
        plen = plen + a
        hit = ((r["out_tokens"][:, :W] == eos_id) & keep).any(dim=1) if eos_id >= 0 else torch.zeros_like(done)
        done = done | hit | (plen >= L)
        n = torch.where(done, torch.zeros_like(n), r["next_len"])
        d = torch.where(j[None, :W - 1] < n[:, None], r["next_draft"][:, :W - 1], torch.full_like(d, -1))
    out = {k: (torch.stack(v) if v else torch.zeros((0, B), dtype=i32, device=device)) for k, v in recs.items()}
    out["tokens"] = tokens[:, :L]
    out["length"] = plen
    out["calls"] = len(recs["num_out"])
    return out

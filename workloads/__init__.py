"""Seeded synthetic inputs for draft-block verification.

Shared by the tests, the smoke check and the benchmark.  This module holds no
verification arithmetic: it only draws logits, uniforms, Gumbel noise, draft
tokens and draft trees with torch's own random and sampling routines (the
draft tokens stand in for a drafter's sampling, done with torch.multinomial /
torch.argmax), so that the HIP path and the CPU oracle receive identical
inputs.

Seeds: base S0; stream j of configuration c uses S0 + 1000*c + j with
  j = 0 target logits, 1 peak positions, 2 draft noise, 3 draft-sampling
  uniforms, 4 accept uniforms, 5 resample uniforms, 6 Gumbel, 7 tree,
  8 draft lengths / root masks.
"""

import math

import torch

S0 = 20261202


def _gen(c, j, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(S0 + 1000 * c + j)
    return g


def _planted_logits(c, shape, peak, dtype, device="cpu"):
    """z ~ N(0, 3^2) with +peak added at one seeded token per row."""
    *lead, V = shape
    z = torch.randn(*shape, generator=_gen(c, 0, device), device=device) * 3.0
    if peak:
        pos = torch.randint(0, V, (*lead, 1), generator=_gen(c, 1, device), device=device)
        z.scatter_add_(-1, pos, torch.full((*lead, 1), float(peak), device=device))
    return z.to(dtype)


def chain_inputs(c, B, K, V, dtype=torch.bfloat16, sigma=1.0, temperature=1.0,
                 peak=6.0, random_lengths=False, device="cpu"):
    """Target rows [B, K+1, V], draft rows [B, K, V] = target + N(0, sigma^2)
    (rounded to dtype), draft tokens sampled from softmax(draft / T), accept
    and resample uniforms, and draft lengths."""
    tgt = _planted_logits(c, (B, K + 1, V), peak, dtype, device)
    noise = torch.randn(B, K, V, generator=_gen(c, 2, device), device=device) * sigma
    drf = (tgt[:, :K].float() + noise).to(dtype)
    if K > 0:
        probs = torch.softmax(drf.float().reshape(B * K, V) / temperature, dim=-1)
        d = torch.multinomial(probs, 1, generator=_gen(c, 3, device)).reshape(B, K)
    else:
        d = torch.zeros(B, 0, dtype=torch.int64, device=device)
    u_acc = torch.rand(B, K, generator=_gen(c, 4, device), device=device)
    u_res = torch.rand(B, K + 1, generator=_gen(c, 5, device), device=device)
    if random_lengths:
        n = torch.randint(0, K + 1, (B,), generator=_gen(c, 8, device), device=device)
    else:
        n = torch.full((B,), K, dtype=torch.int64, device=device)
    return dict(tgt=tgt, drf=drf, draft_tokens=d.to(torch.int32), u_accept=u_acc,
                u_resample=u_res, draft_len=n.to(torch.int32), temperature=temperature)


# ------------------------------------------------------------------ configs --

def config1(device="cpu"):
    """Tiny rejection verify: B=1, K=4, V=1024, fp32, z ~ N(0,3^2) + 6 peak,
    draft = z + N(0,1), T=1; greedy variant drafts argmax(draft)."""
    x = chain_inputs(1, 1, 4, 1024, torch.float32, sigma=1.0, device=device)
    x["greedy_tokens"] = torch.argmax(x["drf"].float(), dim=-1).to(torch.int32)
    return x


def config2(device="cpu"):
    """Batch lossless verify: B=8, K=8, V=32000 bf16, draft noise 0.5, T=1."""
    return chain_inputs(2, 8, 8, 32000, torch.bfloat16, sigma=0.5, device=device)


C3_SIGMAS = (0.25, 1.0, 2.0)
C3_TEMPS = (0.7, 1.0)
C3_LAMBDAS = (1.0, 0.5, 0.25)


def config3(sigma, temperature, device="cpu"):
    """Lenient sweep setting: B=32, K=16, V=128256 bf16, draft noise sigma,
    temperature T; the uniforms are common to every lambda."""
    return chain_inputs(3, 32, 16, 128256, torch.bfloat16, sigma=sigma,
                        temperature=temperature, device=device)


def config5(device="cpu", B=64, K=32, V=131072):
    """Packed greedy verify + draft: T[B, 2K, V] bf16; rows 0..K-1 are the
    verifier rows (z ~ N(0,3^2) + peak), rows K..2K-1 the drafter rows
    bf16(z + N(0,1)); K-1 drafts at most per sequence (the last verifier row
    is the bonus row), n_b ~ U{0..K-1}; drafts d_i = argmax(z_i + N(0,1))
    with independent noise (a stale previous draft)."""
    c = 5
    z = _planted_logits(c, (B, K, V), 6.0, torch.float32, device)
    packed = torch.empty(B, 2 * K, V, dtype=torch.bfloat16, device=device)
    packed[:, :K] = z.to(torch.bfloat16)
    zb = packed[:, :K].float()
    packed[:, K:] = (zb + torch.randn(B, K, V, generator=_gen(c, 2, device), device=device)).to(torch.bfloat16)
    stale = zb[:, :K - 1] + torch.randn(B, K - 1, V, generator=_gen(c, 3, device), device=device)
    d = torch.argmax(stale, dim=-1).to(torch.int32)
    n = torch.randint(0, K, (B,), generator=_gen(c, 8, device), device=device).to(torch.int32)
    return dict(packed=packed, tgt=packed[:, :K], draft_rows=packed[:, K:], draft_tokens=d,
                draft_len=n, K=K - 1, W=K)


# --------------------------------------------------------------------- tree --

def gumbel_noise(shape, generator, device="cpu"):
    """Gumbel(0,1) = -log(-log U) with U clamped to [2^-24, 1 - 2^-24]."""
    u = torch.rand(*shape, generator=generator, device=device)
    u = u.clamp(2.0 ** -24, 1.0 - 2.0 ** -24)
    return -torch.log(-torch.log(u))


def tree_inputs(c, B, S, L, V, dtype=torch.bfloat16, sigma_node=0.1, temperature=1.0,
                max_depth=8, device="cpu", runner_up_below=0.6, order_temp=0.5):
    """Draft trees grown by seeded prefix-mass sampling from root statistics.

    Per sequence: c0 ~ U{0..L/2-1} committed positions at the root; root
    logits Z0 [L, V] ~ N(0, 3^2); Gumbel table G [L, V].  Stand-in drafter:
    position order q(s|y) = softmax over masked s of log conf0(s) / order_temp
    with conf0 the root's max probability; token hypotheses = the coupled
    stale draw argmax(Z0[s]/T + G[s]) plus the runner-up when conf0(s) <
    runner_up_below; prefix mass m(z) = m(y) q(s|y) p0_s(v).  Nodes are added
    by sampling candidates proportional to m without replacement (depth <=
    max_depth, no duplicate children) until S nodes exist.  Node logits are
    bf16(Z0 + sigma_node * sqrt(depth) * N(0,1)).
    """
    gt = _gen(c, 7, "cpu")
    gm = _gen(c, 8, "cpu")
    g0 = _gen(c, 0, device)
    gG = _gen(c, 6, device)
    gn = _gen(c, 2, device)
    logits = torch.empty(B, S, L, V, dtype=dtype, device=device)
    gumbel = torch.empty(B, L, V, dtype=torch.float32, device=device)
    masked = torch.zeros(B, S, L, dtype=torch.bool)
    parent = torch.full((B, S), -1, dtype=torch.int32)
    epos = torch.zeros(B, S, dtype=torch.int32)
    etok = torch.zeros(B, S, dtype=torch.int32)
    depth = torch.zeros(B, S, dtype=torch.int32)
    num_states = torch.zeros(B, dtype=torch.int32)
    for b in range(B):
        z0 = (torch.randn(L, V, generator=g0, device=device) * 3.0).to(dtype)
        G = gumbel_noise((L, V), gG, device)
        gumbel[b] = G
        zf = z0.float()
        p0 = torch.softmax(zf / temperature if temperature > 0 else zf, dim=-1)
        conf0 = torch.softmax(zf, dim=-1).max(dim=-1).values.cpu().double()
        score = zf / temperature + G if temperature > 0 else zf
        top2 = torch.topk(score, 2, dim=-1).indices.cpu()
        ptop = torch.gather(p0, 1, top2.to(p0.device)).cpu().double()
        n0 = int(torch.randint(0, L // 2, (1,), generator=gm))
        committed = torch.randperm(L, generator=gm)[:n0]
        root_mask = torch.ones(L, dtype=torch.bool)
        root_mask[committed] = False

        states = [root_mask.clone()]
        mass = [1.0]
        nd = [0]
        kids = [set()]
        cand = {}

        def add_candidates(y):
            m = states[y]
            pos = torch.nonzero(m).flatten().tolist()
            if not pos or nd[y] >= max_depth:
                return
            w = torch.tensor([math.log(conf0[s]) / order_temp for s in pos], dtype=torch.float64)
            qpos = torch.softmax(w, dim=0).tolist()
            for s, qs in zip(pos, qpos):
                toks = [int(top2[s, 0])]
                ps = [float(ptop[s, 0])]
                if conf0[s] < runner_up_below:
                    toks.append(int(top2[s, 1]))
                    ps.append(float(ptop[s, 1]))
                for v, pv in zip(toks, ps):
                    cand[(y, s, v)] = mass[y] * qs * pv

        add_candidates(0)
        while len(states) < S and cand:
            keys = list(cand.keys())
            w = torch.tensor([cand[k] for k in keys], dtype=torch.float64)
            w = w / w.sum()
            k = keys[int(torch.multinomial(w, 1, generator=gt))]
            mz = cand.pop(k)
            y, s, v = k
            if (s, v) in kids[y]:
                continue
            kids[y].add((s, v))
            z = len(states)
            st = states[y].clone()
            st[s] = False
            states.append(st)
            mass.append(mz)
            nd.append(nd[y] + 1)
            kids.append(set())
            parent[b, z] = y
            epos[b, z] = s
            etok[b, z] = v
            add_candidates(z)
        ns = len(states)
        num_states[b] = ns
        # Unused slots (z >= num_states) are ignored by the verifier.
        for z in range(ns, S):
            states.append(root_mask.clone())
            nd.append(0)
            parent[b, z] = 0
        for z in range(S):
            masked[b, z] = states[z]
            depth[b, z] = nd[z]
        # node logits
        for z in range(S):
            if z == 0:
                logits[b, 0] = z0
            else:
                eps = torch.randn(L, V, generator=gn, device=device)
                logits[b, z] = (zf + sigma_node * math.sqrt(float(nd[z])) * eps).to(dtype)
    return dict(logits=logits, gumbel=gumbel, masked=masked, parent=parent, edge_pos=epos,
                edge_tok=etok, depth=depth, num_states=num_states, temperature=temperature)


def config4(device="cpu", sigma_node=0.1, B=16, S=64, L=32, V=151936):
    """Coupled-Gumbel tree verify: B=16 trees of S=64 states, block L=32,
    V=151936 bf16, T=1."""
    return tree_inputs(4, B, S, L, V, torch.bfloat16, sigma_node=sigma_node,
                       temperature=1.0, device=device)


# -------------------------------------------------------------- any-order --

def anyorder_inputs(c, B, U, V, dtype=torch.bfloat16, missing=0.1, agree=0.85, device="cpu",
                    with_draft_rows=True, full=False):
    """One any-order greedy verification call per sequence.

    u_b ~ U{1..U} unresolved slots (all U when ``full``) at increasing output
    positions; the order is a seeded permutation of the slots (standing in
    for a confidence order chosen before the call); verifier rows by rank are
    z ~ N(0, 3^2) with a +6 planted peak; the draft at the slot of rank r is
    the verifier's argmax with probability ``agree`` and a uniform token
    otherwise, and is missing (-1) with probability ``missing``; drafter rows
    by slot are dtype(z + N(0, 1)) of the slot's own verifier row.
    """
    tgt = _planted_logits(c, (B, U, V), 6.0, dtype, device)
    g3 = _gen(c, 3, "cpu")
    g8 = _gen(c, 8, "cpu")
    best = torch.argmax(tgt.float(), dim=-1).cpu()     # by rank
    if full:
        u = torch.full((B,), U, dtype=torch.int32)
    else:
        u = torch.randint(1, U + 1, (B,), generator=g8).to(torch.int32)
    order = torch.zeros(B, U, dtype=torch.int32)
    drafts = torch.full((B, U), -1, dtype=torch.int32)
    positions = torch.zeros(B, U, dtype=torch.int32)
    for b in range(B):
        n = int(u[b])
        perm = torch.randperm(n, generator=g3)
        order[b, :n] = perm.to(torch.int32)
        order[b, n:] = torch.arange(n, U, dtype=torch.int32)
        start = int(torch.randint(1, 1000, (1,), generator=g8))
        gaps = torch.randint(1, 3, (U,), generator=g8)
        positions[b] = (start + torch.cumsum(gaps, 0)).to(torch.int32)
        coin = torch.rand(n, generator=g3)
        other = torch.randint(0, V, (n,), generator=g3)
        for r in range(n):
            if coin[r] < missing:
                continue
            drafts[b, int(perm[r])] = int(best[b, r]) if coin[r] < missing + (1 - missing) * agree else int(other[r])
    out = dict(tgt=tgt, order=order, draft_tokens=drafts, num_active=u, positions=positions)
    if with_draft_rows:
        dr = (tgt.float() + torch.randn(B, U, V, generator=_gen(c, 5, device), device=device)).to(dtype)
        out["draft_rows"] = dr
    return out


def config5_any_order(device="cpu"):
    """Any-order packed greedy verify: B=64 sequences, window U=32 slots,
    V=131072 bf16, verifier rows by rank plus drafter rows by slot."""
    return anyorder_inputs(6, 64, 32, 131072, torch.bfloat16, device=device)


# ------------------------------------------------------- joint-space chain --

def spot_chain_inputs(c, B, K, V, dtype=torch.bfloat16, sigma=1.0, temperature=1.0, on_star=0.85,
                      gumbel=True, L=32, random_lengths=False, peak=20.0, device="cpu"):
    """A drafted chain of K links per sequence on the joint (position, token)
    space, with the target's rows at each link's position.

    Target rows [B, K+1, V]: z ~ N(0, 3^2) + ``peak`` at one token (the
    default makes the target's argmax carry most of the mass, as the pages
    report for T <= 1).  Drafter rows at the same positions:
    (z + N(0, sigma^2)) * m, the sharpness m in {0.5, 1, 1.5} per link (so
    the drafter's confidence falls on both sides of typical gate
    thresholds).  pos_star ~ U{0..L-1}; the proposal sits on pos_star with
    probability ``on_star`` (else on the next position mod L); q_pos_star ~
    U(0.3, 1); the proposed token is the drafter's Gumbel argmax under the
    link's shared noise row (a coupled drafter), noise rows Gumbel(0, 1)
    float32 [B, K+1, V] (None without ``gumbel``, then the proposal is a
    draw from the drafter's softmax).
    """
    tgt = _planted_logits(c, (B, K + 1, V), peak, dtype, device)
    noise = torch.randn(B, K, V, generator=_gen(c, 2, device), device=device) * sigma
    m = torch.tensor([0.5, 1.0, 1.5], device=device)[
        torch.randint(0, 3, (B, K, 1), generator=_gen(c, 6, device), device=device)]
    drf = ((tgt[:, :K].float() + noise) * m).to(dtype)
    g8 = _gen(c, 8, "cpu")
    pos_star = torch.randint(0, L, (B, K + 1), generator=g8).to(torch.int32)
    off = torch.rand(B, K, generator=g8) >= on_star
    prop_pos = torch.where(off, (pos_star[:, :K] + 1) % L, pos_star[:, :K]).to(torch.int32)
    q_pos = 0.3 + 0.7 * torch.rand(B, K, generator=g8)
    G = gumbel_noise((B, K + 1, V), _gen(c, 9, device), device) if gumbel else None
    if K > 0 and G is not None:
        d = torch.argmax(drf.float() / temperature + G[:, :K], dim=-1)
    elif K > 0:
        probs = torch.softmax(drf.float().reshape(B * K, V) / temperature, dim=-1)
        d = torch.multinomial(probs, 1, generator=_gen(c, 3, device)).reshape(B, K)
    else:
        d = torch.zeros(B, 0, dtype=torch.int64, device=device)
    u_acc = torch.rand(B, K, generator=_gen(c, 4, device), device=device)
    u_res = torch.rand(B, K + 1, generator=_gen(c, 5, device), device=device)
    if random_lengths:
        n = torch.randint(0, K + 1, (B,), generator=g8)
    else:
        n = torch.full((B,), K, dtype=torch.int64)
    return dict(tgt=tgt, drf=drf, pos_star=pos_star, prop_pos=prop_pos, prop_tok=d.to(torch.int32).cpu(),
                q_pos_star=q_pos, gumbel=G, u_accept=u_acc, u_resample=u_res, draft_len=n.to(torch.int32),
                temperature=temperature)


def config4_spot_chain(device="cpu"):
    """Joint-space chain, hybrid gate: B=16 sequences, K=8 links, V=151936
    bf16, sigma=1, T=1, Gumbel rows for every target row."""
    return spot_chain_inputs(41, 16, 8, 151936, torch.bfloat16, device=device)


# ------------------------------------------------------------- sparse Q --

def sparse_inputs(c, B, K, V, dtype=torch.bfloat16, topk=20, sigma=1.0, temperature=1.0,
                  random_lengths=False, kmax=None, peak=6.0, device="cpu"):
    """A drafted chain whose drafter distributions are stored sparse: each
    draft row keeps the ``topk`` most likely tokens of softmax(drafter / T),
    renormalised (top-k truncation), as (token, probability) entries sorted
    by probability; the draft token is drawn from that truncated Q with a
    seeded uniform.  Target rows [B, K+1, V]: z ~ N(0, 3^2) + ``peak`` at one
    token; the drafter logits z + N(0, sigma^2) are not passed on.
    """
    kmax = topk if kmax is None else kmax
    tgt = _planted_logits(c, (B, K + 1, V), peak, dtype, device)
    drf = (tgt[:, :K].float() + torch.randn(B, K, V, generator=_gen(c, 2, device), device=device) * sigma)
    probs = torch.softmax(drf / temperature, dim=-1)
    top = torch.topk(probs, topk, dim=-1)
    qp = top.values / top.values.sum(dim=-1, keepdim=True)
    u = torch.rand(B, K, 1, generator=_gen(c, 3, device), device=device)
    pick = (torch.cumsum(qp, dim=-1) <= u * qp.sum(dim=-1, keepdim=True)).sum(dim=-1).clamp(max=topk - 1)
    d = torch.gather(top.indices, -1, pick.unsqueeze(-1)).squeeze(-1)
    q_idx = torch.zeros(B, K, kmax, dtype=torch.int32)
    q_prob = torch.zeros(B, K, kmax, dtype=torch.float32)
    q_idx[:, :, :topk] = top.indices.to(torch.int32).cpu()
    q_prob[:, :, :topk] = qp.float().cpu()
    q_nnz = torch.full((B, K), topk, dtype=torch.int32)
    u_acc = torch.rand(B, K, generator=_gen(c, 4, device), device=device)
    u_res = torch.rand(B, K + 1, generator=_gen(c, 5, device), device=device)
    if random_lengths:
        n = torch.randint(0, K + 1, (B,), generator=_gen(c, 8, "cpu"))
    else:
        n = torch.full((B,), K, dtype=torch.int64)
    return dict(tgt=tgt, q_idx=q_idx, q_prob=q_prob, q_nnz=q_nnz, draft_tokens=d.to(torch.int32).cpu(),
                u_accept=u_acc, u_resample=u_res, draft_len=n.to(torch.int32), temperature=temperature)


def config3_sparse(device="cpu"):
    """Sparse stored-Q verify: B=32, K=16, V=151936 bf16, top-k = 20 drafter
    storage (the truncation Qwen3 recommends for this vocabulary), T=1, a
    +20 target peak (the target's argmax carries most of the mass)."""
    return sparse_inputs(31, 32, 16, 151936, torch.bfloat16, topk=20, peak=20.0, device=device)


def config3_truncate(device="cpu"):
    """Drafter-side storage of the sparse-Q workload: drafter rows
    [32, 16, 151936] bf16 = z + N(0, 1) (z the planted target logits),
    truncated to top-k 20, top-p 0.9."""
    c = 32
    z = _planted_logits(c, (32, 16, 151936), 20.0, torch.float32, device)
    drf = (z + torch.randn(32, 16, 151936, generator=_gen(c, 2, device), device=device)).to(torch.bfloat16)
    n = torch.full((32,), 16, dtype=torch.int32)
    return dict(drf=drf, draft_len=n, top_k=20, top_p=0.9)


# ------------------------------------------------------------------ DDTree --

def ddtree_inputs(c, B, L, V, dtype=torch.bfloat16, temperature=1.0, peak_lo=12.0, peak_hi=24.0,
                  masked_min=0.5, device="cpu"):
    """Inputs of draft-tree construction for a partly decoded block.

    stale [B, L, V]: z ~ N(0, 3^2) plus a peak at one seeded token, the peak
    height per row uniform in [peak_lo, peak_hi], so that the stale top-1
    probability falls on both sides of 0.6 across rows.  masked [B, L]: each
    sequence has a seeded number of masked positions in [masked_min * L, L]
    at seeded places.  gumbel [B, L, V] float32 (None at T = 0).  Two
    stand-in order models (the learned order model is not part of this
    work): order_table [B, L+1, L], row c (the last committed position) =
    -0.5 |s - c - 1| + N(0, 1), row L (the root) = -0.25 s + N(0, 1), a
    tendency to commit next to the last commit; and a set-dependent model
    order_A [B, L], order_B [B, L, L] whose logits for a state are order_A +
    the sum of order_B rows over the positions it has committed.
    """
    z = torch.randn(B, L, V, generator=_gen(c, 0, device), device=device) * 3.0
    pos = torch.randint(0, V, (B, L, 1), generator=_gen(c, 1, device), device=device)
    h = peak_lo + (peak_hi - peak_lo) * torch.rand(B, L, 1, generator=_gen(c, 2, device), device=device)
    z.scatter_add_(-1, pos, h)
    stale = z.to(dtype)
    gm = _gen(c, 8, "cpu")
    masked = torch.zeros(B, L, dtype=torch.uint8)
    lo = max(0, int(math.ceil(masked_min * L)))
    for b in range(B):
        k = int(torch.randint(lo, L + 1, (1,), generator=gm))
        masked[b, torch.randperm(L, generator=gm)[:k]] = 1
    G = gumbel_noise((B, L, V), _gen(c, 6, device), device) if temperature > 0 else None
    go = _gen(c, 9, "cpu")
    s = torch.arange(L, dtype=torch.float32)
    table = torch.randn(B, L + 1, L, generator=go)
    table[:, :L] += -0.5 * (s[None, :] - s[:, None] - 1).abs()
    table[:, L] += -0.25 * s
    oa = torch.randn(B, L, generator=_gen(c, 10, "cpu"))
    ob = torch.randn(B, L, L, generator=_gen(c, 11, "cpu")) * 0.7
    return dict(stale=stale, masked=masked.to(device), gumbel=G, temperature=temperature,
                order_table=table.to(device), order_A=oa.to(device), order_B=ob.to(device))


def config4_ddtree(device="cpu"):
    """DDTree construction: B=16 blocks of L=32 positions, V=151936 bf16
    stale rows, T=1 (coupled stale draw with Gumbel rows), budget D=20."""
    return ddtree_inputs(45, 16, 32, 151936, torch.bfloat16, temperature=1.0, device=device)


# ------------------------------------------------- Packed-SS loop driver --

LOOP_PEAK = 30.0


def packed_loop_inputs(c, B, W, V, L, dtype=torch.bfloat16, eps_pct=10, R=256, device="cpu"):
    """A synthetic model for a multi-iteration Packed-SS loop: its greedy
    continuation of sequence b is a seeded token string T[b] (the target's
    own greedy output), and every logit row is one of R seeded rows z ~ N(0,
    3^2) with one entry set to LOOP_PEAK = 30 (above every other logit).

    * Verify row r of a call (the token after the prefix P and r draft
      tokens) peaks at T[b, |P| + r] when those r draft tokens equal T there,
      else at a token hashed from (b, position).
    * Draft row j (position |P| + j, conditioned on P only) peaks at
      T[b, |P| + j], except when a coin hashed from (b, position, call) falls
      below eps_pct percent: then at a hashed token.

    The rows are pure data (gathers of table rows and one scatter), computed
    the same way on the CPU and on the GPU."""
    table = (torch.randn(R, V, generator=_gen(c, 0, "cpu")) * 3.0).to(dtype)
    T = torch.randint(0, V, (B, L + 2 * W), generator=_gen(c, 1, "cpu"))
    return dict(table=table.to(device), T=T.to(device), B=B, W=W, V=V, L=L, R=R, eps_pct=eps_pct)


def packed_loop_rows(inp, plen, d, n, t, seqs=None):
    """Packed rows [B, 2W, V] of call t for prefix lengths plen [B], drafts
    d [B, W-1] (-1 padded) and draft lengths n [B]: verify rows 0..W-1, then
    draft rows W..2W-1.  With seqs (a list of sequence indices) only those
    sequences' rows, in that order.  Tensors on the device of inp."""
    W, V, R = inp["W"], inp["V"], inp["R"]
    T, table = inp["T"], inp["table"]
    dev = T.device
    seq = torch.arange(inp["B"], device=dev) if seqs is None else torch.as_tensor(seqs, device=dev).long()
    B = seq.numel()
    T = T[seq]
    plen = plen.to(dev).long()
    d = d.to(dev).long()
    n = n.to(dev).long()
    r = torch.arange(W, device=dev)
    pos = plen[:, None] + r[None, :]                                    # [B, W]
    bb = seq[:, None]
    truth = torch.gather(T, 1, pos)
    # verify row r sees the draft tokens before it: all equal to T there?
    dm = torch.full((B, W), -1, dtype=torch.long, device=dev)
    dm[:, :W - 1] = torch.where(r[None, :W - 1] < n[:, None], d, torch.full_like(d, -1))
    agree = (dm == truth).long()
    ok = torch.ones((B, W), dtype=torch.long, device=dev)
    ok[:, 1:] = torch.cumprod(agree, dim=1)[:, :W - 1]
    other = (pos * 2654435761 + bb * 97 + 12345) % V
    vtok = torch.where(ok.bool(), truth, other)
    coin = (((pos * 40503 + bb * 31 + t * 17 + 7) * 2654435761) >> 16) % 100
    dtok = torch.where(coin >= inp["eps_pct"], truth, (pos * 2246822519 + bb * 13 + t * 7) % V)
    vrow = (bb * 131 + pos * 7) % R
    drow = (bb * 31 + pos * 11 + 5) % R
    rows = torch.cat([vrow, drow], dim=1)                               # [B, 2W]
    packed = table[rows.reshape(-1)].reshape(B, 2 * W, V).clone()
    peak = torch.cat([vtok, dtok], dim=1)[:, :, None]
    packed.scatter_(2, peak, torch.full(peak.shape, LOOP_PEAK, dtype=packed.dtype, device=dev))
    return packed


def config5_loop(device="cpu"):
    """Packed-SS loop: B=64 sequences, W=32 (31 draft positions verified +
    the bonus row, 32 draft rows per call), V=131072 bf16, L=256 new tokens,
    a drafter wrong at 10% of positions."""
    return packed_loop_inputs(51, 64, 32, 131072, 256, torch.bfloat16, eps_pct=10, device=device)

"""Seeded random shapes through the chain entry points (greedy, lossless,
lenient, Cactus) against the oracle: batch sizes, draft lengths (ragged),
vocabularies on and off the tile and vector boundaries, both dtypes,
temperatures, EOS and length budgets drawn per case."""

import sys

import numpy as np
import pytest
import torch

import draft_block_verification_amd as dbv
import oracle
import workloads
from tests.parity import check_greedy, check_sampling

pytestmark = pytest.mark.gpu

CASES = 80


def _np(x):
    return {k: (v.double().numpy() if v.is_floating_point() else v.numpy()) if torch.is_tensor(v) else v
            for k, v in x.items()}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("seed", [11, 12])
def test_random_chain_cases(dev, seed):
    rng = np.random.default_rng(seed)
    for n in range(CASES // 2):
        B = int(rng.integers(1, 40))
        K = int(rng.choice([0, 1, 2, 3, 5, 8, 13, 31, 64]))
        V = int(rng.choice([1, 2, 7, 100, 511, 513, 4096, 8193, 20011, 32000, 70001]))
        dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
        rule = str(rng.choice(["rejection", "lenient", "cactus", "greedy"]))
        T = float(rng.choice([1.0, 0.7, 1.3]))
        x = workloads.chain_inputs(int(rng.integers(100, 1100)), B, K, V, dtype,
                                   sigma=float(rng.choice([0.1, 1.0, 3.0])), temperature=T,
                                   random_lengths=bool(rng.random() < 0.7))
        eos = int(rng.integers(0, V)) if rng.random() < 0.3 else -1
        bud = torch.randint(0, K + 3, (B,), dtype=torch.int32) if rng.random() < 0.3 else None
        lam = float(rng.choice([0.0, 0.3, 0.9, 1.0]))
        delta = float(rng.choice([0.0, 0.1, 1.0, 5.0]))
        print("[case]", seed, n, rule, B, K, V, dtype, T, eos, bud is not None, lam, delta, flush=True)
        sys.stdout.flush()
        xd = {k: v.to(dev) if torch.is_tensor(v) else v for k, v in x.items()}
        xn = _np(x)
        bd = None if bud is None else bud.to(dev)
        bn = None if bud is None else bud.numpy()
        name = str(dtype).split(".")[1]
        if rule == "greedy":
            rows = xd["drf"] if K > 0 else None
            g = dbv.verify_greedy(xd["tgt"], xd["draft_tokens"], xd["draft_len"], rows, eos_id=eos, len_budget=bd)
            o = oracle.verify_greedy(xn["tgt"], xn["draft_tokens"], xn["draft_len"], xn["drf"] if K > 0 else None,
                                     eos_id=eos, len_budget=bn)
            check_greedy(g, o)
            continue
        kw = dict(draft_len=xd["draft_len"], temperature_target=T, temperature_draft=T, eos_id=eos, len_budget=bd)
        args = (xn["tgt"], xn["drf"], xn["draft_tokens"], xn["draft_len"], T, T)
        uni = (xn["u_accept"], xn["u_resample"])
        if rule == "rejection":
            g = dbv.verify_rejection(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"], **kw)
            o = oracle.verify_rejection(*args, *uni, eos_id=eos, len_budget=bn)
            check_sampling(g, xn, o, 0.0, T, T, name, eos_id=eos, len_budget=bn)
        elif rule == "lenient":
            g = dbv.verify_lenient(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"], lam,
                                   **kw)
            o = oracle.verify_lenient(*args, lam, *uni, eos_id=eos, len_budget=bn)
            check_sampling(g, xn, o, lam, T, T, name, eos_id=eos, len_budget=bn)
        else:
            g = dbv.verify_cactus(xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"], delta,
                                  **kw)
            o = oracle.verify_cactus(*args, delta, *uni, eos_id=eos, len_budget=bn)
            check_sampling(g, xn, o, 0.0, T, T, name, eos_id=eos, len_budget=bn, delta=delta)


@pytest.mark.parametrize("seed", [21, 22])
def test_random_tree_spot_any_order_cases(dev, seed):
    # Same idea for the Gumbel tree (T = 0 and T > 0), the
    # joint-space chain (with and without coupled-noise rows, three gates)
    # and any-order greedy verification (with and without drafter rows and
    # positions).
    import tests.test_parity_gpu as fixed
    from tests.parity import check_any_order, check_spot, check_tree
    rng = np.random.default_rng(seed)
    for n in range(CASES // 2):
        kind = str(rng.choice(["tree", "spot", "any-order"]))
        dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
        name = str(dtype).split(".")[1]
        c = int(rng.integers(100, 5000))
        if kind == "tree":
            B, S = int(rng.integers(1, 6)), int(rng.choice([2, 5, 12, 33, 64]))
            L, V = int(rng.choice([2, 4, 6, 9, 16])), int(rng.choice([7, 513, 5003, 20011]))
            T = float(rng.choice([0.0, 0.7, 1.0]))
            sig = float(rng.choice([0.05, 0.5]))
            print("[case]", seed, n, kind, B, S, L, V, dtype, T, flush=True)
            x = workloads.tree_inputs(c, B, S, L, V, dtype, sigma_node=sig, temperature=T if T > 0 else 1.0)
            g = dbv.verify_gumbel_tree(x["logits"].to(dev), x["parent"].to(dev), x["edge_pos"].to(dev),
                                       x["edge_tok"].to(dev), masked=x["masked"].to(dev),
                                       gumbel=x["gumbel"].to(dev) if T > 0 else None, temperature=T,
                                       num_states=x["num_states"].to(dev))
            xn = fixed._np_inputs(x)
            xn["masked"] = x["masked"].numpy()
            o = oracle.verify_gumbel_tree(xn["logits"], xn["masked"], xn["parent"], xn["edge_pos"],
                                          xn["edge_tok"], xn["num_states"], xn["gumbel"], T)
            check_tree(g, xn, o, name, T)
        elif kind == "spot":
            B, K, V = int(rng.integers(1, 24)), int(rng.choice([1, 2, 5, 8, 16])), int(rng.choice([513, 5003, 40000]))
            gum = bool(rng.random() < 0.6)
            tau = float(rng.choice([0.3, 0.6, 0.9]))
            T = float(rng.choice([0.7, 1.0]))
            ragged = bool(rng.random() < 0.7)
            print("[case]", seed, n, kind, B, K, V, dtype, gum, tau, flush=True)
            x = workloads.spot_chain_inputs(c, B, K, V, dtype, temperature=T, random_lengths=ragged, gumbel=gum)
            g, xn, o = fixed._spot_run(dev, x, tau=tau, gumbel=gum)
            check_spot(g, xn, o, T, T, tau, name)
        else:
            B, U, V = int(rng.integers(1, 40)), int(rng.choice([1, 2, 5, 16, 32])), int(rng.choice([7, 513, 5003]))
            agree = float(rng.choice([0.3, 0.8, 0.97]))
            missing = float(rng.choice([0.0, 0.15, 0.5]))
            rows, pos = bool(rng.random() < 0.7), bool(rng.random() < 0.7)
            print("[case]", seed, n, kind, B, U, V, dtype, rows, pos, flush=True)
            x = workloads.anyorder_inputs(c, B, U, V, dtype, agree=agree, missing=missing)
            g, o = fixed._ao_run(dev, x, draft_rows=rows, positions=pos)
            check_any_order(g, o)


@pytest.mark.parametrize("seed", [31, 32])
def test_random_truncate_sparse_ddtree_cases(dev, seed):
    # Top-k / top-p truncation (tied rows included), verification against
    # stored sparse Q, and DDTree hypotheses plus the level-batched build.
    import tests.test_parity_ddtree_gpu as dd
    import tests.test_parity_gpu as fixed
    from tests.parity import np64, npi
    rng = np.random.default_rng(seed)
    for n in range(CASES // 2):
        kind = str(rng.choice(["truncate", "sparse", "ddtree"]))
        dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
        name = str(dtype).split(".")[1]
        c = int(rng.integers(100, 5000))
        if kind == "truncate":
            B, K, V = int(rng.integers(1, 8)), int(rng.integers(1, 6)), int(rng.choice([1, 5, 300, 4097, 20011]))
            k, p = int(rng.choice([1, 2, 5, 20, 64, 256])), float(rng.choice([1.0, 0.9, 0.5, 0.05]))
            T, scale = float(rng.choice([0.5, 0.8, 1.0, 2.0])), float(rng.choice([0.3, 3.0, 10.0]))
            kmax = int(rng.choice([k, 256]))
            ties = bool(rng.random() < 0.3)
            print("[case]", seed, n, kind, B, K, V, dtype, k, p, T, kmax, ties, flush=True)
            rows = torch.randn(B, K, V, generator=torch.Generator().manual_seed(c)) * scale
            rows = (torch.round(rows) if ties else rows).to(dtype)
            lengths = torch.randint(0, K + 1, (B,), dtype=torch.int32, generator=torch.Generator().manual_seed(c))
            g = dbv.truncate_top_k_top_p(rows.to(dev), k, p, kmax=kmax, lengths=lengths.to(dev), temperature=T)
            fixed._trunc_check(g, np64(rows), T, k, p, kmax, npi(lengths), name)
        elif kind == "sparse":
            B, K, V = int(rng.integers(1, 16)), int(rng.choice([1, 3, 8])), int(rng.choice([300, 5003, 40000]))
            topk, peak = int(rng.choice([1, 5, 20, 64])), float(rng.choice([2.0, 6.0]))
            print("[case]", seed, n, kind, B, K, V, dtype, topk, peak, flush=True)
            x = workloads.sparse_inputs(c, B, K, V, dtype, topk=topk, peak=peak, random_lengths=True)
            g, xn, o, qfun = fixed._sparse_run(dev, x)
            check_sampling(g, xn, o, 0.0, x["temperature"], x["temperature"], name, qfun=qfun)
        else:
            B, L, V = int(rng.integers(1, 12)), int(rng.choice([1, 2, 5, 16, 32, 64])), int(rng.choice([7, 513, 2053]))
            T, D = float(rng.choice([0.0, 0.6, 1.0])), int(rng.choice([0, 1, 3, 8, 20, 64]))
            tau, gamma = float(rng.choice([0.7, 1.0, 1.3])), float(rng.choice([0.0, 0.0, 0.01, 0.05]))
            rub, mm = float(rng.choice([0.6, 0.3, 0.9])), float(rng.choice([0.0, 0.5, 1.0]))
            print("[case]", seed, n, kind, B, L, V, dtype, T, D, tau, gamma, rub, mm, flush=True)
            x = workloads.ddtree_inputs(c, B, L, V, dtype, temperature=T, masked_min=mm)
            h, st = dd._run_build(x, dev, D, tau, gamma, runner_up_below=rub)
            order = oracle.table_order(np64(x["order_table"]))
            o = dd._oracle(x, order, D, tau, gamma, runner_up_below=rub)
            dd._check_all(h, st, o, x, order, D, tau, gamma, name)

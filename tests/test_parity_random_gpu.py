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

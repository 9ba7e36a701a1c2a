"""The multi-iteration Packed-SS loop on the GPU (verify_greedy through the C
ABI, bookkeeping on the device) against the loop oracle, call by call, on
the synthetic model with a known greedy continuation."""

import sys

import numpy as np
import pytest
import torch

import oracle.loop as oloop
import workloads
from draft_block_verification_amd.loop import packed_ss_greedy_loop
from tests.parity import npi

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _gpu_model(inp):
    return lambda plen, d, n, t: workloads.packed_loop_rows(inp, plen, d, n, t)


def _cpu_model(inp):
    def fn(plen, d, n, t):
        return workloads.packed_loop_rows(inp, torch.as_tensor(plen), torch.as_tensor(d), torch.as_tensor(n),
                                          t).double().numpy()
    return fn


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("W,eps,eos", [(8, 10, -1), (8, 40, -1), (5, 0, -1), (6, 25, 4000)])
def test_loop_parity(dev, dtype, W, eps, eos):
    say("packed loop", dtype, W, eps, eos)
    B, V, L = 6, 4099, 70
    inp = workloads.packed_loop_inputs(400 + eps + W, B, W, V, L, dtype, eps_pct=eps)
    if eos >= 0:
        inp["T"][inp["T"] == eos] = 1
        inp["T"][2, 33] = eos
    g = packed_ss_greedy_loop(_gpu_model({**inp, "table": inp["table"].to(dev), "T": inp["T"].to(dev)}),
                              B, W, L, 400, dev, eos_id=eos)
    torch.cuda.synchronize()
    toks, calls = oloop.packed_ss_greedy(_cpu_model(inp), B, W, L, 400, eos_id=eos)
    assert g["calls"] == len(calls)
    for k in ("num_out", "accept_len", "draft_len", "status"):
        np.testing.assert_array_equal(npi(g[k]), np.stack([c[k] for c in calls]), err_msg=k)
    gt = npi(g["tokens"])
    for b in range(B):
        assert gt[b, :len(toks[b])].tolist() == toks[b]
        assert (gt[b, len(toks[b]):] == -1).all()
        assert toks[b] == inp["T"][b, :len(toks[b])].tolist()
    say("tokens per call", np.mean([c["num_out"][b] for c in calls for b in range(B) if c["draft_len"][b] >= 0]))


def test_loop_full_size(dev):
    """The benchmarked loop (B=64, W=32, V=131072 bf16, L=256): the output
    is the verifier's greedy continuation for every sequence, and the calls
    account for every token."""
    say("packed loop full size")
    inp = workloads.config5_loop(device=dev)
    g = packed_ss_greedy_loop(_gpu_model(inp), 64, 32, 256, 1000, dev)
    torch.cuda.synchronize()
    T = inp["T"].cpu()
    assert torch.equal(g["tokens"].cpu(), T[:, :256].to(torch.int32))
    assert (npi(g["num_out"]).sum(axis=0) == 256).all()
    assert (npi(g["status"]) == 0).all()
    say("calls", g["calls"], "tokens per call", 64 * 256 / max(1, int((npi(g["num_out"]) > 0).sum())))

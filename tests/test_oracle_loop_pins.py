"""Pins of the multi-iteration Packed-SS loop oracle (Packed-SS, Sec. 3.1
and Algorithm 1) on a synthetic model whose greedy continuation is known:
greedy exactness, the closed-form call pattern of a perfect and of an
always-wrong drafter, the length limit and EOS."""

import numpy as np
import pytest
import torch

import oracle.loop as lp
import workloads


def _model(inp):
    def fn(plen, d, n, t):
        return workloads.packed_loop_rows(inp, torch.as_tensor(plen), torch.as_tensor(d), torch.as_tensor(n),
                                          t).double().numpy()
    return fn


@pytest.mark.parametrize("eps", [0, 10, 50, 100])
def test_greedy_exactness(eps):
    """The emitted string is the verifier's own greedy decoding, whatever
    the drafter does (Packed-SS Sec. 3.1)."""
    B, W, V, L = 3, 5, 64, 23
    inp = workloads.packed_loop_inputs(200 + eps, B, W, V, L, torch.float32, eps_pct=eps)
    toks, calls = lp.packed_ss_greedy(_model(inp), B, W, L, 500)
    for b in range(B):
        assert toks[b] == inp["T"][b, :L].tolist()
    assert all((c["status"] == 0).all() for c in calls)


def test_perfect_drafter_alternates():
    """A drafter that is always right: call 1 has no draft (1 token); its W
    draft rows leave W - 1 correct drafts, all accepted plus the bonus (W
    tokens), which leaves an empty draft again: 1, W, 1, W, ..."""
    B, W, V, L = 2, 6, 80, 40
    inp = workloads.packed_loop_inputs(300, B, W, V, L, torch.float32, eps_pct=0)
    toks, calls = lp.packed_ss_greedy(_model(inp), B, W, L, 100)
    pattern = [int(c["num_out"][0]) for c in calls]
    exp = []
    left = L
    k = 0
    while left > 0:
        a = min(1 if k % 2 == 0 else W, left)
        exp.append(a)
        left -= a
        k += 1
    assert pattern == exp
    assert len(calls) == len(exp)


def test_always_wrong_drafter_one_token_per_call():
    B, W, V, L = 2, 4, 500, 17
    inp = workloads.packed_loop_inputs(301, B, W, V, L, torch.float32, eps_pct=100)
    toks, calls = lp.packed_ss_greedy(_model(inp), B, W, L, 100)
    assert len(calls) == L
    assert all(int(c["num_out"][b]) == 1 for c in calls for b in range(B))
    # every draft after the first call had W - 1 tokens, none accepted
    assert all(int(c["accept_len"][b]) == 0 for c in calls for b in range(B))


def test_length_limit_and_eos():
    B, W, V, L = 2, 6, 64, 30
    inp = workloads.packed_loop_inputs(302, B, W, V, L, torch.float32, eps_pct=0)
    T = inp["T"]
    eos = 63
    T[T == eos] = 0
    T[0, 11] = eos                     # sequence 0 ends with the EOS at its 12th token
    toks, calls = lp.packed_ss_greedy(_model(inp), B, W, L, 100, eos_id=eos)
    assert toks[0] == T[0, :12].tolist()
    assert toks[1] == T[1, :L].tolist()
    # once stopped, a sequence accepts nothing and keeps an empty draft
    done = np.cumsum([int(c["num_out"][0]) for c in calls])
    stop = int(np.argmax(done == 12))
    assert done[stop] == 12 and stop + 1 < len(calls)
    for c in calls[stop + 1:]:
        assert int(c["num_out"][0]) == 0 and int(c["draft_len"][0]) == 0

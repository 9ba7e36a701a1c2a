"""verify_rejection_noalloc (the entry point that allocates nothing) against
verify_rejection on the same inputs: every output identical, on two calls in
a row whose second has a smaller batch and vocabulary (the library's scratch
keeps the first call's contents), and a call beyond the scratch limit is
refused without launching."""

import sys

import pytest
import torch

import draft_block_verification_amd as dbv
import workloads

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _same(a, b):
    for k in a:
        assert torch.equal(a[k], b[k]), k


def _inputs(seed, B, K, V, dtype):
    x = workloads.chain_inputs(seed, B, K, V, dtype, sigma=1.0)
    return x


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_equals_rejection_twice(dev, dtype):
    for seed, B, K, V in ((81, 32, 16, 128256), (82, 5, 7, 3001)):
        say("noalloc", dtype, B, K, V)
        x = _inputs(seed, B, K, V, dtype)
        xd = {k: v.to(dev) if torch.is_tensor(v) else v for k, v in x.items()}
        args = (xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"])
        kw = dict(draft_len=xd["draft_len"], margins=True)
        ref = dbv.verify_rejection(*args, **kw)
        got = dbv.verify_rejection_noalloc(*args, **kw)
        torch.cuda.synchronize()
        _same(ref, got)
        assert int((got["status"] & dbv.SEQ_ERROR_MASK).sum()) == 0


def test_noalloc_refuses_beyond_its_scratch(dev):
    say("noalloc limit")
    B, K, V = 1024, 64, 151936
    # one row of logits seen through zero sequence and row strides: the
    # call is refused before anything would read it
    row = torch.zeros(V, dtype=torch.bfloat16, device=dev)
    tgt = row.expand(B, K + 1, V)
    drf = row.expand(B, K, V)
    d = torch.zeros(B, K, dtype=torch.int32, device=dev)
    ua = torch.zeros(B, K, device=dev)
    ur = torch.zeros(B, K + 1, device=dev)
    with pytest.raises(dbv.DBVError) as e:
        dbv.verify_rejection_noalloc(tgt, drf, d, ua, ur)
    assert e.value.code == 2   # DBV_ERR_UNSUPPORTED

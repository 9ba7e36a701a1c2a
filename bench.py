#!/usr/bin/env python3
"""Benchmark of parallel draft-block verification on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]

A step is one verify call over one batch of synthetic inputs already resident
in HBM: every row statistic / argmax, the acceptance tests, the prefix scan,
and the correction or bonus draw.  Workloads (sizes of the pages' setups):

  c1  tiny rejection verify       B=1  K=4  V=1024   fp32
  c2  batch lossless verify       B=8  K=8  V=32000  bf16   (default)
  c3  lenient verify              B=32 K=16 V=128256 bf16, sigma=1, T=1, lambda=0.5
  c4  coupled-Gumbel tree verify  B=16 S=64 L=32 V=151936 bf16
  c5  packed greedy verify+draft  B=64 K=32 V=131072 bf16
  c3c modified-Cactus verify      B=32 K=16 V=128256 bf16, sigma=1, T=1, delta=1
  c5ao any-order greedy verify    B=64 U=32 V=131072 bf16 (verifier rows by rank,
                                  drafter rows by slot)
  c4s joint-space chain, hybrid   B=16 K=8 V=151936 bf16, T=1, tau=0.6, Gumbel
                                  rows for every target row
  c3q stored sparse-Q verify      B=32 K=16 V=151936 bf16, top-k = 20 drafter Q
  c3t top-k/top-p storage         B=32 K=16 V=151936 bf16 drafter rows -> top-k 20,
                                  top-p 0.9 sparse Q (positions = rows stored)
  c4d DDTree construction         B=16 L=32 V=151936 bf16 stale rows, T=1 (Gumbel
                                  rows), budget D=20: hypotheses + top-D search
                                  (positions = tree states drafted)
  c5loop Packed-SS loop           B=64 W=32 V=131072 bf16, 256 new tokens per
                                  sequence: verify_greedy once per model call
                                  over a synthetic model with a known greedy
                                  continuation; a step is one verify call, the
                                  model's rows are written between steps
                                  (untimed); reports tokens per call

Inputs smaller than 1 GiB are replicated into several buffer sets and the
steps rotate over them, so the 256 MiB last-level cache cannot serve them.
Prints one JSON line: whole-job verified draft positions per second, the
roofline of the row-streaming kernel (timed alone with HIP events that the
launch stamps at the kernel's start and end), and the CPU oracle timed on a
bounded sample.  `roofline.traffic` is the HBM bytes per launch that the
stored counter readings (profiles/traffic.json) give for the same kernel
sources, else null.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "verified draft positions/sec and achieved HBM GB/s vs MI355X peak (1 GPU)"
ROTATE_BYTES = 1 << 30         # replicate inputs up to this many bytes

DESCR = {
    "c1": "tiny rejection verify B=1 K=4 V=1024 fp32",
    "c2": "batch lossless verify B=8 K=8 V=32000 bf16",
    "c3": "lenient verify B=32 K=16 V=128256 bf16 sigma=1 T=1 lambda=0.5",
    "c4": "coupled-Gumbel tree verify B=16 S=64 L=32 V=151936 bf16",
    "c5": "packed greedy verify+draft B=64 K=32 V=131072 bf16",
    "c3c": "modified-Cactus verify B=32 K=16 V=128256 bf16 sigma=1 T=1 delta=1",
    "c5ao": "any-order greedy verify B=64 U=32 V=131072 bf16",
    "c4s": "joint-space chain hybrid B=16 K=8 V=151936 bf16 T=1 tau=0.6",
    "c3q": "sparse stored-Q verify B=32 K=16 V=151936 bf16 top-k=20",
    "c3t": "top-k/top-p truncation B=32 K=16 V=151936 bf16 top-k=20 top-p=0.9",
    "c4d": "DDTree construction B=16 L=32 V=151936 bf16 T=1 D=20",
    "c5loop": "Packed-SS greedy loop B=64 W=32 V=131072 bf16 L=256, drafter right at 90% of positions",
}
DD_BUDGET = 20
SPOT_TAU = 0.6
CACTUS_DELTA = 1.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="c2", choices=sorted(DESCR))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain device copy of COPY_PROBE_BYTES five times "
                         "(the reference kernel for scaling HBM counters)")
    return ap.parse_args()


COPY_PROBE_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic.json")


# The source file that defines each measured kernel; its counter readings
# hold only for that file and the headers every kernel file includes.
KERNEL_FILES = {"k_sample_rows": "kernels_chain.hip", "k_greedy_rows": "kernels_chain.hip",
                "k_tree_conf": "kernels_tree.hip", "k_ao_rows": "kernels_anyorder.hip",
                "k_truncate": "kernels_truncate.hip", "k_dd_rows": "kernels_ddtree.hip"}
SHARED_HEADERS = ("dbv_device.h", "dbv_launch.h", "dbv_plan.h")


def kernel_source_hash(kernel):
    """Hash of the HIP sources of `kernel`: counter readings apply only to
    the code they were taken on."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(HERE, "draft_block_verification_amd", "csrc")
    for f in (KERNEL_FILES[kernel],) + SHARED_HEADERS:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the stored counter readings
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel factor), or None when
    there are none for these sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    e = t.get("workloads", {}).get(workload)
    if not e or e.get("kernel") != kernel or e.get("source_hash") != kernel_source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


# --------------------------------------------------------------- workloads ---

class _Steps:
    """Prepared calls enqueued one after the other as one step."""

    def __init__(self, calls):
        self.calls = calls
        self.outputs = calls[-1].outputs

    def __call__(self):
        for c in self.calls:
            c()
        return self.outputs


class Case:
    """One workload: prepared calls over R rotated input sets, plus what the
    roofline and the CPU baseline need."""

    def __init__(self, name, dev):
        import draft_block_verification_amd as dbv
        import workloads
        self.name = name
        self.dev = dev
        eb = 2
        if name in ("c1", "c2", "c3", "c3c"):
            if name == "c1":
                x = workloads.config1()
                eb = 4
            elif name == "c2":
                x = workloads.config2()
            else:
                x = workloads.config3(1.0, 1.0)
            self.lam = 0.5 if name == "c3" else 0.0
            B, K1, V = x["tgt"].shape
            K = K1 - 1
            n = x["draft_len"].long()
            self.positions = int(n.sum())
            self.kernel_bytes = int(((2 * n + 1) * V * eb).sum())      # target n+1 rows, draft n rows
            self.kernel = "k_sample_rows"
            per_set = (x["tgt"].numel() + x["drf"].numel()) * eb
            self.cpu_inputs = x
            self.calls = []
            R = self._rotation(per_set)
            for _ in range(R):
                xd = {k: v.to(dev).clone() if torch.is_tensor(v) else v for k, v in x.items()}
                kw = dict(draft_len=xd["draft_len"], temperature_target=x["temperature"],
                          temperature_draft=x["temperature"], prepare=True)
                args = (xd["tgt"], xd["drf"], xd["draft_tokens"], xd["u_accept"], xd["u_resample"])
                if name == "c3":
                    c = dbv.verify_lenient(*args, self.lam, **kw)
                elif name == "c3c":
                    c = dbv.verify_cactus(*args, CACTUS_DELTA, **kw)
                else:
                    c = dbv.verify_rejection(*args, **kw)
                self.calls.append(c)
            self.shape = dict(B=B, K=K, V=V)
        elif name == "c5":
            x = workloads.config5()
            K, W = x["K"], x["W"]
            B, _, V = x["packed"].shape
            n = x["draft_len"].long()
            self.positions = int(n.sum())
            self.kernel_bytes = int(((n + 1 + W) * V * eb).sum())
            self.kernel = "k_greedy_rows"
            per_set = x["packed"].numel() * eb
            self.cpu_inputs = x
            self.calls = []
            for _ in range(self._rotation(per_set)):
                p = x["packed"].to(dev)
                self.calls.append(dbv.verify_greedy(p[:, :K + 1], x["draft_tokens"].to(dev),
                                                    x["draft_len"].to(dev), p[:, K + 1:], prepare=True))
            self.shape = dict(B=B, K=K, W=W, V=V)
        elif name == "c3q":
            x = workloads.config3_sparse()
            B, K1, V = x["tgt"].shape
            K = K1 - 1
            n = x["draft_len"].long()
            self.positions = int(n.sum())
            self.kernel_bytes = int(((n + 1) * V * eb).sum())     # target rows only; Q is a few KB
            self.kernel = "k_sample_rows"
            per_set = x["tgt"].numel() * eb
            self.cpu_inputs = x
            self.calls = []
            for _ in range(self._rotation(per_set)):
                xd = {k: v.to(dev).clone() if torch.is_tensor(v) else v for k, v in x.items()}
                self.calls.append(dbv.verify_sparse(
                    xd["tgt"], xd["q_idx"], xd["q_prob"], xd["q_nnz"], xd["draft_tokens"], xd["u_accept"],
                    xd["u_resample"], draft_len=xd["draft_len"], prepare=True))
            self.shape = dict(B=B, K=K, V=V)
        elif name == "c3t":
            x = workloads.config3_truncate()
            B, K, V = x["drf"].shape
            n = x["draft_len"].long()
            self.positions = int(n.sum())
            self.kernel_bytes = int((n * V * eb).sum())                 # drafter rows 0..n-1, read once
            self.kernel = "k_truncate"
            per_set = x["drf"].numel() * eb
            self.cpu_inputs = x
            self.calls = []
            for _ in range(self._rotation(per_set)):
                xd = {k: v.to(dev).clone() if torch.is_tensor(v) else v for k, v in x.items()}
                self.calls.append(dbv.truncate_top_k_top_p(xd["drf"], x["top_k"], x["top_p"], kmax=x["top_k"],
                                                           lengths=xd["draft_len"], prepare=True))
            self.shape = dict(B=B, K=K, V=V)
        elif name == "c4d":
            x = workloads.config4_ddtree()
            B, L, V = x["stale"].shape
            nm = int(x["masked"].sum())
            self.positions = B * DD_BUDGET
            self.kernel_bytes = nm * V * (eb + 4)                      # masked stale rows + Gumbel rows
            self.kernel = "k_dd_rows"
            per_set = x["stale"].numel() * eb + x["gumbel"].numel() * 4
            self.cpu_inputs = x
            self.calls = []
            for _ in range(self._rotation(per_set)):
                xd = {k: v.to(dev).clone() if torch.is_tensor(v) else v for k, v in x.items()}
                h = dbv.ddtree_hypotheses(xd["stale"], xd["masked"], temperature=1.0, gumbel=xd["gumbel"],
                                          prepare=True)
                t = dbv.ddtree_build(xd["masked"], h.outputs["hyp_tok"], h.outputs["hyp_prob"],
                                     xd["order_table"], DD_BUDGET, status=h.outputs["status"], prepare=True)
                self.calls.append(_Steps([h, t]))
            self.shape = dict(B=B, L=L, V=V, D=DD_BUDGET, masked_rows=nm)
        elif name == "c4s":
            x = workloads.config4_spot_chain()
            B, K1, V = x["tgt"].shape
            K = K1 - 1
            n = x["draft_len"].long()
            self.positions = int(n.sum())
            # target rows 0..n with their float32 Gumbel rows, drafter rows 0..n-1
            self.kernel_bytes = int(((n + 1) * V * (eb + 4) + n * V * eb).sum())
            self.kernel = "k_sample_rows"
            per_set = (x["tgt"].numel() + x["drf"].numel()) * eb + x["gumbel"].numel() * 4
            self.cpu_inputs = x
            self.calls = []
            for _ in range(self._rotation(per_set)):
                xd = {k: v.to(dev).clone() if torch.is_tensor(v) else v for k, v in x.items()}
                self.calls.append(dbv.verify_spot_chain(
                    xd["tgt"], xd["drf"], xd["pos_star"], xd["prop_pos"], xd["prop_tok"], xd["q_pos_star"],
                    xd["u_accept"], xd["u_resample"], gumbel=xd["gumbel"], tau=SPOT_TAU, draft_len=xd["draft_len"],
                    prepare=True))
            self.shape = dict(B=B, K=K, V=V)
        elif name == "c5ao":
            x = workloads.config5_any_order()
            B, U, V = x["tgt"].shape
            u = x["num_active"].long()
            kappa = self._kappa(x)
            nver = torch.minimum(kappa + 1, u)
            self.positions = int(kappa.sum())                            # drafted positions checked
            self.kernel_bytes = int(((nver + u) * V * eb).sum())         # verifier rows read + drafter rows
            self.kernel = "k_ao_rows"
            per_set = (x["tgt"].numel() + x["draft_rows"].numel()) * eb
            self.cpu_inputs = x
            self.calls = []
            for _ in range(self._rotation(per_set)):
                xd = {k: v.to(dev).clone() for k, v in x.items()}
                self.calls.append(dbv.verify_greedy_any_order(
                    xd["tgt"], xd["order"], xd["draft_tokens"], num_active=xd["num_active"],
                    positions=xd["positions"], draft_rows=xd["draft_rows"], prepare=True))
            self.shape = dict(B=B, U=U, V=V)
        else:  # c4
            x = workloads.config4(device=dev)
            B, S, L, V = x["logits"].shape
            ns = x["num_states"].long()
            self.positions = int((ns - 1).sum())
            m = x["masked"].clone()
            for b in range(B):
                m[b, int(ns[b]):] = False
            self.kernel_bytes = int(m.sum()) * V * eb
            self.kernel = "k_tree_conf"
            self.cpu_inputs = x
            self.calls = [dbv.verify_gumbel_tree(
                x["logits"], x["parent"].to(dev), x["edge_pos"].to(dev), x["edge_tok"].to(dev),
                masked=x["masked"].to(dev), gumbel=x["gumbel"], temperature=1.0,
                num_states=x["num_states"].to(dev), prepare=True)]
            self.shape = dict(B=B, S=S, L=L, V=V)
            per_set = x["logits"].numel() * eb + x["gumbel"].numel() * 4
        self.rotation = len(self.calls)
        self.bytes_per_set = per_set

    @staticmethod
    def _kappa(x):
        """Leading ranks whose slot holds a draft, per sequence (host-side
        count of the positions a call verifies)."""
        d = torch.gather(x["draft_tokens"].long(), 1, x["order"].long())
        r = torch.arange(d.shape[1])[None, :]
        have = (d >= 0) & (r < x["num_active"].long()[:, None])
        return torch.cumprod(have.long(), dim=1).sum(dim=1)

    @staticmethod
    def _rotation(per_set):
        return int(max(1, min(256, math.ceil(ROTATE_BYTES / max(per_set, 1)))))

    # ------------------------------------------------------------ oracle --
    def cpu_baseline(self, seconds):
        """The oracle as it stands on a bounded sample of this workload."""
        import oracle
        from tests.parity import np64, npi
        x = self.cpu_inputs
        done_pos = 0
        calls = 0
        t0 = time.perf_counter()
        if self.name in ("c1", "c2", "c3", "c3c"):
            B = x["tgt"].shape[0]
            nb = min(B, 4) if self.name in ("c3", "c3c") else B
            tgt, drf = np64(x["tgt"][:nb]), np64(x["drf"][:nb])
            d, n = npi(x["draft_tokens"][:nb]), npi(x["draft_len"][:nb])
            ua, ur = np64(x["u_accept"][:nb]), np64(x["u_resample"][:nb])
            T = x["temperature"]
            t0 = time.perf_counter()
            while True:
                if self.name == "c3c":
                    oracle.verify_cactus(tgt, drf, d, n, T, T, CACTUS_DELTA, ua, ur)
                else:
                    oracle.verify_lenient(tgt, drf, d, n, T, T, self.lam, ua, ur)
                done_pos += int(n.sum())
                calls += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            sample = f"{nb} of {B} sequences, {calls} oracle calls"
        elif self.name == "c5":
            K, W = x["K"], x["W"]
            nb = 4
            p = x["packed"][:nb]
            tgt, dr = np64(p[:, :K + 1]), np64(p[:, K + 1:])
            d, n = npi(x["draft_tokens"][:nb]), npi(x["draft_len"][:nb])
            t0 = time.perf_counter()
            while True:
                oracle.verify_greedy(tgt, d, n, dr)
                done_pos += int(n.sum())
                calls += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            sample = f"{nb} of 64 sequences, {calls} oracle calls"
        elif self.name == "c3t":
            nb = 1
            rows = np64(x["drf"][:nb])
            npos = int(x["draft_len"][:nb].sum())
            t0 = time.perf_counter()
            while True:
                oracle.truncate_rows(rows, 1.0, x["top_k"], x["top_p"], x["top_k"], npi(x["draft_len"][:nb]))
                done_pos += npos
                calls += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            sample = f"{nb} of 32 sequences, {calls} oracle calls"
        elif self.name == "c4d":
            nb = 1
            st, m = np64(x["stale"][:nb]), npi(x["masked"][:nb])
            G = np64(x["gumbel"][:nb])
            fn = oracle.table_order(np64(x["order_table"][:nb]))
            t0 = time.perf_counter()
            while True:
                oracle.build_ddtree(st, m, fn, DD_BUDGET, 1.0, gumbel=G)
                done_pos += nb * DD_BUDGET
                calls += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            sample = f"{nb} of 16 blocks, {calls} oracle calls"
        elif self.name == "c3q":
            nb = 4
            xs = {k: v[:nb] if torch.is_tensor(v) else v for k, v in x.items()}
            args = [np64(xs["tgt"]), npi(xs["q_idx"]), np64(xs["q_prob"]), npi(xs["q_nnz"]),
                    npi(xs["draft_tokens"]), npi(xs["draft_len"]), 1.0, np64(xs["u_accept"]),
                    np64(xs["u_resample"])]
            npos = int(xs["draft_len"].sum())
            t0 = time.perf_counter()
            while True:
                oracle.verify_sparse(*args)
                done_pos += npos
                calls += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            sample = f"{nb} of 32 sequences, {calls} oracle calls"
        elif self.name == "c4s":
            nb = 2
            xs = {k: v[:nb] if torch.is_tensor(v) else v for k, v in x.items()}
            args = [np64(xs["tgt"]), np64(xs["drf"]), npi(xs["pos_star"]), npi(xs["prop_pos"]),
                    npi(xs["prop_tok"]), np64(xs["q_pos_star"]), npi(xs["draft_len"]), 1.0, 1.0,
                    np64(xs["u_accept"]), np64(xs["u_resample"])]
            G = np64(xs["gumbel"])
            npos = int(xs["draft_len"].sum())
            t0 = time.perf_counter()
            while True:
                oracle.verify_spot_chain(*args, gumbel=G, tau=SPOT_TAU)
                done_pos += npos
                calls += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            sample = f"{nb} of 16 sequences, {calls} oracle calls"
        elif self.name == "c5ao":
            nb = 4
            args = (np64(x["tgt"][:nb]), npi(x["order"][:nb]), npi(x["num_active"][:nb]),
                    npi(x["positions"][:nb]), npi(x["draft_tokens"][:nb]), np64(x["draft_rows"][:nb]))
            kap = int(self._kappa({k: v[:nb] for k, v in x.items()}).sum())
            t0 = time.perf_counter()
            while True:
                oracle.verify_greedy_any_order(*args)
                done_pos += kap
                calls += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            sample = f"{nb} of 64 sequences, {calls} oracle calls"
        else:
            b = 0
            logits = np64(x["logits"][b:b + 1])
            G = np64(x["gumbel"][b:b + 1])
            m = x["masked"][b:b + 1].numpy()
            ns = npi(x["num_states"][b:b + 1])
            t0 = time.perf_counter()
            while True:
                oracle.verify_gumbel_tree(logits, m, npi(x["parent"][b:b + 1]), npi(x["edge_pos"][b:b + 1]),
                                          npi(x["edge_tok"][b:b + 1]), ns, G, 1.0)
                done_pos += int(ns[0]) - 1
                calls += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            sample = f"1 of 16 trees, {calls} oracle calls"
        dt = time.perf_counter() - t0
        return {"value": done_pos / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
                "sample": f"{sample} in {dt:.1f} s (numpy float64, one thread; host has {os.cpu_count()} cpus)"}


def run_loop(args, dev):
    """The Packed-SS loop workload: every verify call of the loop is timed
    (whole call on the stream, and its row kernel through the timing hook);
    the synthetic model's rows are written between calls and not timed.
    Before each timed call a 2 GiB scratch write pushes the freshly written
    rows out of the caches, so the call reads its inputs from HBM like the
    other workloads; a second pass without it is reported beside."""
    import draft_block_verification_amd as dbv
    from draft_block_verification_amd import _lib
    import workloads
    inp = workloads.config5_loop(device=dev)
    B, W, V, L = inp["B"], inp["W"], inp["V"], inp["L"]
    lib = _lib.load()
    rec = {"ms": [], "kms": [], "pos": 0, "bytes": 0, "calls": 0, "tokens": 0}
    scratch = torch.empty(1 << 30, dtype=torch.int16, device=dev)

    def model(plen, d, n, t):
        return workloads.packed_loop_rows(inp, plen, d, n, t)

    def timed_loop(record, flush=True):
        plen = torch.zeros(B, dtype=torch.int32, device=dev)
        d = torch.full((B, W - 1), -1, dtype=torch.int32, device=dev)
        n = torch.zeros(B, dtype=torch.int32, device=dev)
        done = torch.zeros(B, dtype=torch.bool, device=dev)
        j = torch.arange(W, device=dev)
        for t in range(4 * L):
            if bool(done.all()):
                break
            packed = model(plen, d, n, t)
            budget = torch.where(done, torch.zeros_like(plen), L - plen)
            call = dbv.verify_greedy(packed[:, :W], d, n, packed[:, W:], len_budget=budget, prepare=True)
            if flush:
                scratch.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            k0.record(); k1.record()
            torch.cuda.synchronize()
            lib.verify_set_timing_events(k0._as_parameter_, k1._as_parameter_)
            e0.record()
            r = call()
            e1.record()
            lib.verify_set_timing_events(None, None)
            torch.cuda.synchronize()
            if record:
                rec["ms"].append(e0.elapsed_time(e1))
                rec["kms"].append(k0.elapsed_time(k1))
                nn = n.long()
                rec["pos"] += int(nn.sum())
                rec["bytes"] += int(((nn + 1 + W) * V * 2).sum())
                rec["calls"] += 1
                rec["tokens"] += int(r["num_out"].sum())
            a = r["num_out"]
            plen = plen + a
            done = done | (plen >= L)
            n = torch.where(done, torch.zeros_like(n), r["next_len"])
            d = torch.where(j[None, :W - 1] < n[:, None], r["next_draft"][:, :W - 1], torch.full_like(d, -1))
            if int((r["status"] & dbv.SEQ_ERROR_MASK).sum()):
                print(json.dumps({"error": "verification reported data errors"}))
                sys.exit(1)
        return plen

    timed_loop(False)                     # warm-up: one whole decode
    plen = timed_loop(True)
    ms = sum(rec["ms"]) / rec["calls"]
    kms = sum(rec["kms"])
    achieved = rec["bytes"] / (kms * 1e-3) / 1e9
    flushed = dict(rec)
    rec.update({"ms": [], "kms": [], "pos": 0, "bytes": 0, "calls": 0, "tokens": 0})
    timed_loop(True, flush=False)
    no_flush = {"ms_per_step": sum(rec["ms"]) / rec["calls"],
                "kernel_ms": sum(rec["kms"]) / rec["calls"],
                "frac": rec["bytes"] / (sum(rec["kms"]) * 1e-3) / 1e9 / PEAK_HBM_GBS}
    rec = flushed
    line = {
        "metric": METRIC,
        "value": rec["pos"] / (sum(rec["ms"]) * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": rec["calls"],
        "warmup": rec["calls"],
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": dict(workload=DESCR["c5loop"], B=B, W=W, V=V, L=L, logits="bf16",
                       calls=rec["calls"], tokens=rec["tokens"],
                       tokens_per_call=rec["tokens"] / (rec["calls"] * B),
                       verified_positions=rec["pos"], all_done=bool((plen >= L).all()),
                       rows_still_in_cache=no_flush),
        "roofline": {
            "bound": "hbm",
            "kernel": "k_greedy_rows",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": None,
            "bytes_per_launch": rec["bytes"] / rec["calls"],
            "kernel_ms": kms / rec["calls"],
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle.loop as oloop
        t0 = time.perf_counter()
        nb = 2
        sub = workloads.packed_loop_inputs(51, 64, W, V, L, torch.bfloat16, eps_pct=10)

        def model_nb(pl, dd, nn, t):
            # the oracle loop over the first nb sequences of the same model
            return workloads.packed_loop_rows(sub, torch.as_tensor(pl), torch.as_tensor(dd), torch.as_tensor(nn),
                                              t, seqs=list(range(nb))).double().numpy()
        toks, calls = oloop.packed_ss_greedy(model_nb, nb, W, L, 4 * L)
        dt = time.perf_counter() - t0
        pos = int(sum(int(c["draft_len"].sum()) for c in calls))
        line["cpu_baseline"] = {"value": pos / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
                                "sample": f"the whole loop for {nb} of 64 sequences ({len(calls)} calls) in "
                                          f"{dt:.1f} s (numpy float64, one thread)"}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; runs on several GPUs are not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    import draft_block_verification_amd as dbv
    from draft_block_verification_amd import _lib
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "c5loop":
        run_loop(args, dev)
        return
    steps = args.steps if args.steps is not None else (20 if args.workload == "c4" else 200)
    warmup = args.warmup if args.warmup is not None else (3 if args.workload == "c4" else 20)

    case = Case(args.workload, dev)
    R = case.rotation
    for i in range(warmup):
        case.calls[i % R]()
    torch.cuda.synchronize()

    # Whole-step timing (events on torch's current stream = the launch stream).
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        case.calls[i % R]()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps

    # The row-streaming kernel alone: the library stamps these events at the
    # kernel's own start and end (hipExtLaunchKernel).
    lib = _lib.load()
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in kev:          # create the underlying HIP events (lazy in torch)
        a.record()
        b.record()
    torch.cuda.synchronize()
    for i in range(steps):
        lib.verify_set_timing_events(kev[i][0]._as_parameter_, kev[i][1]._as_parameter_)
        case.calls[i % R]()
    lib.verify_set_timing_events(None, None)
    torch.cuda.synchronize()
    kms = sum(a.elapsed_time(b) for a, b in kev) / steps
    achieved = case.kernel_bytes / (kms * 1e-3) / 1e9

    out = case.calls[0].outputs
    st = out["status"].cpu() if "status" in out else (out["q_nnz"].cpu() < 0).to(torch.int32)
    if int((st & dbv.SEQ_ERROR_MASK).sum()) != 0:
        print(json.dumps({"error": "verification reported data errors", "status": st.tolist()}))
        sys.exit(1)

    line = {
        "metric": METRIC,
        "value": case.positions / (ms * 1e-3),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": dict(workload=DESCR[args.workload], **case.shape,
                       logits="f32" if args.workload == "c1" else "bf16",
                       positions_per_step=case.positions, rotation_sets=R,
                       wall_s=round(wall, 4)),
        "roofline": {
            "bound": "hbm",
            "kernel": case.kernel,
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": measured_traffic(args.workload, case.kernel),
            "bytes_per_launch": case.kernel_bytes,
            "kernel_ms": kms,
        },
        "cpu_baseline": None,
    }
    if args.copy_probe:
        n = COPY_PROBE_BYTES // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_probe_bytes"] = COPY_PROBE_BYTES
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = case.cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of parallel draft-block verification on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]

A step is one verify call over one batch of synthetic inputs already resident
in HBM: every row statistic / argmax, the acceptance tests, the prefix scan,
and the correction or bonus draw.  Workloads (sizes of the pages' setups):

  c1  tiny rejection verify       B=1  K=4  V=1024   fp32
  c2  batch lossless verify       B=8  K=8  V=32000  bf16
  c1r, c2r                        c1 replicated 32768 times and c2 128 times
                                  along B: one call of at least 1 GB
  c3  lenient verify              B=32 K=16 V=128256 bf16, sigma=1, T=1, lambda=0.5
  c4  coupled-Gumbel tree verify  B=16 S=64 L=32 V=151936 bf16   (default: the
                                  largest workload that fits one GPU)
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

Inputs smaller than 2 GiB are replicated into several buffer sets and the
steps rotate over them, so the 256 MiB last-level cache cannot serve them
(one 1.2 GB set read again at every step measured 19% below its bytes in
HBM fetches: the cache kept part of it).
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
ROTATE_BYTES = 2 << 30         # replicate inputs up to this many bytes

DESCR = {
    "c1": "tiny rejection verify B=1 K=4 V=1024 fp32",
    "c1r": "tiny rejection verify replicated R=32768: B=32768 K=4 V=1024 fp32 (1.2 GB per call)",
    "c2r": "batch lossless verify replicated R=128: B=1024 K=8 V=32000 bf16 (1.1 GB per call)",
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
CHAIN = ("c1", "c2", "c3", "c3c", "c1r", "c2r")
REPLICATE = {"c1r": 32768, "c2r": 128}
DD_BUDGET = 20
SPOT_TAU = 0.6
CACTUS_DELTA = 1.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="c4", choices=sorted(DESCR))
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

    def timed(self, begin, end):
        """The first call's row-streaming kernel between the events."""
        self.calls[0].timed(begin, end)
        for c in self.calls[1:]:
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
        if name in CHAIN:
            if name in ("c1", "c1r"):
                x = workloads.config1()
                eb = 4
            elif name in ("c2", "c2r"):
                x = workloads.config2()
            else:
                x = workloads.config3(1.0, 1.0)
            if name in REPLICATE:
                # the batch replicated R times along B: one call of >= 1 GB
                R = REPLICATE[name]
                x = {k: (v.repeat((R,) + (1,) * (v.dim() - 1)) if torch.is_tensor(v) else v)
                     for k, v in x.items()}
            self.lam = 0.5 if name == "c3" else 0.0
            B, K1, V = x["tgt"].shape
            K = K1 - 1
            n = x["draft_len"].long()
            self.positions = int(n.sum())
            self.kernel_bytes = int(((2 * n + 1) * V * eb).sum())      # target n+1 rows, draft n rows
            self.rows = int((2 * n + 1).sum())
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
            self.rows = int((n + 1 + W).sum())
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
            self.rows = int((n + 1).sum())
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
            self.rows = int(n.sum())
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
            self.rows = nm
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
            self.rows = int((2 * n + 1).sum())
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
            self.rows = int((nver + u).sum())
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
            self.rows = int(m.sum())                                   # masked rows of valid states
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
    def cpu_items(self):
        """The oracle's units of work on a bounded sample of this workload:
        (function, items, positions per item).  Items are whole oracle calls
        over one sequence (chains), one block (DDTree) or one tree state
        (the tree: state transitions, the per-state unit the walk then
        combines; a tree's drafted positions are counted per state)."""
        import oracle
        from tests.parity import np64, npi
        x = self.cpu_inputs
        name = self.name
        if name in CHAIN:
            B = min(x["tgt"].shape[0], 64)
            T = x["temperature"]
            tgt, drf = np64(x["tgt"]), np64(x["drf"])
            d, n = npi(x["draft_tokens"]), npi(x["draft_len"])
            ua, ur = np64(x["u_accept"]), np64(x["u_resample"])
            lam = self.lam

            def fn(b):
                sl = slice(b, b + 1)
                if name == "c3c":
                    oracle.verify_cactus(tgt[sl], drf[sl], d[sl], n[sl], T, T, CACTUS_DELTA, ua[sl], ur[sl])
                else:
                    oracle.verify_lenient(tgt[sl], drf[sl], d[sl], n[sl], T, T, lam, ua[sl], ur[sl])
            return fn, list(range(B)), [int(v) for v in n]
        if name == "c5":
            K = x["K"]
            p = x["packed"]
            d, n = npi(x["draft_tokens"]), npi(x["draft_len"])
            nb = 16

            def fn(b):
                oracle.verify_greedy(np64(p[b:b + 1, :K + 1]), d[b:b + 1], n[b:b + 1], np64(p[b:b + 1, K + 1:]))
            return fn, list(range(nb)), [int(v) for v in n[:nb]]
        if name == "c3t":
            n = npi(x["draft_len"])
            nb = 16

            def fn(b):
                oracle.truncate_rows(np64(x["drf"][b:b + 1]), 1.0, x["top_k"], x["top_p"], x["top_k"], n[b:b + 1])
            return fn, list(range(nb)), [int(v) for v in n[:nb]]
        if name == "c4d":
            nb = 16
            tab = np64(x["order_table"])

            def fn(b):
                oracle.build_ddtree(np64(x["stale"][b:b + 1]), npi(x["masked"][b:b + 1]),
                                    oracle.table_order(tab[b:b + 1]), DD_BUDGET, 1.0, gumbel=np64(x["gumbel"][b:b + 1]))
            return fn, list(range(nb)), [DD_BUDGET] * nb
        if name == "c3q":
            B = x["tgt"].shape[0]
            a = dict(tgt=np64(x["tgt"]), qi=npi(x["q_idx"]), qp=np64(x["q_prob"]), qn=npi(x["q_nnz"]),
                     d=npi(x["draft_tokens"]), n=npi(x["draft_len"]), ua=np64(x["u_accept"]),
                     ur=np64(x["u_resample"]))

            def fn(b):
                sl = slice(b, b + 1)
                oracle.verify_sparse(a["tgt"][sl], a["qi"][sl], a["qp"][sl], a["qn"][sl], a["d"][sl], a["n"][sl],
                                     1.0, a["ua"][sl], a["ur"][sl])
            return fn, list(range(B)), [int(v) for v in a["n"]]
        if name == "c4s":
            B = x["tgt"].shape[0]
            a = {k: (np64(v) if v.is_floating_point() else npi(v)) if torch.is_tensor(v) else v
                 for k, v in x.items()}

            def fn(b):
                sl = slice(b, b + 1)
                oracle.verify_spot_chain(a["tgt"][sl], a["drf"][sl], a["pos_star"][sl], a["prop_pos"][sl],
                                         a["prop_tok"][sl], a["q_pos_star"][sl], a["draft_len"][sl], 1.0, 1.0,
                                         a["u_accept"][sl], a["u_resample"][sl], gumbel=a["gumbel"][sl],
                                         tau=SPOT_TAU)
            return fn, list(range(B)), [int(v) for v in a["draft_len"]]
        if name == "c5ao":
            kap = self._kappa(x)
            nb = 16

            def fn(b):
                sl = slice(b, b + 1)
                oracle.verify_greedy_any_order(np64(x["tgt"][sl]), npi(x["order"][sl]), npi(x["num_active"][sl]),
                                               npi(x["positions"][sl]), npi(x["draft_tokens"][sl]),
                                               np64(x["draft_rows"][sl]))
            return fn, list(range(nb)), [int(v) for v in kap[:nb]]
        # c4: the first trees' states (a bounded sample); logits upcast to
        # float32 (exact for bf16) on the host once.
        nt = 2
        logits = x["logits"][:nt].float().cpu().numpy()
        gum = x["gumbel"][:nt].cpu().numpy()
        masked = x["masked"][:nt].cpu().numpy()
        ns = npi(x["num_states"][:nt])
        items = [(b, z) for b in range(nt) for z in range(int(ns[b]))]

        def fn(item):
            b, z = item
            mpos = [s for s in range(masked.shape[2]) if masked[b, z, s]]
            oracle.state_transition(logits[b, z], mpos, gum[b], 1.0)
        # each non-root state is one drafted position of its tree
        return fn, items, [1 if z > 0 else 0 for (_, z) in items]

    def cpu_baseline(self, seconds):
        """The oracle as it stands, on a bounded sample of this workload: on
        one core, then on every core of the host's share (a process pool over
        the same items).  Positions per second of oracle time."""
        fn, items, pos = self.cpu_items()
        one = _time_items(fn, items, pos, seconds / 2, 1)
        # The host's share is 16 CPUs: 15 workers beside this process.
        cores = max(1, min(15, (os.cpu_count() or 2) - 1))
        many = _time_items(fn, items, pos, seconds / 2, cores)
        unit = "positions/s"
        what = {"c4": "tree states", "c4d": "blocks"}.get(self.name, "sequences")
        return {"value": many["rate"], "unit": unit, "cores": many["cores"], "kind": "oracle",
                "sample": f"{len(items)} {what} of the workload, {many['items']} items in {many['s']:.1f} s over "
                          f"{many['cores']} processes (numpy float64)",
                "one_core": {"value": one["rate"], "unit": unit, "cores": 1,
                             "sample": f"{one['items']} items in {one['s']:.1f} s"},
                "host_cpus": os.cpu_count(), "cpu_model": _cpu_model()}


_CPU_WORK = {}


def _cpu_item(i):
    _CPU_WORK["fn"](_CPU_WORK["items"][i])
    return i


def _time_items(fn, items, pos, seconds, cores):
    """Run fn over the items (cycling) for about `seconds`, on `cores`
    processes (forked after the inputs are in memory, so they are shared)."""
    import multiprocessing as mp
    _CPU_WORK["fn"], _CPU_WORK["items"] = fn, items
    done_pos = done = 0
    t0 = time.perf_counter()
    if cores == 1:
        while True:
            for i in range(len(items)):
                fn(items[i])
                done_pos += pos[i]
                done += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            if time.perf_counter() - t0 >= seconds:
                break
    else:
        ctx = mp.get_context("fork")
        with ctx.Pool(cores) as pool:
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < seconds:
                for i in pool.imap_unordered(_cpu_item, range(len(items))):
                    done_pos += pos[i]
                    done += 1
    dt = time.perf_counter() - t0
    return {"rate": done_pos / dt, "items": done, "s": dt, "cores": cores}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def run_loop(args, dev):
    """The Packed-SS loop workload: every verify call of the loop is timed
    (whole call on the stream, and its row kernel through the timing hook);
    the synthetic model's rows are written between calls and not timed.
    Before each timed call a 2 GiB scratch write pushes the freshly written
    rows out of the caches, so the call reads its inputs from HBM like the
    other workloads; a second pass without it is reported beside."""
    import draft_block_verification_amd as dbv
    import workloads
    inp = workloads.config5_loop(device=dev)
    B, W, V, L = inp["B"], inp["W"], inp["V"], inp["L"]
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
            e0.record()
            r = call.timed(k0, k1)
            e1.record()
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
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in kev:          # create the underlying HIP events (lazy in torch)
        a.record()
        b.record()
    torch.cuda.synchronize()
    for i in range(steps):
        case.calls[i % R].timed(kev[i][0], kev[i][1])
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
                       logits="f32" if args.workload in ("c1", "c1r") else "bf16",
                       positions_per_step=case.positions, rows_per_step=case.rows, rotation_sets=R,
                       wall_s=round(wall, 4)),
        "rows_per_s": case.rows / (ms * 1e-3),
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

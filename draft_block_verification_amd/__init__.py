"""Parallel verification of a drafted token block on AMD MI355X (gfx950).

Thin PyTorch binding of libdbv (include/dbv.h): it checks tensor layouts,
allocates outputs and scratch with torch on the tensors' device, and passes
raw device pointers and the current HIP stream to the C ABI.  Every step of
the verification runs in the library's HIP kernels; there is no fallback.

Entry points (same names as the C ABI):
  verify_greedy, verify_rejection, verify_rejection_noalloc, verify_lenient, verify_cactus,
  verify_sparse, truncate_top_k_top_p, verify_spot_chain,
  verify_greedy_any_order, verify_gumbel_tree,
  ddtree_hypotheses, ddtree_level, ddtree_build
"""

import ctypes

import torch

from . import _lib
from ._lib import (  # noqa: F401
    DBV_BF16, DBV_F32, DBV_TREE_FIXED_POSITION, DBV_TREE_STATE_EQUALITY,
    SEQ_BAD_INPUT, SEQ_EMPTY_ROW, SEQ_ERROR_MASK, SEQ_NONFINITE, SEQ_Q_ZERO,
    SEQ_Z_ZERO,
)

__all__ = [
    "verify_greedy", "verify_rejection", "verify_rejection_noalloc", "verify_lenient", "verify_cactus",
    "verify_sparse", "verify_spot_chain", "truncate_top_k_top_p",
    "verify_greedy_any_order", "verify_gumbel_tree", "ddtree_hypotheses", "ddtree_level", "ddtree_build",
    "workspace_size", "DBVError", "Prepared",
]


class Prepared:
    """A verify call whose arguments (pointers, sizes, stream) were marshalled
    once: calling it enqueues the same verification again on the same
    buffers, with no Python-side allocation.  ``outputs`` holds the result
    tensors; ``keep`` keeps every buffer the pointers refer to alive.
    ``options`` (a dbv_options struct, or None) is passed with every call;
    ``timed(begin, end)`` passes the same options plus a pair of timing
    events for this call only."""

    def __init__(self, fn, name, args, outputs, keep, options=None):
        self._fn, self._name, self._args = fn, name, tuple(args)
        self.outputs, self._keep = outputs, keep
        self._opts = options
        self._opts_ref = None if options is None else ctypes.byref(options)

    def __call__(self):
        _check(self._fn(*self._args, self._opts_ref), self._name)
        return self.outputs

    def with_options(self, **fields):
        """The same call with these dbv_options fields set as well (e.g.
        max_groups); the outputs are shared with this call."""
        o = _lib.Options()
        if self._opts is not None:
            ctypes.pointer(o)[0] = self._opts
        for k, v in fields.items():
            setattr(o, k, v)
        return Prepared(self._fn, self._name, self._args, self.outputs, self._keep, o)

    def timed(self, begin, end):
        """Enqueue the call with its row-streaming kernel launched between
        the torch.cuda.Event pair (begin, end), stamped at the kernel's own
        start and end."""
        o = _lib.Options()
        if self._opts is not None:
            ctypes.pointer(o)[0] = self._opts
        o.row_begin, o.row_end = begin.cuda_event, end.cuda_event
        _check(self._fn(*self._args, ctypes.byref(o)), self._name)
        return self.outputs


class DBVError(RuntimeError):
    def __init__(self, code, where):
        super().__init__(f"{where}: {_lib.status_string(code)} (status {code})")
        self.code = code


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return DBV_BF16
    if t.dtype == torch.float32:
        return DBV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _rows3(t, name):
    """A [B, R, V] view with unit vocabulary stride; returns its strides."""
    if t.dim() != 3:
        raise ValueError(f"{name} must be [B, rows, V]")
    if t.stride(2) != 1 and t.size(2) > 1:
        raise ValueError(f"{name} needs a contiguous vocabulary axis")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on a GPU")
    return t.stride(0), t.stride(1)


def _i32(t, shape, name, device):
    if t is None:
        return None
    t = torch.as_tensor(t, dtype=torch.int32, device=device).contiguous()
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}")
    return t


def _f32(t, shape, name, device):
    t = torch.as_tensor(t, dtype=torch.float32, device=device).contiguous()
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}")
    return t


def workspace_size(kind, B, K_or_S, L, V, dtype_code):
    return int(_lib.load().verify_workspace_size(kind, B, K_or_S, L, V, dtype_code))


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _check(code, where):
    if code != _lib.DBV_OK:
        raise DBVError(code, where)


def verify_greedy(tgt, draft_tokens, draft_len=None, draft_rows=None, eos_id=-1,
                  len_budget=None, workspace=None, prepare=False):
    """Greedy verification and next-draft retention (Packed-SS, Algorithm 1).

    tgt [B, K+1, V] and draft_rows [B, W, V] (bf16 or fp32, views allowed),
    draft_tokens [B, K], draft_len [B] or None, len_budget [B] or None.
    Returns a dict of int32 tensors: accept_len, out_tokens, num_out,
    next_draft, next_len, status.  With prepare=True a Prepared call is
    returned instead of running it.
    """
    lib = _lib.load()
    dev = tgt.device
    B, K1, V = tgt.shape
    K = K1 - 1
    ts, tr = _rows3(tgt, "tgt")
    dt = _dtype_code(tgt)
    W = 0
    ds = drs = 0
    if draft_rows is not None:
        if draft_rows.dtype != tgt.dtype or draft_rows.shape[0] != B or draft_rows.shape[2] != V:
            raise ValueError("draft_rows must be [B, W, V] with the dtype of tgt")
        ds, drs = _rows3(draft_rows, "draft_rows")
        W = draft_rows.shape[1]
    d = _i32(draft_tokens, (B, K), "draft_tokens", dev)
    n = _i32(draft_len, (B,), "draft_len", dev)
    bud = _i32(len_budget, (B,), "len_budget", dev)
    out = {
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "out_tokens": torch.empty(B, K + 1, dtype=torch.int32, device=dev),
        "num_out": torch.empty(B, dtype=torch.int32, device=dev),
        "next_draft": torch.empty(B, W, dtype=torch.int32, device=dev),
        "next_len": torch.empty(B, dtype=torch.int32, device=dev),
        "status": torch.empty(B, dtype=torch.int32, device=dev),
    }
    need = workspace_size(_lib.DBV_KIND_GREEDY, B, K, W, V, dt)
    ws = workspace if workspace is not None else _workspace(need, dev)
    args = (B, K, V, dt, tgt.data_ptr(), ts, tr, _ptr(d), _ptr(n),
            _ptr(draft_rows), ds, drs, W, int(eos_id), _ptr(bud),
            out["accept_len"].data_ptr(), out["out_tokens"].data_ptr(), out["num_out"].data_ptr(),
            out["next_draft"].data_ptr() if W else None, out["next_len"].data_ptr(),
            out["status"].data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    call = Prepared(lib.verify_greedy, "verify_greedy", args, out, (tgt, draft_rows, d, n, bud, ws))
    return call if prepare else call()


def _chain_margins(out, B, K, dev, margins, row_tv=False):
    """Optional diagnostics of a chain sampling call: the per-decision
    margins (dbv_options accept_margin [B, K], draw_margin [B]) and the
    per-row TV(p, q) (row_tv [B, K]); returns the options or None."""
    if not margins and not row_tv:
        return None
    o = _lib.Options()
    if margins:
        out["accept_margin"] = torch.empty(B, K, dtype=torch.float32, device=dev)
        out["draw_margin"] = torch.empty(B, dtype=torch.float32, device=dev)
        o.accept_margin, o.draw_margin = out["accept_margin"].data_ptr(), out["draw_margin"].data_ptr()
    if row_tv:
        out["row_tv"] = torch.empty(B, K, dtype=torch.float32, device=dev)
        o.row_tv = out["row_tv"].data_ptr()
    return o


def _sampling(fn_name, tgt, drf, draft_tokens, draft_len, temperature_target,
              temperature_draft, lam, u_accept, u_resample, eos_id, len_budget,
              workspace, diagnostics, prepare, margins=False, noalloc=False, row_tv=False):
    lib = _lib.load()
    dev = tgt.device
    B, K1, V = tgt.shape
    K = K1 - 1
    ts, tr = _rows3(tgt, "tgt")
    dt = _dtype_code(tgt)
    if drf.dtype != tgt.dtype or tuple(drf.shape) != (B, K, V):
        raise ValueError("drf must be [B, K, V] with the dtype of tgt")
    ds, dr = _rows3(drf, "drf")
    d = _i32(draft_tokens, (B, K), "draft_tokens", dev)
    n = _i32(draft_len, (B,), "draft_len", dev)
    bud = _i32(len_budget, (B,), "len_budget", dev)
    ua = _f32(u_accept, (B, K), "u_accept", dev)
    ur = _f32(u_resample, (B, K + 1), "u_resample", dev)
    out = {
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "out_tokens": torch.empty(B, K + 1, dtype=torch.int32, device=dev),
        "num_out": torch.empty(B, dtype=torch.int32, device=dev),
        "status": torch.empty(B, dtype=torch.int32, device=dev),
    }
    if diagnostics:
        for k in ("p_draft", "q_draft", "alpha"):
            out[k] = torch.empty(B, K, dtype=torch.float32, device=dev)
        out["residual_mass"] = torch.empty(B, dtype=torch.float32, device=dev)
    args = [B, K, V, dt, tgt.data_ptr(), ts, tr, drf.data_ptr(), ds, dr, _ptr(d), _ptr(n),
            float(temperature_target), float(temperature_draft)]
    if fn_name in ("verify_lenient", "verify_cactus"):
        args.append(float(lam))
    args += [ua.data_ptr() if K else None, ur.data_ptr(), int(eos_id), _ptr(bud),
             out["accept_len"].data_ptr(), out["out_tokens"].data_ptr(), out["num_out"].data_ptr(),
             _ptr(out.get("p_draft")), _ptr(out.get("q_draft")), _ptr(out.get("alpha")),
             _ptr(out.get("residual_mass")), out["status"].data_ptr()]
    ws = None
    if noalloc:
        fn_name = "verify_rejection_noalloc"
    else:
        need = workspace_size(_lib.DBV_KIND_REJECTION, B, K, 0, V, dt)
        ws = workspace if workspace is not None else _workspace(need, dev)
        args += [ws.data_ptr(), ws.numel()]
    args.append(_stream(dev))
    opts = _chain_margins(out, B, K, dev, margins, row_tv)
    call = Prepared(getattr(lib, fn_name), fn_name, tuple(args), out,
                    (tgt, drf, d, n, bud, ua, ur, ws), opts)
    return call if prepare else call()


def verify_rejection(tgt, drf, draft_tokens, u_accept, u_resample, draft_len=None,
                     temperature_target=1.0, temperature_draft=1.0, eos_id=-1,
                     len_budget=None, workspace=None, diagnostics=True, prepare=False, margins=False,
                     row_tv=False):
    """Lossless rejection-sampling verification (Packed-SS, Algorithm 2).

    tgt [B, K+1, V], drf [B, K, V] (same dtype), draft_tokens [B, K],
    u_accept [B, K], u_resample [B, K+1].  Returns accept_len, out_tokens,
    num_out, status and (with diagnostics) p_draft, q_draft, alpha,
    residual_mass; with margins also accept_margin [B, K] and draw_margin
    [B], the per-decision margins of dbv_options; with row_tv the per-row
    TV(p_i, q_i) [B, K] (diagnostic mode, one more pass over the rows).
    """
    return _sampling("verify_rejection", tgt, drf, draft_tokens, draft_len,
                     temperature_target, temperature_draft, 0.0, u_accept, u_resample,
                     eos_id, len_budget, workspace, diagnostics, prepare, margins, row_tv=row_tv)


def verify_rejection_noalloc(tgt, drf, draft_tokens, u_accept, u_resample, draft_len=None,
                             temperature_target=1.0, temperature_draft=1.0, eos_id=-1,
                             len_budget=None, diagnostics=True, prepare=False, margins=False):
    """verify_rejection through the entry point that allocates nothing: its
    scratch is the library's own device array (at most 4 MiB of workspace;
    calls that overlap on one GPU race).  Outputs as verify_rejection."""
    return _sampling("verify_rejection", tgt, drf, draft_tokens, draft_len,
                     temperature_target, temperature_draft, 0.0, u_accept, u_resample,
                     eos_id, len_budget, None, diagnostics, prepare, margins, noalloc=True)


def verify_lenient(tgt, drf, draft_tokens, u_accept, u_resample, lam, draft_len=None,
                   temperature_target=1.0, temperature_draft=1.0, eos_id=-1,
                   len_budget=None, workspace=None, diagnostics=True, prepare=False, margins=False,
                   row_tv=False):
    """Linear lenient verification, p~ = (1 - lam) p + lam q (Two Tradeoffs,
    Theorem 1 and Algorithm 1).  Arguments as verify_rejection plus lam."""
    return _sampling("verify_lenient", tgt, drf, draft_tokens, draft_len,
                     temperature_target, temperature_draft, lam, u_accept, u_resample,
                     eos_id, len_budget, workspace, diagnostics, prepare, margins, row_tv=row_tv)


def verify_cactus(tgt, drf, draft_tokens, u_accept, u_resample, delta, draft_len=None,
                  temperature_target=1.0, temperature_draft=1.0, eos_id=-1,
                  len_budget=None, workspace=None, diagnostics=True, prepare=False, margins=False,
                  row_tv=False):
    """Verification with the modified Cactus rule (Two Tradeoffs, App. E):
    the drafted token's target mass is raised to the largest gamma whose
    rescaled target stays within KL budget delta of p.  Arguments as
    verify_rejection plus delta >= 0 (0 = lossless)."""
    return _sampling("verify_cactus", tgt, drf, draft_tokens, draft_len,
                     temperature_target, temperature_draft, delta, u_accept, u_resample,
                     eos_id, len_budget, workspace, diagnostics, prepare, margins, row_tv=row_tv)


def verify_sparse(tgt, q_idx, q_prob, q_nnz, draft_tokens, u_accept, u_resample, draft_len=None,
                  temperature_target=1.0, eos_id=-1, len_budget=None, workspace=None, diagnostics=True,
                  prepare=False, margins=False, row_tv=False):
    """Lossless verification against stored sparse drafter distributions
    (Packed-SS Sec. 3.2: only Q's nonzero entries are stored under top-k /
    top-p truncation).

    tgt [B, K+1, V]; q_idx [B, K, kmax] int, q_prob [B, K, kmax] float32,
    q_nnz [B, K] (entries in use per row); draft_tokens [B, K]; u_accept
    [B, K]; u_resample [B, K+1].  Outputs as verify_rejection.
    """
    lib = _lib.load()
    dev = tgt.device
    B, K1, V = tgt.shape
    K = K1 - 1
    ts, tr = _rows3(tgt, "tgt")
    dt = _dtype_code(tgt)
    kmax = int(torch.as_tensor(q_idx).shape[-1]) if K > 0 else 0
    qi = _i32(q_idx, (B, K, kmax), "q_idx", dev)
    qp = _f32(q_prob, (B, K, kmax), "q_prob", dev)
    qn = _i32(q_nnz, (B, K), "q_nnz", dev)
    d = _i32(draft_tokens, (B, K), "draft_tokens", dev)
    n = _i32(draft_len, (B,), "draft_len", dev)
    bud = _i32(len_budget, (B,), "len_budget", dev)
    ua = _f32(u_accept, (B, K), "u_accept", dev)
    ur = _f32(u_resample, (B, K + 1), "u_resample", dev)
    out = {
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "out_tokens": torch.empty(B, K + 1, dtype=torch.int32, device=dev),
        "num_out": torch.empty(B, dtype=torch.int32, device=dev),
        "status": torch.empty(B, dtype=torch.int32, device=dev),
    }
    if diagnostics:
        for k in ("p_draft", "q_draft", "alpha"):
            out[k] = torch.empty(B, K, dtype=torch.float32, device=dev)
        out["residual_mass"] = torch.empty(B, dtype=torch.float32, device=dev)
    need = workspace_size(_lib.DBV_KIND_REJECTION, B, K, 0, V, dt)
    ws = workspace if workspace is not None else _workspace(need, dev)
    args = (B, K, V, dt, tgt.data_ptr(), ts, tr, _ptr(qi), _ptr(qp), _ptr(qn), kmax, _ptr(d), _ptr(n),
            float(temperature_target), _ptr(ua), ur.data_ptr(), int(eos_id), _ptr(bud),
            out["accept_len"].data_ptr(), out["out_tokens"].data_ptr(), out["num_out"].data_ptr(),
            _ptr(out.get("p_draft")), _ptr(out.get("q_draft")), _ptr(out.get("alpha")),
            _ptr(out.get("residual_mass")), out["status"].data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    opts = _chain_margins(out, B, K, dev, margins, row_tv)
    call = Prepared(lib.verify_sparse, "verify_sparse", args, out, (tgt, qi, qp, qn, d, n, bud, ua, ur, ws), opts)
    return call if prepare else call()


def truncate_top_k_top_p(rows, top_k, top_p=1.0, kmax=None, lengths=None, temperature=1.0, prepare=False):
    """Top-k / top-p truncation of drafter rows [B, K, V] into the stored
    sparse form verify_sparse reads (Packed-SS Sec. 3.2).  Returns q_idx
    [B, K, kmax] int32, q_prob [B, K, kmax] float32 and q_nnz [B, K] int32
    (-1 for a row that is not a distribution; entries past q_nnz are 0)."""
    lib = _lib.load()
    dev = rows.device
    B, K, V = rows.shape
    ss, rs = _rows3(rows, "rows")
    dt = _dtype_code(rows)
    kmax = int(top_k) if kmax is None else int(kmax)
    n = _i32(lengths, (B,), "lengths", dev)
    out = {
        "q_idx": torch.zeros(B, K, kmax, dtype=torch.int32, device=dev),
        "q_prob": torch.zeros(B, K, kmax, dtype=torch.float32, device=dev),
        "q_nnz": torch.empty(B, K, dtype=torch.int32, device=dev),
    }
    args = (B, K, V, dt, rows.data_ptr(), ss, rs, _ptr(n), float(temperature), int(top_k), float(top_p), kmax,
            out["q_idx"].data_ptr(), out["q_prob"].data_ptr(), out["q_nnz"].data_ptr(), _stream(dev))
    call = Prepared(lib.truncate_top_k_top_p, "truncate_top_k_top_p", args, out, (rows, n))
    return call if prepare else call()


def verify_spot_chain(tgt, drf, pos_star, prop_pos, prop_tok, q_pos_star, u_accept, u_resample,
                      gumbel=None, tau=0.6, draft_len=None, temperature_target=1.0, temperature_draft=1.0,
                      eos_id=-1, len_budget=None, workspace=None, diagnostics=True, prepare=False,
                      margins=False, row_tv=False):
    """Chain verification on the joint (position, token) space (SPOT App. B,
    Eq. 10-14), gated per link between rejection sampling and coupled-noise
    match when Gumbel rows are given (match where the drafter's confidence
    at the link reaches tau).

    tgt [B, K+1, V] target rows at each link's position s*; drf [B, K, V]
    drafter rows at s*; pos_star [B, K+1]; prop_pos, prop_tok [B, K];
    q_pos_star [B, K] (the drafter's probability of s*); u_accept [B, K];
    u_resample [B, K+1]; gumbel [B, K+1, V] float32 or None.  Outputs as
    verify_rejection.
    """
    lib = _lib.load()
    dev = tgt.device
    B, K1, V = tgt.shape
    K = K1 - 1
    ts, tr = _rows3(tgt, "tgt")
    dt = _dtype_code(tgt)
    if drf.dtype != tgt.dtype or tuple(drf.shape) != (B, K, V):
        raise ValueError("drf must be [B, K, V] with the dtype of tgt")
    ds, dr = _rows3(drf, "drf")
    gs = gr = 0
    if gumbel is not None:
        if gumbel.dtype != torch.float32 or tuple(gumbel.shape) != (B, K + 1, V):
            raise ValueError("gumbel must be float32 [B, K+1, V]")
        gs, gr = _rows3(gumbel, "gumbel")
    ps = _i32(pos_star, (B, K + 1), "pos_star", dev)
    pp = _i32(prop_pos, (B, K), "prop_pos", dev)
    d = _i32(prop_tok, (B, K), "prop_tok", dev)
    c = _f32(q_pos_star, (B, K), "q_pos_star", dev)
    n = _i32(draft_len, (B,), "draft_len", dev)
    bud = _i32(len_budget, (B,), "len_budget", dev)
    ua = _f32(u_accept, (B, K), "u_accept", dev)
    ur = _f32(u_resample, (B, K + 1), "u_resample", dev)
    out = {
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "out_tokens": torch.empty(B, K + 1, dtype=torch.int32, device=dev),
        "num_out": torch.empty(B, dtype=torch.int32, device=dev),
        "status": torch.empty(B, dtype=torch.int32, device=dev),
    }
    if diagnostics:
        for k in ("p_draft", "q_draft", "alpha"):
            out[k] = torch.empty(B, K, dtype=torch.float32, device=dev)
        out["residual_mass"] = torch.empty(B, dtype=torch.float32, device=dev)
    need = workspace_size(_lib.DBV_KIND_REJECTION, B, K, 0, V, dt)
    ws = workspace if workspace is not None else _workspace(need, dev)
    args = (B, K, V, dt, tgt.data_ptr(), ts, tr, drf.data_ptr(), ds, dr, _ptr(ps), _ptr(pp), _ptr(d), _ptr(c),
            _ptr(n), float(temperature_target), float(temperature_draft), _ptr(gumbel), gs, gr, float(tau),
            _ptr(ua), ur.data_ptr(), int(eos_id), _ptr(bud), out["accept_len"].data_ptr(),
            out["out_tokens"].data_ptr(), out["num_out"].data_ptr(), _ptr(out.get("p_draft")),
            _ptr(out.get("q_draft")), _ptr(out.get("alpha")), _ptr(out.get("residual_mass")),
            out["status"].data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    opts = _chain_margins(out, B, K, dev, margins, row_tv)
    call = Prepared(lib.verify_spot_chain, "verify_spot_chain", args, out,
                    (tgt, drf, gumbel, ps, pp, d, c, n, bud, ua, ur, ws), opts)
    return call if prepare else call()


def verify_greedy_any_order(tgt, order, draft_tokens, num_active=None, positions=None,
                            draft_rows=None, eos_id=-1, end_pos=None, workspace=None, prepare=False):
    """One any-order greedy verification call (Packed-SS, App. C, Algorithm 3).

    tgt [B, U, V] verifier rows in rank order; order [B, U] (slot checked at
    rank r); draft_tokens [B, U] by slot (-1 = missing); num_active [B] or
    None; positions [B, U] or None; draft_rows [B, U, V] by slot or None;
    end_pos [B] or None.  Returns accept_len, num_accepted, acc_pos, acc_tok,
    new_end, next_draft, status (int32).
    """
    lib = _lib.load()
    dev = tgt.device
    B, U, V = tgt.shape
    ts, tr = _rows3(tgt, "tgt")
    dt = _dtype_code(tgt)
    ds = drs = 0
    if draft_rows is not None:
        if draft_rows.dtype != tgt.dtype or tuple(draft_rows.shape) != (B, U, V):
            raise ValueError("draft_rows must be [B, U, V] with the dtype of tgt")
        ds, drs = _rows3(draft_rows, "draft_rows")
    o = _i32(order, (B, U), "order", dev)
    d = _i32(draft_tokens, (B, U), "draft_tokens", dev)
    na = _i32(num_active, (B,), "num_active", dev)
    ps = _i32(positions, (B, U), "positions", dev)
    ep = _i32(end_pos, (B,), "end_pos", dev)
    out = {
        "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
        "num_accepted": torch.empty(B, dtype=torch.int32, device=dev),
        "acc_pos": torch.empty(B, U, dtype=torch.int32, device=dev),
        "acc_tok": torch.empty(B, U, dtype=torch.int32, device=dev),
        "new_end": torch.empty(B, dtype=torch.int32, device=dev),
        "next_draft": torch.empty(B, U, dtype=torch.int32, device=dev),
        "status": torch.empty(B, dtype=torch.int32, device=dev),
    }
    need = workspace_size(_lib.DBV_KIND_ANY_ORDER, B, U, 0, V, dt)
    ws = workspace if workspace is not None else _workspace(need, dev)
    args = (B, U, V, dt, tgt.data_ptr(), ts, tr, _ptr(o), _ptr(na), _ptr(ps), _ptr(d),
            _ptr(draft_rows), ds, drs, int(eos_id), _ptr(ep),
            out["accept_len"].data_ptr(), out["num_accepted"].data_ptr(), out["acc_pos"].data_ptr(),
            out["acc_tok"].data_ptr(), out["new_end"].data_ptr(), out["next_draft"].data_ptr(),
            out["status"].data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    call = Prepared(lib.verify_greedy_any_order, "verify_greedy_any_order", args, out,
                    (tgt, draft_rows, o, d, na, ps, ep, ws))
    return call if prepare else call()


def verify_gumbel_tree(logits, parent, edge_pos, edge_tok, masked=None, gumbel=None,
                       temperature=1.0, num_states=None, next_pos=None,
                       mode=DBV_TREE_STATE_EQUALITY, workspace=None, prepare=False, margins=False):
    """Shared-Gumbel state-equality verification of a draft tree (SPOT,
    Sec. 4.3, App. A.1).

    logits [B, S, L, V] (vocabulary contiguous), masked [B, S, L] bool/uint8,
    parent / edge_pos / edge_tok [B, S], gumbel [B, L, V] float32 (None at
    temperature 0), num_states [B] or None, next_pos [B, S] in the
    fixed-position mode.  Returns sel_pos, sel_tok, sel_conf, path_len,
    path_nodes, commit_pos, commit_tok, num_commits, status; with margins
    also pos_margin and tok_margin [B, S] (dbv_options).
    """
    lib = _lib.load()
    dev = logits.device
    if logits.dim() != 4 or (logits.stride(3) != 1 and logits.size(3) > 1) or not logits.is_cuda:
        raise ValueError("logits must be a GPU tensor [B, S, L, V] with a contiguous vocabulary axis")
    B, S, L, V = logits.shape
    dt = _dtype_code(logits)
    par = _i32(parent, (B, S), "parent", dev)
    ep = _i32(edge_pos, (B, S), "edge_pos", dev)
    et = _i32(edge_tok, (B, S), "edge_tok", dev)
    ns = _i32(num_states, (B,), "num_states", dev)
    npos = _i32(next_pos, (B, S), "next_pos", dev)
    m = None
    if masked is not None:
        m = torch.as_tensor(masked, device=dev).to(torch.uint8).contiguous()
        if tuple(m.shape) != (B, S, L):
            raise ValueError("masked must be [B, S, L]")
    gs = gp = 0
    if gumbel is not None:
        if gumbel.dtype != torch.float32 or gumbel.dim() != 3 or gumbel.shape[0] != B \
                or gumbel.shape[1] != L or gumbel.shape[2] != V or gumbel.stride(2) != 1:
            raise ValueError("gumbel must be float32 [B, L, V] with a contiguous vocabulary axis")
        gs, gp = gumbel.stride(0), gumbel.stride(1)
    out = {
        "sel_pos": torch.empty(B, S, dtype=torch.int32, device=dev),
        "sel_tok": torch.empty(B, S, dtype=torch.int32, device=dev),
        "sel_conf": torch.empty(B, S, dtype=torch.float32, device=dev),
        "path_len": torch.empty(B, dtype=torch.int32, device=dev),
        "path_nodes": torch.empty(B, S, dtype=torch.int32, device=dev),
        "commit_pos": torch.empty(B, S, dtype=torch.int32, device=dev),
        "commit_tok": torch.empty(B, S, dtype=torch.int32, device=dev),
        "num_commits": torch.empty(B, dtype=torch.int32, device=dev),
        "status": torch.empty(B, dtype=torch.int32, device=dev),
    }
    need = workspace_size(_lib.DBV_KIND_TREE, B, S, L, V, dt)
    ws = workspace if workspace is not None else _workspace(need, dev)
    args = (B, S, L, V, dt, logits.data_ptr(), logits.stride(0), logits.stride(1), logits.stride(2),
            _ptr(m), par.data_ptr(), ep.data_ptr(), et.data_ptr(), _ptr(ns), _ptr(npos),
            _ptr(gumbel), gs, gp, float(temperature), int(mode),
            out["sel_pos"].data_ptr(), out["sel_tok"].data_ptr(), out["sel_conf"].data_ptr(),
            out["path_len"].data_ptr(), out["path_nodes"].data_ptr(), out["commit_pos"].data_ptr(),
            out["commit_tok"].data_ptr(), out["num_commits"].data_ptr(), out["status"].data_ptr(),
            ws.data_ptr(), ws.numel(), _stream(dev))
    opts = None
    if margins:
        out["pos_margin"] = torch.empty(B, S, dtype=torch.float32, device=dev)
        out["tok_margin"] = torch.empty(B, S, dtype=torch.float32, device=dev)
        opts = _lib.Options(pos_margin=out["pos_margin"].data_ptr(), tok_margin=out["tok_margin"].data_ptr())
    call = Prepared(lib.verify_gumbel_tree, "verify_gumbel_tree", args, out,
                    (logits, m, par, ep, et, ns, npos, gumbel, ws), opts)
    return call if prepare else call()


def ddtree_hypotheses(stale, masked, temperature=0.0, gumbel=None, runner_up_below=0.6, workspace=None,
                      prepare=False):
    """Token hypotheses of the masked positions (SPOT Sec. 4.2, Eq. 4).

    stale [B, L, V] stale target logits (bf16 or fp32), masked [B, L];
    gumbel [B, L, V] float32 when temperature > 0.  Returns hyp_tok [B, L, 2]
    int32, hyp_prob [B, L, 2] float32 and status [B] int32."""
    lib = _lib.load()
    dev = stale.device
    B, L, V = stale.shape
    ss, sp = _rows3(stale, "stale")
    dt = _dtype_code(stale)
    m = torch.as_tensor(masked, device=dev).to(torch.uint8).contiguous()
    if tuple(m.shape) != (B, L):
        raise ValueError("masked must be [B, L]")
    gs = gp = 0
    if temperature > 0:
        if gumbel is None or gumbel.dtype != torch.float32 or tuple(gumbel.shape) != (B, L, V):
            raise ValueError("gumbel must be float32 [B, L, V] when temperature > 0")
        gs, gp = _rows3(gumbel, "gumbel")
    else:
        gumbel = None
    out = {
        "hyp_tok": torch.empty(B, L, 2, dtype=torch.int32, device=dev),
        "hyp_prob": torch.empty(B, L, 2, dtype=torch.float32, device=dev),
        "status": torch.empty(B, dtype=torch.int32, device=dev),
    }
    need = workspace_size(_lib.DBV_KIND_DDTREE_HYPOTHESES, B, L, 0, V, dt)
    ws = workspace if workspace is not None else _workspace(need, dev)
    args = (B, L, V, dt, stale.data_ptr(), ss, sp, m.data_ptr(), _ptr(gumbel), gs, gp, float(temperature),
            float(runner_up_below), out["hyp_tok"].data_ptr(), out["hyp_prob"].data_ptr(),
            out["status"].data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    call = Prepared(lib.ddtree_hypotheses, "ddtree_hypotheses", args, out, (stale, m, gumbel, ws))
    return call if prepare else call()


def _dd_state(B, L, D, dev, status):
    st = {
        "parent": torch.empty(B, D + 1, dtype=torch.int32, device=dev),
        "edge_pos": torch.empty(B, D + 1, dtype=torch.int32, device=dev),
        "edge_tok": torch.empty(B, D + 1, dtype=torch.int32, device=dev),
        "mass": torch.empty(B, D + 1, dtype=torch.float32, device=dev),
        "node_masked": torch.empty(B, D + 1, L, dtype=torch.uint8, device=dev),
        "num_nodes": torch.empty(B, dtype=torch.int32, device=dev),
        "frontier": torch.empty(B, max(D, 1), dtype=torch.int32, device=dev),
        "num_frontier": torch.empty(B, dtype=torch.int32, device=dev),
        "status": (torch.zeros(B, dtype=torch.int32, device=dev) if status is None
                   else _i32(status, (B,), "status", dev)),
    }
    st["_ws"] = _workspace(workspace_size(_lib.DBV_KIND_DDTREE, B, D, L, 0, 0), dev)
    return st


def _dd_inputs(masked, hyp_tok, hyp_prob, dev):
    m = torch.as_tensor(masked, device=dev).to(torch.uint8).contiguous()
    B, L = m.shape
    ht = _i32(hyp_tok, (B, L, 2), "hyp_tok", dev)
    hp = _f32(hyp_prob, (B, L, 2), "hyp_prob", dev)
    return m, ht, hp, B, L


def _dd_out_ptrs(st):
    return (st["parent"].data_ptr(), st["edge_pos"].data_ptr(), st["edge_tok"].data_ptr(), st["mass"].data_ptr(),
            st["node_masked"].data_ptr(), st["num_nodes"].data_ptr(), st["frontier"].data_ptr(),
            st["num_frontier"].data_ptr(), st["status"].data_ptr(), st["_ws"].data_ptr(), st["_ws"].numel())


def ddtree_level(masked, hyp_tok, hyp_prob, order_logits, D, tau=1.0, gamma=0.0, state=None, status=None):
    """One level of the DDTree search (SPOT App. C.2, Algorithm 2).

    masked [B, L] the current state's masked positions; hyp_tok / hyp_prob
    from ddtree_hypotheses; order_logits [B, F, L] float32, row j = the
    order model's logits for frontier slot j (the root on the first level).
    state=None starts a new search (status [B], e.g. the hypotheses' own,
    is read and updated in place: a sequence in error is skipped); pass the
    returned state back for the next level.  The
    state dict holds parent, edge_pos, edge_tok, mass, node_masked,
    num_nodes, frontier, num_frontier and status."""
    lib = _lib.load()
    dev = order_logits.device
    m, ht, hp, B, L = _dd_inputs(masked, hyp_tok, hyp_prob, dev)
    o = order_logits
    if o.dtype != torch.float32 or o.dim() != 3 or o.shape[0] != B or o.shape[2] != L or o.stride(2) != 1:
        raise ValueError("order_logits must be float32 [B, F, L] with a contiguous last axis")
    first = state is None
    if o.shape[1] < (1 if first else D):
        raise ValueError("order_logits needs a row per frontier slot: 1 on the first level, D after")
    st = _dd_state(B, L, D, dev, status) if first else state
    args = (B, L, D, m.data_ptr(), ht.data_ptr(), hp.data_ptr(), o.data_ptr(), o.stride(0), o.stride(1),
            float(tau), float(gamma), int(first)) + _dd_out_ptrs(st) + (_stream(dev),)
    _check(lib.ddtree_level(*args, None), "ddtree_level")
    st["_keep"] = (m, ht, hp, o)
    return st


def ddtree_build(masked, hyp_tok, hyp_prob, order_table, D, tau=1.0, gamma=0.0, status=None, prepare=False):
    """The whole DDTree search in one launch with a first-order order
    model: order_table [B, L+1, L] float32, row c = the order logits of a
    state whose last committed position is c (row L: the root).  Returns the
    state dict of ddtree_level after its last level."""
    lib = _lib.load()
    dev = order_table.device
    m, ht, hp, B, L = _dd_inputs(masked, hyp_tok, hyp_prob, dev)
    o = order_table
    if o.dtype != torch.float32 or tuple(o.shape) != (B, L + 1, L) or o.stride(2) != 1:
        raise ValueError("order_table must be float32 [B, L+1, L] with a contiguous last axis")
    st = _dd_state(B, L, D, dev, status)
    args = (B, L, D, m.data_ptr(), ht.data_ptr(), hp.data_ptr(), o.data_ptr(), o.stride(0), o.stride(1),
            float(tau), float(gamma)) + _dd_out_ptrs(st) + (_stream(dev),)
    call = Prepared(lib.ddtree_build, "ddtree_build", args, st, (m, ht, hp, o))
    return call if prepare else call()

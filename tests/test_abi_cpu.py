"""C-ABI checks that need no GPU: the library loads, exports every entry
point declared in include/dbv.h, sizes workspaces and rejects invalid host
arguments before launching anything."""

import ctypes
import os
import re

import pytest

from draft_block_verification_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dbv.h")

FAKE = 0x10000  # a 256-byte aligned non-null address; never dereferenced here


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?:dbv_status|size_t|const char\s*\*|int|void)\s+(\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libdbv.so not built")
    return _lib.load()


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def test_exports_match_header(lib):
    declared = _declared_functions()
    assert declared == sorted(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_strings(lib):
    assert lib.verify_abi_version() == 2
    for code in range(6):
        assert lib.verify_status_string(code)
    assert b"unknown" in lib.verify_status_string(99)


def test_workspace_sizes(lib):
    g = lib.verify_workspace_size(_lib.DBV_KIND_GREEDY, 64, 31, 32, 131072, _lib.DBV_BF16)
    assert g >= 64 * (32 + 32) * 8 and g % 256 == 0
    r = lib.verify_workspace_size(_lib.DBV_KIND_REJECTION, 32, 16, 0, 128256, _lib.DBV_BF16)
    assert r > 0 and r % 256 == 0
    t = lib.verify_workspace_size(_lib.DBV_KIND_TREE, 16, 64, 32, 151936, _lib.DBV_BF16)
    assert t >= 16 * 64 * 32 * 8
    assert lib.verify_workspace_size(_lib.DBV_KIND_TREE, 16, 0, 32, 100, 1) == 0
    assert lib.verify_workspace_size(_lib.DBV_KIND_GREEDY, 1, -1, 0, 100, 1) == 0
    assert lib.verify_workspace_size(_lib.DBV_KIND_GREEDY, 1, 4, 0, 0, 1) == 0
    assert lib.verify_workspace_size(_lib.DBV_KIND_GREEDY, 1, 4, 0, 10, 7) == 0
    a = lib.verify_workspace_size(_lib.DBV_KIND_ANY_ORDER, 64, 32, 0, 131072, _lib.DBV_BF16)
    assert a >= 64 * 64 * 8 * 4 and a % 256 == 0
    assert lib.verify_workspace_size(_lib.DBV_KIND_ANY_ORDER, 1, 2000, 0, 100, 1) == 0


def _greedy(lib, **kw):
    a = dict(B=2, K=3, V=100, dt=_lib.DBV_BF16, tgt=FAKE, ts=400, tr=100, d=FAKE, n=None,
             dr=FAKE, ds=400, drs=100, W=4, eos=-1, bud=None, acc=FAKE, out=FAKE, num=FAKE,
             nd=FAKE, nl=FAKE, st=FAKE, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.verify_greedy(a["B"], a["K"], a["V"], a["dt"], a["tgt"], a["ts"], a["tr"], a["d"],
                             a["n"], a["dr"], a["ds"], a["drs"], a["W"], a["eos"], a["bud"],
                             a["acc"], a["out"], a["num"], a["nd"], a["nl"], a["st"], a["ws"],
                             a["wsb"], a["stream"], a.get("opts"))


def _reject(lib, lenient=False, cactus=False, **kw):
    a = dict(B=2, K=3, V=100, dt=_lib.DBV_BF16, tgt=FAKE, ts=400, tr=100, drf=FAKE, ds=300,
             dr=100, d=FAKE, n=None, tt=1.0, td=1.0, lam=0.5, delta=1.0, ua=FAKE, ur=FAKE, eos=-1, bud=None,
             acc=FAKE, out=FAKE, num=FAKE, pd=None, qd=None, al=None, rm=None, st=FAKE, ws=FAKE,
             wsb=1 << 20, stream=None)
    a.update(kw)
    head = [a["B"], a["K"], a["V"], a["dt"], a["tgt"], a["ts"], a["tr"], a["drf"], a["ds"], a["dr"],
            a["d"], a["n"], a["tt"], a["td"]]
    tail = [a["ua"], a["ur"], a["eos"], a["bud"], a["acc"], a["out"], a["num"], a["pd"], a["qd"],
            a["al"], a["rm"], a["st"], a["ws"], a["wsb"], a["stream"], a.get("opts")]
    if lenient:
        return lib.verify_lenient(*(head + [a["lam"]] + tail))
    if cactus:
        return lib.verify_cactus(*(head + [a["delta"]] + tail))
    return lib.verify_rejection(*(head + tail))


def _tree(lib, **kw):
    a = dict(B=2, S=8, L=4, V=100, dt=_lib.DBV_BF16, lg=FAKE, ss=3200, sy=400, sp=100, m=FAKE,
             par=FAKE, ep=FAKE, et=FAKE, ns=None, npos=None, g=FAKE, gs=400, gp=100, T=1.0,
             mode=_lib.DBV_TREE_STATE_EQUALITY, o=FAKE, ws=FAKE, wsb=1 << 22, stream=None)
    a.update(kw)
    o = a["o"]
    return lib.verify_gumbel_tree(a["B"], a["S"], a["L"], a["V"], a["dt"], a["lg"], a["ss"], a["sy"],
                                  a["sp"], a["m"], a["par"], a["ep"], a["et"], a["ns"], a["npos"],
                                  a["g"], a["gs"], a["gp"], a["T"], a["mode"], o, o, o, o, o, o, o,
                                  o, o, a["ws"], a["wsb"], a["stream"], a.get("opts"))


def _sparse(lib, **kw):
    a = dict(B=2, K=3, V=100, dt=_lib.DBV_BF16, tgt=FAKE, ts=400, tr=100, qi=FAKE, qp=FAKE, qn=FAKE, kmax=20,
             d=FAKE, n=None, tt=1.0, ua=FAKE, ur=FAKE, eos=-1, bud=None, o=FAKE, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    o = a["o"]
    return lib.verify_sparse(a["B"], a["K"], a["V"], a["dt"], a["tgt"], a["ts"], a["tr"], a["qi"], a["qp"], a["qn"],
                             a["kmax"], a["d"], a["n"], a["tt"], a["ua"], a["ur"], a["eos"], a["bud"], o, o, o,
                             None, None, None, None, o, a["ws"], a["wsb"], a["stream"], a.get("opts"))


def _trunc(lib, **kw):
    a = dict(B=2, K=3, V=100, dt=_lib.DBV_BF16, rows=FAKE, ss=300, rs=100, n=None, T=1.0, k=20, p=0.9, kmax=20,
             o=FAKE, stream=None)
    a.update(kw)
    o = a["o"]
    return lib.truncate_top_k_top_p(a["B"], a["K"], a["V"], a["dt"], a["rows"], a["ss"], a["rs"], a["n"], a["T"],
                                    a["k"], a["p"], a["kmax"], o, o, o, a["stream"], a.get("opts"))


def _ddhyp(lib, **kw):
    a = dict(B=2, L=8, V=100, dt=_lib.DBV_BF16, stale=FAKE, ss=800, sp=100, m=FAKE, g=FAKE, gs=800, gp=100,
             T=1.0, below=0.6, o=FAKE, st=FAKE, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    o = a["o"]
    return lib.ddtree_hypotheses(a["B"], a["L"], a["V"], a["dt"], a["stale"], a["ss"], a["sp"], a["m"], a["g"],
                                 a["gs"], a["gp"], a["T"], a["below"], o, o, a["st"], a["ws"], a["wsb"],
                                 a["stream"], a.get("opts"))


def _ddtree(lib, level=False, **kw):
    a = dict(B=2, L=8, D=5, m=FAKE, ht=FAKE, hp=FAKE, order=FAKE, os=72, orow=8, tau=1.0, gamma=0.0, first=1,
             o=FAKE, nm=FAKE, fr=FAKE, st=FAKE, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    o = a["o"]
    head = (a["B"], a["L"], a["D"], a["m"], a["ht"], a["hp"], a["order"], a["os"], a["orow"], a["tau"],
            a["gamma"])
    tail = (o, o, o, o, a["nm"], o, a["fr"], o, a["st"], a["ws"], a["wsb"], a["stream"], a.get("opts"))
    if level:
        return lib.ddtree_level(*head, a["first"], *tail)
    return lib.ddtree_build(*head, *tail)


def _spot(lib, **kw):
    a = dict(B=2, K=3, V=100, dt=_lib.DBV_BF16, tgt=FAKE, ts=400, tr=100, drf=FAKE, ds=300, dr=100, ps=FAKE,
             pp=FAKE, d=FAKE, c=FAKE, n=None, tt=1.0, td=1.0, g=FAKE, gs=400, gr=100, tau=0.6, ua=FAKE, ur=FAKE,
             eos=-1, bud=None, o=FAKE, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    o = a["o"]
    return lib.verify_spot_chain(a["B"], a["K"], a["V"], a["dt"], a["tgt"], a["ts"], a["tr"], a["drf"], a["ds"],
                                 a["dr"], a["ps"], a["pp"], a["d"], a["c"], a["n"], a["tt"], a["td"], a["g"],
                                 a["gs"], a["gr"], a["tau"], a["ua"], a["ur"], a["eos"], a["bud"], o, o, o, None,
                                 None, None, None, o, a["ws"], a["wsb"], a["stream"], a.get("opts"))


def _any_order(lib, **kw):
    a = dict(B=2, U=4, V=100, dt=_lib.DBV_BF16, tgt=FAKE, ts=400, tr=100, order=FAKE, na=None, pos=None,
             d=FAKE, dr=FAKE, ds=400, drs=100, eos=-1, end=None, o=FAKE, nd=FAKE, st=FAKE, ws=FAKE,
             wsb=1 << 20, stream=None)
    a.update(kw)
    o = a["o"]
    return lib.verify_greedy_any_order(a["B"], a["U"], a["V"], a["dt"], a["tgt"], a["ts"], a["tr"], a["order"],
                                       a["na"], a["pos"], a["d"], a["dr"], a["ds"], a["drs"], a["eos"], a["end"],
                                       o, o, o, o, o, a["nd"], a["st"], a["ws"], a["wsb"], a["stream"], a.get("opts"))


INVALID = _lib.DBV_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(K=-1), dict(K=5000), dict(V=0), dict(W=-2), dict(dt=3), dict(tgt=None),
    dict(d=None), dict(dr=None), dict(ts=-1), dict(acc=None), dict(out=None), dict(num=None),
    dict(tgt=FAKE + 1),
])
def test_greedy_rejects_bad_args(lib, kw):
    assert _greedy(lib, **kw) == INVALID


@pytest.mark.parametrize("kw", [
    dict(tt=0.0), dict(td=-1.0), dict(tt=float("nan")), dict(td=float("inf")), dict(drf=None),
    dict(ua=None), dict(ur=None), dict(d=None), dict(V=0), dict(dr=-5), dict(tgt=FAKE + 1),
])
def test_rejection_rejects_bad_args(lib, kw):
    assert _reject(lib, **kw) == INVALID
    assert _reject(lib, lenient=True, **kw) == INVALID
    assert _reject(lib, cactus=True, **kw) == INVALID


@pytest.mark.parametrize("lam", [-0.01, 1.01, float("nan")])
def test_lenient_rejects_bad_lambda(lib, lam):
    assert _reject(lib, lenient=True, lam=lam) == INVALID


@pytest.mark.parametrize("delta", [-0.01, float("nan"), float("inf")])
def test_cactus_rejects_bad_budget(lib, delta):
    assert _reject(lib, cactus=True, delta=delta) == INVALID


@pytest.mark.parametrize("kw", [
    dict(S=0), dict(S=5000), dict(L=0), dict(V=0), dict(mode=2), dict(T=-0.5), dict(T=float("nan")),
    dict(m=None), dict(g=None), dict(par=None), dict(ep=None), dict(et=None), dict(o=None),
    dict(mode=_lib.DBV_TREE_FIXED_POSITION, npos=None), dict(gs=-1), dict(g=FAKE + 2),
])
def test_tree_rejects_bad_args(lib, kw):
    assert _tree(lib, **kw) == INVALID


@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(U=-1), dict(U=5000), dict(V=0), dict(dt=3), dict(tgt=None), dict(order=None),
    dict(d=None), dict(o=None), dict(ts=-1), dict(drs=-1), dict(tgt=FAKE + 1), dict(dr=FAKE + 1),
])
def test_any_order_rejects_bad_args(lib, kw):
    assert _any_order(lib, **kw) == INVALID


@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(K=-1), dict(K=5000), dict(V=0), dict(dt=3), dict(tgt=None), dict(ps=None), dict(pp=None),
    dict(c=None), dict(d=None), dict(drf=None), dict(ua=None), dict(ur=None), dict(o=None), dict(tt=0.0),
    dict(td=float("nan")), dict(tau=float("nan")), dict(gs=-1), dict(gr=-2), dict(g=FAKE + 2), dict(tgt=FAKE + 1),
])
def test_spot_chain_rejects_bad_args(lib, kw):
    assert _spot(lib, **kw) == INVALID


@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(K=-1), dict(V=0), dict(dt=3), dict(tgt=None), dict(qi=None), dict(qp=None), dict(qn=None),
    dict(kmax=-1), dict(d=None), dict(ua=None), dict(ur=None), dict(o=None), dict(tt=0.0), dict(tgt=FAKE + 1),
])
def test_sparse_rejects_bad_args(lib, kw):
    assert _sparse(lib, **kw) == INVALID


def test_sparse_limits(lib):
    assert _sparse(lib, kmax=257) == _lib.DBV_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(K=-1), dict(V=0), dict(dt=3), dict(rows=None), dict(ss=-1), dict(T=0.0), dict(T=float("nan")),
    dict(k=0), dict(k=21), dict(p=0.0), dict(p=1.5), dict(p=float("nan")), dict(kmax=0), dict(o=None),
    dict(rows=FAKE + 1),
])
def test_truncate_rejects_bad_args(lib, kw):
    assert _trunc(lib, **kw) == INVALID


def test_truncate_limits(lib):
    assert _trunc(lib, kmax=300, k=20) == _lib.DBV_ERR_UNSUPPORTED
    assert _trunc(lib, V=(1 << 21) + 1) == _lib.DBV_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(L=0), dict(L=65), dict(V=0), dict(dt=3), dict(stale=None), dict(m=None), dict(o=None),
    dict(ss=-1), dict(gp=-1), dict(T=-1.0), dict(T=float("nan")), dict(T=float("inf")), dict(g=None),
    dict(below=float("nan")), dict(stale=FAKE + 1), dict(g=FAKE + 2),
])
def test_ddtree_hypotheses_rejects_bad_args(lib, kw):
    assert _ddhyp(lib, **kw) == INVALID


@pytest.mark.parametrize("level", [False, True])
@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(L=0), dict(L=65), dict(D=-1), dict(D=65), dict(m=None), dict(ht=None), dict(hp=None),
    dict(order=None), dict(os=-1), dict(orow=-1), dict(tau=0.0), dict(tau=float("nan")), dict(gamma=-0.1),
    dict(gamma=float("inf")), dict(o=None), dict(fr=None), dict(order=FAKE + 2),
])
def test_ddtree_rejects_bad_args(lib, level, kw):
    assert _ddtree(lib, level=level, **kw) == INVALID


def test_ddtree_workspace(lib):
    h = lib.verify_workspace_size(_lib.DBV_KIND_DDTREE_HYPOTHESES, 16, 32, 0, 151936, _lib.DBV_BF16)
    assert h >= 16 * 32 * 8 and h % 256 == 0
    assert lib.verify_workspace_size(_lib.DBV_KIND_DDTREE_HYPOTHESES, 16, 65, 0, 100, 1) == 0
    t = lib.verify_workspace_size(_lib.DBV_KIND_DDTREE, 16, 20, 32, 0, 0)
    assert t >= 16 * 21 * 16 and t % 256 == 0
    assert lib.verify_workspace_size(_lib.DBV_KIND_DDTREE, 16, 65, 32, 0, 0) == 0
    assert _ddhyp(lib, wsb=16) == _lib.DBV_ERR_WORKSPACE
    assert _ddtree(lib, wsb=16) == _lib.DBV_ERR_WORKSPACE
    assert _ddtree(lib, level=True, ws=FAKE + 8) == _lib.DBV_ERR_WORKSPACE


def test_workspace_errors(lib):
    assert _greedy(lib, ws=None) == _lib.DBV_ERR_WORKSPACE
    assert _greedy(lib, wsb=8) == _lib.DBV_ERR_WORKSPACE
    assert _greedy(lib, ws=FAKE + 64) == _lib.DBV_ERR_WORKSPACE
    assert _reject(lib, wsb=16) == _lib.DBV_ERR_WORKSPACE
    assert _tree(lib, wsb=16) == _lib.DBV_ERR_WORKSPACE
    assert _any_order(lib, wsb=16) == _lib.DBV_ERR_WORKSPACE
    assert _spot(lib, wsb=16) == _lib.DBV_ERR_WORKSPACE
    assert _sparse(lib, wsb=16) == _lib.DBV_ERR_WORKSPACE


def test_optional_arguments_are_accepted(lib):
    # T = 0 needs no Gumbel table; W = 0 needs no draft rows; fixed mode needs
    # no mask.  These pass host validation (then meet the device check).
    if _gpu_visible():
        pytest.skip("would launch with fake pointers on a GPU")
    nodev = _lib.DBV_ERR_NO_DEVICE
    assert _tree(lib, T=0.0, g=None) == nodev
    assert _tree(lib, mode=_lib.DBV_TREE_FIXED_POSITION, npos=FAKE, m=None) == nodev
    assert _greedy(lib, W=0, dr=None, nd=None, nl=None) == nodev
    assert _reject(lib, K=0, drf=None, d=None, ua=None) == nodev
    assert _any_order(lib, dr=None, nd=None, st=None) == nodev
    assert _any_order(lib, U=0, order=None, d=None) == nodev
    assert _spot(lib, g=None, tau=float("inf")) == nodev
    assert _sparse(lib, kmax=0, qi=None, qp=None) == nodev
    assert _trunc(lib, n=FAKE, p=1.0) == nodev
    assert _trunc(lib, B=0, rows=None, o=None) == nodev
    assert _sparse(lib, K=0, qi=None, qp=None, qn=None, d=None, ua=None) == nodev
    assert _spot(lib, K=0, drf=None, pp=None, d=None, c=None, ua=None) == nodev
    assert _ddhyp(lib, T=0.0, g=None, st=None) == nodev
    assert _ddhyp(lib, B=0, stale=None, m=None, o=None) == nodev
    assert _ddtree(lib, nm=None, st=None) == nodev
    assert _ddtree(lib, level=True, D=0, fr=None) == nodev


def test_valid_call_without_gpu_reports_no_device(lib):
    if _gpu_visible():
        pytest.skip("a GPU is visible")
    assert _greedy(lib) == _lib.DBV_ERR_NO_DEVICE
    assert _reject(lib) == _lib.DBV_ERR_NO_DEVICE
    assert _reject(lib, lenient=True) == _lib.DBV_ERR_NO_DEVICE
    assert _reject(lib, cactus=True, delta=0.0) == _lib.DBV_ERR_NO_DEVICE
    assert _tree(lib) == _lib.DBV_ERR_NO_DEVICE
    assert _any_order(lib, na=FAKE, pos=FAKE, eos=3, end=FAKE) == _lib.DBV_ERR_NO_DEVICE


def test_product_path_fails_loudly_without_library(monkeypatch, tmp_path):
    # The binding never falls back: a missing library is an error.
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()


def _opts(**kw):
    return ctypes.byref(_lib.Options(**kw))


def test_options_struct_matches_header():
    # dbv_options: two uint32 then seven pointers, in this order.
    text = open(HEADER).read()
    body = re.search(r"typedef struct dbv_options \{(.*?)\} dbv_options;", text, re.S).group(1)
    fields = re.findall(r"(\w+);", body)
    assert fields == [f for f, _ in _lib.Options._fields_]
    assert ctypes.sizeof(_lib.Options) == 8 + 7 * ctypes.sizeof(ctypes.c_void_p)


def test_options_are_validated(lib):
    # One timing event without the other, or a size too small for them.
    assert _greedy(lib, opts=_opts(row_begin=FAKE)) == INVALID
    assert _reject(lib, opts=_opts(row_end=FAKE)) == INVALID
    bad = _lib.Options()
    bad.size = 8
    assert _tree(lib, opts=ctypes.byref(bad)) == INVALID
    # Diagnostic outputs an entry point does not produce.
    assert _greedy(lib, opts=_opts(accept_margin=FAKE)) == INVALID
    assert _tree(lib, opts=_opts(draw_margin=FAKE)) == INVALID
    assert _tree(lib, opts=_opts(row_tv=FAKE)) == INVALID
    assert _any_order(lib, opts=_opts(row_tv=FAKE)) == INVALID
    assert _trunc(lib, opts=_opts(pos_margin=FAKE)) == INVALID
    assert _ddhyp(lib, opts=_opts(tok_margin=FAKE)) == INVALID
    assert _ddtree(lib, opts=_opts(accept_margin=FAKE)) == INVALID
    assert _reject(lib, opts=_opts(pos_margin=FAKE)) == INVALID
    assert _spot(lib, opts=_opts(tok_margin=FAKE)) == INVALID
    assert _sparse(lib, opts=_opts(pos_margin=FAKE)) == INVALID


def test_options_accepted_without_gpu(lib):
    if _gpu_visible():
        pytest.skip("would launch with fake pointers on a GPU")
    nodev = _lib.DBV_ERR_NO_DEVICE
    ev = dict(row_begin=FAKE, row_end=FAKE)
    assert _greedy(lib, opts=_opts(**ev)) == nodev
    assert _reject(lib, opts=_opts(accept_margin=FAKE, draw_margin=FAKE, **ev)) == nodev
    assert _reject(lib, lenient=True, opts=_opts(accept_margin=FAKE)) == nodev
    assert _spot(lib, opts=_opts(draw_margin=FAKE)) == nodev
    assert _sparse(lib, opts=_opts(accept_margin=FAKE)) == nodev
    assert _tree(lib, opts=_opts(pos_margin=FAKE, tok_margin=FAKE, **ev)) == nodev
    assert _reject(lib, cactus=True, opts=_opts(row_tv=FAKE)) == nodev
    assert _sparse(lib, opts=_opts(row_tv=FAKE)) == nodev
    assert _ddtree(lib, opts=_opts(**ev)) == nodev


def _noalloc(lib, **kw):
    a = dict(B=2, K=3, V=100, dt=_lib.DBV_BF16, tgt=FAKE, ts=400, tr=100, drf=FAKE, ds=300,
             dr=100, d=FAKE, n=None, tt=1.0, td=1.0, ua=FAKE, ur=FAKE, eos=-1, bud=None,
             acc=FAKE, out=FAKE, num=FAKE, st=FAKE, stream=None)
    a.update(kw)
    return lib.verify_rejection_noalloc(a["B"], a["K"], a["V"], a["dt"], a["tgt"], a["ts"], a["tr"], a["drf"],
                                        a["ds"], a["dr"], a["d"], a["n"], a["tt"], a["td"], a["ua"], a["ur"],
                                        a["eos"], a["bud"], a["acc"], a["out"], a["num"], None, None, None, None,
                                        a["st"], a["stream"], a.get("opts"))


@pytest.mark.parametrize("kw", [
    dict(B=-1), dict(K=-1), dict(K=5000), dict(V=0), dict(dt=3), dict(tgt=None), dict(drf=None), dict(ua=None),
    dict(ur=None), dict(d=None), dict(tt=0.0), dict(td=float("nan")), dict(acc=None), dict(tgt=FAKE + 1),
])
def test_noalloc_rejects_bad_args(lib, kw):
    assert _noalloc(lib, **kw) == INVALID


def test_noalloc_limit(lib):
    # The workspace of this call would exceed the library's 4 MiB scratch.
    need = lib.verify_workspace_size(_lib.DBV_KIND_REJECTION, 4096, 64, 0, 151936, _lib.DBV_BF16)
    assert need > 4 << 20
    assert _noalloc(lib, B=4096, K=64, V=151936) == _lib.DBV_ERR_UNSUPPORTED
    assert _noalloc(lib, V=(1 << 21) + 1) == _lib.DBV_ERR_UNSUPPORTED


def test_noalloc_without_gpu_reports_no_device(lib):
    if _gpu_visible():
        pytest.skip("a GPU is visible")
    assert _noalloc(lib) == _lib.DBV_ERR_NO_DEVICE
    assert _noalloc(lib, B=32, K=16, V=151936) == _lib.DBV_ERR_NO_DEVICE

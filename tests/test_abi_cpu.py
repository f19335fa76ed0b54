"""C-ABI checks that need no GPU: exported symbols, host-only entry points, and
argument validation (every rejected call returns before touching the device).

Invalid calls are made with fake, 256-byte-aligned addresses that are never
dereferenced: each case fails a check that runs before any HIP call.
"""
import ctypes
import os
import re
from fractions import Fraction

import pytest
from hypothesis import given, settings, strategies as st

import oracle
from sparse_mixture_experts_10_amd import _native, api

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = [os.path.join(INCLUDE, h) for h in sorted(os.listdir(INCLUDE)) if h.endswith(".h")]
OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x7f0000000000)   # aligned, never dereferenced
MIS = ctypes.c_void_p(0x7f0000000008)    # 8-byte aligned only
NULL = None


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(moe_\w+)\s*\(", src, flags=re.M))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    lib = _native.load()
    names = declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_native.SIGNATURES), "binding signatures must cover the header exactly"


def test_status_strings_and_version():
    lib = _native.load()
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, 12345):
        assert lib.moe_status_string(code)
    assert api.moe_version() == 2


@settings(max_examples=300, deadline=None)
@given(num=st.integers(0, 10**6), den=st.integers(1, 10**4), k=st.integers(1, 32),
       T=st.integers(0, 10**7), E=st.integers(1, 256))
def test_capacity_matches_oracle(num, den, k, T, E):
    """Host capacity C = ceil(C_f k T / E) against the oracle's exact rational form."""
    assert api.moe_capacity(num, den, k, T, E) == oracle.capacity(Fraction(num, den), k, T, E)


def test_capacity_workloads_and_errors():
    assert api.moe_capacity(4, 1, 2, 16, 4) == 32
    assert api.moe_capacity(5, 4, 2, 4096, 8) == 1280
    assert api.moe_capacity(1, 1, 1, 16384, 64) == 256
    lib = _native.load()
    out = ctypes.c_int64(0)
    assert lib.moe_capacity(1, 0, 1, 1, 1, ctypes.byref(out)) == INVALID
    assert lib.moe_capacity(-1, 1, 1, 1, 1, ctypes.byref(out)) == INVALID
    assert lib.moe_capacity(1, 1, 0, 1, 1, ctypes.byref(out)) == INVALID
    assert lib.moe_capacity(1, 1, 1, 1, 1, None) == INVALID
    assert lib.moe_capacity(2**62, 1, 32, 2**40, 1, ctypes.byref(out)) == INVALID   # overflow


def test_workspace_sizes():
    assert api.moe_workspace_bytes(api.OP_ROUTER, T=100, d=8, E=8) == 0
    assert api.moe_workspace_bytes(api.OP_COMBINE) == 0
    d = api.moe_workspace_bytes(api.OP_DISPATCH, T=4096, E=8)
    assert d >= 64 * 8 * 4 + 16 * 8 * 4 and d % 256 == 0   # chunk counts, group counts
    assert api.moe_workspace_bytes(api.OP_FFN, F=1536, max_rows=1000) >= 1000 * 24 * 4
    assert api.moe_workspace_bytes(api.OP_STATS, T=1000, E=128) >= 4 * 129 * 8
    lib = _native.load()
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_bytes(99, 1, 1, 1, 1, 1, 1, ctypes.byref(n)) == INVALID
    assert lib.moe_workspace_bytes(api.OP_DISPATCH, -1, 1, 1, 1, 1, 1, ctypes.byref(n)) == INVALID
    assert lib.moe_workspace_bytes(api.OP_DISPATCH, 1, 1, 1, 1, 1, 1, None) == INVALID


def _router(**kw):
    a = dict(x=FAKE, dt=1, T=16, d=8, W=FAKE, bg=NULL, bs=NULL, E=4, k=2, lg=FAKE, lse=FAKE, idx=FAKE, g=FAKE)
    a.update(kw)
    return _native.load().moe_router_topk(a["x"], a["dt"], a["T"], a["d"], a["W"], a["bg"], a["bs"], a["E"],
                                          a["k"], a.get("nz"), 0.5, a.get("tau", 1.0), a["lg"], a["lse"], a["idx"], a["g"],
                                          a.get("ws"), a.get("wsb", 0), None)


def test_router_validation():
    assert _router(k=0) == INVALID
    assert _router(k=5) == INVALID            # k > E
    assert _router(E=0) == INVALID
    assert _router(E=257, k=2) == UNSUPPORTED
    assert _router(E=64, k=33) == UNSUPPORTED
    assert _router(T=-1) == INVALID
    assert _router(d=12) == INVALID           # rows not 16-byte multiples
    assert _router(dt=7) == UNSUPPORTED
    assert _router(x=NULL) == INVALID
    assert _router(idx=NULL) == INVALID
    assert _router(x=MIS) == INVALID
    assert _router(T=0) == OK                 # empty batch: nothing to do
    assert _router(T=2**30, k=2) == UNSUPPORTED
    # the gate temperature must be finite and positive (checked before T = 0 returns)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert _router(tau=bad) == INVALID
        assert _router(tau=bad, T=0) == INVALID
    assert _router(tau=0.5, T=0) == OK
    # bf16 x with a large W_g takes the MFMA path, which needs the workspace
    assert _router(E=128, d=4096, k=8, ws=None) == WORKSPACE
    assert _router(E=128, d=4096, k=8, ws=FAKE, wsb=16) == WORKSPACE
    assert api.moe_workspace_bytes(api.OP_ROUTER, T=32768, d=4096, E=128) >= 3 * 128 * 4096 * 2 + 32768
    assert api.moe_workspace_bytes(api.OP_ROUTER, T=4096, d=512, E=8) == 0


def _mlp_router(**kw):
    a = dict(x=FAKE, dt=1, T=16, d=8, W1=FAKE, b1=NULL, H=16, W2=FAKE, b2=NULL, bs=NULL, E=4, k=2, lg=FAKE,
             lse=FAKE, idx=FAKE, g=FAKE, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return _native.load().moe_mlp_router_topk(a["x"], a["dt"], a["T"], a["d"], a["W1"], a["b1"], a["H"], a["W2"],
                                              a["b2"], a["bs"], a["E"], a["k"], None, 0.0, a.get("tau", 1.0),
                                              a["lg"], a["lse"],
                                              a["idx"], a["g"], a["ws"], a["wsb"], None)


def test_mlp_router_validation():
    assert _mlp_router(H=12) == INVALID            # hidden width not a multiple of 8
    assert _mlp_router(H=264) == UNSUPPORTED
    assert _mlp_router(k=5) == INVALID
    assert _mlp_router(W1=NULL) == INVALID
    assert _mlp_router(W2=MIS) == INVALID
    assert _mlp_router(ws=NULL) == WORKSPACE
    assert _mlp_router(wsb=100) == WORKSPACE
    assert _mlp_router(T=0) == OK
    assert _mlp_router(tau=0.0) == INVALID
    assert _mlp_router(tau=float("nan")) == INVALID
    assert api.moe_workspace_bytes(api.OP_MLP_ROUTER, T=1000, F=128) >= 1000 * 128 * 8


def _dispatch(**kw):
    a = dict(idx=FAKE, T=16, k=2, E=4, cap=32, x=FAKE, dt=1, d=8, cnt=FAKE, off=FAKE, slot=FAKE, row=FAKE,
             rt=FAKE, xd=FAKE, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return _native.load().moe_dispatch(a["idx"], a["T"], a["k"], a["E"], a["cap"], a["x"], a["dt"], a["d"],
                                       a["cnt"], a["off"], a["slot"], a["row"], a["rt"], a["xd"], a["ws"],
                                       a["wsb"], None)


def test_dispatch_validation():
    assert _dispatch(cap=-2) == INVALID
    assert _dispatch(k=3, E=2) == INVALID
    assert _dispatch(cnt=NULL) == INVALID
    assert _dispatch(x=NULL) == INVALID       # x and x_disp must both be given or both NULL
    assert _dispatch(xd=MIS) == INVALID
    assert _dispatch(d=4) == INVALID
    assert _dispatch(dt=3) == UNSUPPORTED
    assert _dispatch(ws=NULL) == WORKSPACE
    assert _dispatch(wsb=16) == WORKSPACE
    assert _dispatch(ws=ctypes.c_void_p(0x7f0000000010)) == WORKSPACE   # not 256-byte aligned
    assert _dispatch(slot=NULL) == INVALID


def _route(**kw):
    a = dict(x=FAKE, dt=1, T=16, d=8, W=FAKE, bg=NULL, bs=NULL, E=4, k=2, cap=32, lg=FAKE, lse=FAKE,
             idx=FAKE, g=FAKE, cnt=FAKE, off=FAKE, slot=FAKE, row=FAKE, rt=FAKE, f=FAKE, P=FAKE, L=FAKE,
             ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return _native.load().moe_route(a["x"], a["dt"], a["T"], a["d"], a["W"], a["bg"], a["bs"], a["E"], a["k"],
                                    None, 0.0, a.get("tau", 1.0), a["cap"], 0.01, 1e-3, a["lg"], a["lse"], a["idx"], a["g"], a["cnt"],
                                    a["off"], a["slot"], a["row"], a["rt"], a["f"], a["P"], a["L"], a["ws"],
                                    a["wsb"], None)


def test_route_validation():
    assert _route(k=0) == INVALID
    assert _route(k=5) == INVALID
    assert _route(E=300) == UNSUPPORTED
    assert _route(cap=-2) == INVALID
    assert _route(d=12) == INVALID
    assert _route(dt=5) == UNSUPPORTED
    assert _route(x=NULL) == INVALID
    assert _route(f=NULL) == INVALID
    assert _route(cnt=NULL) == INVALID
    assert _route(rt=NULL) == INVALID
    assert _route(x=MIS) == INVALID
    assert _route(ws=NULL) == WORKSPACE
    assert _route(wsb=64) == WORKSPACE
    assert _route(ws=ctypes.c_void_p(0x7f0000000010)) == WORKSPACE
    assert _route(T=2**30) == UNSUPPORTED
    assert _route(tau=-2.0) == INVALID
    assert _route(tau=float("inf")) == INVALID
    # the routing workspace covers the router's and the dispatch's
    for T, d, E in ((4096, 512, 8), (32768, 4096, 128), (1, 8, 1)):
        r = api.moe_workspace_bytes(api.OP_ROUTE, T=T, d=d, E=E)
        assert r >= api.moe_workspace_bytes(api.OP_ROUTER, T=T, d=d, E=E)
        assert r >= api.moe_workspace_bytes(api.OP_DISPATCH, T=T, E=E)


def _ffn(**kw):
    a = dict(a=FAKE, go=FAKE, G=4, mr=32, d=8, F=16, do=8, dt=1, act=0, W1=FAKE, b1=FAKE, W2=FAKE, b2=FAKE,
             h=FAKE, o=FAKE, sq=NULL, ws=NULL, wsb=0)
    a.update(kw)
    return _native.load().moe_grouped_ffn(a["a"], a.get("ar"), a["go"], a["G"], a["mr"], a["d"], a["F"],
                                          a["do"], a["dt"], a["act"], a["W1"], a["b1"], a["W2"], a["b2"],
                                          a["h"], a["o"], a["sq"], a["ws"], a["wsb"], None)


def test_grouped_ffn_validation():
    assert _ffn(G=0) == INVALID
    assert _ffn(G=300) == UNSUPPORTED
    assert _ffn(F=12) == INVALID
    assert _ffn(act=5) == UNSUPPORTED
    assert _ffn(dt=2) == UNSUPPORTED
    assert _ffn(W2=NULL) == INVALID
    assert _ffn(h=MIS) == INVALID
    assert _ffn(sq=FAKE) == WORKSPACE         # sum of squares needs the workspace
    assert _ffn(mr=-1) == INVALID
    assert _ffn(mr=0) == OK


def test_shared_combine_stats_validation():
    lib = _native.load()
    assert lib.moe_shared_ffn(FAKE, 4, 8, 16, 0, 8, 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.moe_shared_ffn(FAKE, 4, 8, 16, 2, 8, 1, 9, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert lib.moe_shared_ffn(FAKE, 0, 8, 16, 2, 8, 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == OK
    assert lib.moe_combine(FAKE, FAKE, FAKE, None, 4, 0, 8, 1, FAKE, None) == INVALID
    assert lib.moe_combine(FAKE, FAKE, FAKE, None, 4, 2, 6, 1, FAKE, None) == INVALID
    assert lib.moe_combine(FAKE, FAKE, FAKE, MIS, 4, 2, 8, 1, FAKE, None) == INVALID
    assert lib.moe_combine(FAKE, FAKE, FAKE, None, 0, 2, 8, 1, FAKE, None) == OK

    def stats(T=16, E=4, k=2, credit=NULL, mc=NULL, sq=NULL, tl=NULL, el=NULL, ws=FAKE, wsb=1 << 20,
              f=FAKE, P=FAKE, losses=FAKE):
        return lib.moe_route_stats(FAKE, FAKE, FAKE, FAKE, FAKE, T, E, k, 0.01, 1e-3, f, P, losses, sq,
                                   FAKE, FAKE, FAKE, credit, mc, tl, el, ws, wsb, None)
    assert stats(T=0) == INVALID
    assert stats(k=5) == INVALID
    assert stats(credit=FAKE) == INVALID       # credit and mean_credit go together
    assert stats(credit=FAKE, mc=FAKE) == INVALID   # credit needs the hidden sums of squares
    assert stats(ws=NULL) == WORKSPACE
    assert stats(wsb=8) == WORKSPACE
    assert stats(tl=FAKE) == INVALID                # token_loss and expert_loss go together
    assert stats(tl=FAKE, el=FAKE) == INVALID       # the expert loss needs the credit
    assert stats(f=NULL) == INVALID                 # f, P and losses go together
    assert stats(P=NULL, losses=NULL) == INVALID
    assert stats(f=NULL, P=NULL, losses=NULL) == INVALID   # and without credit nothing is asked
    assert lib.moe_balance_losses(FAKE, FAKE, FAKE, FAKE, 0, 4, 2, 0.01, 1e-3, FAKE, FAKE, FAKE, 1 << 20,
                                  None) == INVALID
    assert lib.moe_balance_losses(FAKE, FAKE, FAKE, FAKE, 16, 4, 2, 0.01, 1e-3, FAKE, FAKE, NULL, 0,
                                  None) == WORKSPACE
    assert lib.moe_balance_losses(FAKE, FAKE, FAKE, NULL, 16, 4, 2, 0.01, 1e-3, FAKE, FAKE, FAKE, 1 << 20,
                                  None) == INVALID
    assert lib.moe_selection_bias_update(FAKE, 4, 5, 16, 0.1, FAKE, None) == INVALID
    assert lib.moe_selection_bias_update(FAKE, 4, 2, 16, 0.1, NULL, None) == INVALID
    assert lib.moe_dro_update(FAKE, 0, 0.9, 0.1, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.moe_dro_update(FAKE, 300, 0.9, 0.1, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert lib.moe_dro_update(FAKE, 8, 0.9, 0.1, FAKE, NULL, FAKE, None) == INVALID
    assert api.moe_workspace_bytes(api.OP_BALANCE, T=1000, E=16) >= 4 * 17 * 8


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        api.moe_combine(x, torch.zeros(4, 2, dtype=torch.int32), torch.zeros(4, 2), None, x)


def test_calibration_validation():
    lib = _native.load()
    d = ctypes.c_double(0)
    assert lib.moe_calib_copy(FAKE, FAKE, 17, None) == INVALID
    assert lib.moe_calib_copy(MIS, FAKE, 32, None) == INVALID
    assert lib.moe_calib_copy(NULL, FAKE, 32, None) == INVALID
    assert lib.moe_calib_copy(FAKE, FAKE, 0, None) == OK
    assert lib.moe_calib_read(FAKE, 8, FAKE, None) == INVALID
    assert lib.moe_calib_read(FAKE, 16, NULL, None) == INVALID
    assert lib.moe_calib_mfma(0, 10, FAKE, ctypes.byref(d), None) == INVALID
    assert lib.moe_calib_mfma(1, 10, FAKE, None, None) == INVALID


def _route_noalloc(**kw):
    a = dict(x=FAKE, dt=1, T=16, d=8, W=FAKE, bg=NULL, bs=NULL, E=4, k=2, cap=32, lg=FAKE, lse=FAKE,
             idx=FAKE, g=FAKE, cnt=FAKE, off=FAKE, slot=FAKE, row=FAKE, rt=FAKE, f=FAKE, P=FAKE, L=FAKE)
    a.update(kw)
    return _native.load().moe_route_noalloc(a["x"], a["dt"], a["T"], a["d"], a["W"], a["bg"], a["bs"], a["E"],
                                            a["k"], None, 0.0, a.get("tau", 1.0), a["cap"], 0.01, 1e-3, a["lg"],
                                            a["lse"], a["idx"], a["g"], a["cnt"], a["off"], a["slot"], a["row"],
                                            a["rt"], a["f"], a["P"], a["L"], None)


def _noalloc_max_bytes():
    src = open(os.path.join(INCLUDE, "moe.h")).read()
    m = re.search(r"#define MOE_ROUTE_NOALLOC_MAX_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    return int(m.group(1)) << int(m.group(2))


def test_route_noalloc_validation_and_limit():
    """The no-workspace routing pass checks its arguments as moe_route does and
    rejects, before touching the device, any call needing more scratch than
    its static array holds."""
    assert _route_noalloc(k=5) == INVALID
    assert _route_noalloc(x=NULL) == INVALID
    assert _route_noalloc(tau=0.0) == INVALID
    assert _route_noalloc(dt=5) == UNSUPPORTED
    cap = _noalloc_max_bytes()
    assert cap == 64 << 20
    # the split-weight MFMA router's partials grow with T: find sizes on both sides of the limit
    E, d, k = 128, 4096, 8
    need = lambda T: api.moe_workspace_bytes(api.OP_ROUTE, T=T, d=d, E=E)
    assert need(32768) <= cap                       # the large workload fits
    big = 65536
    assert need(big) > cap
    assert _route_noalloc(T=big, d=d, E=E, k=k) == -5
    assert _native.load().moe_status_string(-5) != _native.load().moe_status_string(12345)

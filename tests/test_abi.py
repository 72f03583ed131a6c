"""The C-ABI library on the host (no GPU): it loads, exports every function
include/xhc.h declares, sizes workspaces and rejects bad arguments before
launching anything."""
import ctypes
import os
import re

import pytest

from residual_stream_architecture_amd import xhc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    txt = open(os.path.join(ROOT, "include", "xhc.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(xhc_[a-z_]+)\s*\(", txt)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert "xhc_forward" in names and "xhc_backward" in names and len(names) >= 11
    for n in names:
        assert hasattr(xhc.lib, n), n


def test_kernel_names():
    names = xhc.kernel_names()
    assert names[:4] == ["pack_wt", "proj", "coef", "mix"]
    assert "bgrad" in names and "bdots" in names and "mixproj" in names
    assert "gram" in names and "bdots_gs" in names


BASE = 1 << 40          # fake, 256-aligned device addresses: validation never dereferences them


def fake(i, off=0):
    return BASE + (i << 32) + off


def good_fwd(desc, inplace=True):
    act = (ctypes.c_int32 * desc.k)(*range(desc.k))
    a = xhc.xhc_fwd_args(
        X=fake(1), out=fake(2), w4=fake(3) if desc.ncomp == 4 else None,
        w8=fake(4) if desc.ncomp == 4 else None, w12=fake(5) if desc.ncomp == 4 else None,
        W=fake(6), bias=None, active=ctypes.cast(act, ctypes.POINTER(ctypes.c_int32)),
        X_new=fake(1) if inplace else fake(7), h_in=fake(8), z_save=fake(9), xact_save=fake(10),
        timer=None)
    return a, act


def good_bwd(desc):
    act = (ctypes.c_int32 * desc.k)(*range(desc.k))
    c4 = desc.ncomp == 4
    a = xhc.xhc_bwd_args(
        X=fake(1), xact=fake(2), out=fake(3), w4=fake(4) if c4 else None, w8=fake(5) if c4 else None,
        w12=fake(6) if c4 else None, W=fake(7), bias=None,
        active=ctypes.cast(act, ctypes.POINTER(ctypes.c_int32)), z_save=fake(8), dX_new=fake(9),
        dh_in=fake(10), dX=fake(11), dout=fake(12), dW=fake(13), db=fake(14),
        dw4=fake(15) if c4 else None, dw8=fake(16) if c4 else None, dw12=fake(17) if c4 else None,
        accumulate=0, timer=None)
    return a, act


def desc16(**kw):
    d = dict(B=2, S=100, C=256, N=16, k=4, ncomp=4, dtype=xhc.XHC_BF16)
    d.update(kw)
    return xhc.make_desc(**d)


def test_workspace_sizes():
    d = desc16()
    f, b = xhc.workspace_size(d, 0), xhc.workspace_size(d, 1)
    assert f > 0 and b > f and f % 256 == 0 and b % 256 == 0
    assert xhc.workspace_size(desc16(C=7), 0) == 0
    assert xhc.workspace_size(d, 5) == 0
    # the headline workload: T=8192, C=4096; the workspace stays small next to the state
    big = desc16(B=2, S=4096, C=4096)
    assert xhc.workspace_size(big, 1) < 0.25 * 8192 * 16 * 4096 * 2


@pytest.mark.parametrize("kw,code", [
    (dict(C=12), -2), (dict(C=0), -2), (dict(k=5), -2), (dict(N=3), -2), (dict(N=17), -2),
    (dict(ncomp=2), -2), (dict(B=0), -2), (dict(dtype=7), -6), (dict(iters=0), -2),
    (dict(iters=65), -2), (dict(B=1 << 14, S=1 << 10, C=1024), -2),
    (dict(gram_schmidt=2), -6), (dict(gram_schmidt=True, gs_eps=0.0), -2),
    (dict(gram_schmidt=True, gs_eps=float("nan")), -2), (dict(gram_schmidt=True, gs_eps=-1e-6), -2)])
def test_bad_descriptions(kw, code):
    d = desc16(**kw)
    a, _ = good_fwd(desc16())
    assert xhc.validate(d, a, 0) == code


def test_gram_schmidt_workspace():
    # Gram-Schmidt adds the Gram partials (forward) and the Sg records
    # (backward); with one component it is the identity and adds nothing
    d, g = desc16(), desc16(gram_schmidt=True)
    T, ncb = 200, 1                                  # C = 256: one channel block of 512
    assert xhc.workspace_size(g, 0) - xhc.workspace_size(d, 0) == -(-ncb * T * 16 * 4 // 256) * 256
    assert xhc.workspace_size(g, 1) > xhc.workspace_size(d, 1)
    d1, g1 = desc16(ncomp=1, N=4), desc16(ncomp=1, N=4, gram_schmidt=True)
    assert xhc.workspace_size(g1, 0) == xhc.workspace_size(d1, 0)
    assert xhc.workspace_size(g1, 1) == xhc.workspace_size(d1, 1)


def test_valid_arguments_pass():
    for kw in [dict(), dict(ncomp=1, N=4), dict(N=1, k=1, ncomp=1, dtype=xhc.XHC_F32), dict(gram_schmidt=True)]:
        d = desc16(**kw)
        a, keep = good_fwd(d)
        assert xhc.validate(d, a, 0) == 0, kw
        a2, keep2 = good_fwd(d, inplace=False)
        assert xhc.validate(d, a2, 0) == 0, kw
        b, keep3 = good_bwd(d)
        assert xhc.validate(d, b, 1) == 0, kw


def test_forward_error_paths():
    d = desc16()
    a, keep = good_fwd(d)
    # null required pointers
    for f in ("X", "out", "W", "X_new", "h_in", "w8"):
        b, k2 = good_fwd(d)
        setattr(b, f, None)
        assert xhc.validate(d, b, 0) == -1, f
    # indices: out of range, repeated
    for bad in ([0, 1, 2, 16], [0, 1, 1, 3], [-1, 1, 2, 3]):
        b, _ = good_fwd(d)
        arr = (ctypes.c_int32 * 4)(*bad)
        b.active = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
        assert xhc.validate(d, b, 0) == -3, bad
    # alignment
    b, _ = good_fwd(d)
    b.out = fake(2, 8)
    assert xhc.validate(d, b, 0) == -5
    # partial overlap of X_new with X, h_in inside X, xact_save overlapping h_in
    b, _ = good_fwd(d)
    b.X_new = fake(1, 4096)
    assert xhc.validate(d, b, 0) == -4
    b, _ = good_fwd(d)
    b.h_in = fake(1, 1024)
    assert xhc.validate(d, b, 0) == -4
    b, _ = good_fwd(d)
    b.xact_save = fake(8, 256)
    assert xhc.validate(d, b, 0) == -4
    # conv weights given for a single-component call
    d1 = desc16(ncomp=1)
    b, _ = good_fwd(d1)
    b.w4 = fake(3)
    assert xhc.validate(d1, b, 0) == -6


def test_backward_error_paths():
    d = desc16()
    for f in ("X", "dX_new", "dh_in", "dX", "dout", "dW", "dw12", "W"):
        b, _ = good_bwd(d)
        setattr(b, f, None)
        assert xhc.validate(d, b, 1) == -1, f
    b, _ = good_bwd(d)
    b.dX = b.dX_new                      # in-place dX is allowed
    assert xhc.validate(d, b, 1) == 0
    b, _ = good_bwd(d)
    b.dX = fake(9, 512)                  # partial overlap is not
    assert xhc.validate(d, b, 1) == -4
    b, _ = good_bwd(d)
    b.dout = fake(3)                     # gradient written over an input
    assert xhc.validate(d, b, 1) == -4
    b, _ = good_bwd(d)
    b.accumulate = 2
    assert xhc.validate(d, b, 1) == -6


def test_calls_fail_before_launch_without_workspace():
    d = desc16()
    a, keep = good_fwd(d)
    rc = xhc.lib.xhc_forward(ctypes.byref(d), ctypes.byref(a), None, 0, None)
    assert rc == -7
    rc = xhc.lib.xhc_forward(ctypes.byref(d), ctypes.byref(a), fake(20), 16, None)
    assert rc == -7
    rc = xhc.lib.xhc_forward(ctypes.byref(d), ctypes.byref(a), fake(20, 128), 1 << 40, None)
    assert rc == -5


def test_noalloc_refuses_before_launch():
    # xhc_forward_noalloc checks everything before its first HIP call: the
    # forward's validation, no timer, and a problem that fits its static
    # scratch array (T = 24576 tokens at C = 4096 needs more than 64 MiB)
    noalloc = xhc.lib.xhc_forward_noalloc
    d = desc16()
    a, keep = good_fwd(d)
    a.X = None
    assert noalloc(ctypes.byref(d), ctypes.byref(a), None) == xhc.XHC_ERR_NULL
    a, keep = good_fwd(d)
    a.timer = fake(30)
    assert noalloc(ctypes.byref(d), ctypes.byref(a), None) == xhc.XHC_ERR_UNSUPPORTED
    big = desc16(B=3, S=8192, C=4096)
    assert xhc.workspace_size(big, 0) > xhc.NOALLOC_SCRATCH_BYTES
    a, keep = good_fwd(big)
    assert noalloc(ctypes.byref(big), ctypes.byref(a), None) == xhc.XHC_ERR_SCRATCH
    # the headline workload's forward fits
    assert xhc.workspace_size(desc16(B=2, S=4096, C=4096), 0) <= xhc.NOALLOC_SCRATCH_BYTES


def good_chain():
    return xhc.xhc_chain_args(carry_in=fake(21), W_next=fake(22), carry_out=fake(23))


def chain_call(d, a, c, ws=None, nbytes=0):
    return xhc.lib.xhc_forward_chain(ctypes.byref(d), ctypes.byref(a), ctypes.byref(c), ws, nbytes, None)


def test_carry_size():
    # one partial record of 16*NT + 4 floats per token and channel block; blocks
    # are 64 channels (bf16) or 32 (fp32) wide, at most 16 of them
    d = desc16()                                 # C = 256 bf16: 4 blocks, P = 48 (NT = 3)
    assert xhc.carry_size(d) == 4 * 200 * 52 * 4
    assert xhc.carry_size(desc16(dtype=xhc.XHC_F32)) == 8 * 200 * 52 * 4
    assert xhc.carry_size(desc16(C=7168)) == 16 * 200 * 52 * 4
    assert xhc.carry_size(desc16(N=4, ncomp=1)) == 4 * 200 * 36 * 4      # P = 24 (NT = 2)
    assert xhc.carry_size(desc16(C=7)) == 0


def test_chain_error_paths():
    d = desc16()
    a, keep = good_fwd(d)
    # valid chain arguments get as far as the workspace check
    assert chain_call(d, a, good_chain()) == -7
    # no chain structure behaves as xhc_forward
    assert xhc.lib.xhc_forward_chain(ctypes.byref(d), ctypes.byref(a), None, None, 0, None) == -7
    # with carry_in the state is not projected: W may be NULL
    b, _ = good_fwd(d)
    b.W = None
    assert chain_call(d, b, good_chain()) == -7
    c = good_chain()
    c.carry_in = None
    assert chain_call(d, b, c) == -1
    # W_next and carry_out come together
    for f in ("W_next", "carry_out"):
        c = good_chain()
        setattr(c, f, None)
        assert chain_call(d, a, c) == -1, f
    # the same buffer for carry in and out is allowed; a partial overlap is not
    c = good_chain()
    c.carry_out = c.carry_in
    assert chain_call(d, a, c) == -7
    c = good_chain()
    c.carry_out = fake(21, 256)
    assert chain_call(d, a, c) == -4
    # carries may not overlap the call's buffers
    for f, v in (("carry_out", fake(1)), ("carry_out", fake(6, 512)), ("carry_in", fake(8)), ("W_next", fake(9))):
        c = good_chain()
        setattr(c, f, v)
        assert chain_call(d, a, c) == -4, f
    c = good_chain()
    c.carry_out = fake(23, 8)
    assert chain_call(d, a, c) == -5
    # the next sublayer may differ in k and ncomp, not in B, S, C, N or dtype
    for kw, code in ((dict(ncomp=1), -7), (dict(k=2), -7), (dict(ncomp=1, gram_schmidt=True), -7),
                     (dict(C=512), -2), (dict(N=8), -2), (dict(S=99), -2), (dict(dtype=xhc.XHC_F32), -2),
                     (dict(k=5), -2)):
        dn = desc16(**kw)
        c = good_chain()
        c.desc_next = ctypes.pointer(dn)
        assert chain_call(d, a, c) == code, kw


def test_strerror():
    for c in range(0, -10, -1):
        assert xhc.strerror(c)
    assert "unknown" in xhc.strerror(-99)


# ---------------------------------------------------------------------------
# router (desc.route > 0)
# ---------------------------------------------------------------------------

def routed_fwd(desc):
    a, act = good_fwd(desc, inplace=False)
    a.W_route, a.b_route, a.route_idx = fake(20), fake(21), fake(22)
    return a, act


def routed_bwd(desc):
    a, act = good_bwd(desc)
    a.xact = None
    a.W_route, a.route_idx, a.dW_route, a.db_route = fake(20), fake(22), fake(23), fake(24)
    return a, act


def test_route_descriptions():
    assert xhc.validate(desc16(route=2), routed_fwd(desc16(route=2))[0], xhc.XHC_PHASE_FWD) == xhc.XHC_OK
    assert xhc.validate(desc16(route=5), routed_fwd(desc16())[0], xhc.XHC_PHASE_FWD) == xhc.XHC_ERR_SHAPE
    assert xhc.validate(desc16(route=-1), routed_fwd(desc16())[0], xhc.XHC_PHASE_FWD) == xhc.XHC_ERR_SHAPE
    # no fixed stream: all 16 streams are candidates
    assert xhc.workspace_size(desc16(route=4), xhc.XHC_PHASE_FWD) > 0
    assert xhc.validate(desc16(route=4), routed_fwd(desc16(route=4))[0], xhc.XHC_PHASE_FWD) == xhc.XHC_OK
    d = desc16(N=12, route=4)
    assert xhc.validate(d, routed_fwd(d)[0], xhc.XHC_PHASE_FWD) == xhc.XHC_OK


def test_route_zsave_stride_and_workspace():
    P = 16 + 16 + 16
    assert xhc.zsave_stride(desc16()) == P + 1
    assert xhc.zsave_stride(desc16(route=2)) == P + 3 + 6
    assert xhc.zsave_stride(desc16(route=3)) == P + 3 + 9
    assert xhc.zsave_stride(desc16(route=9)) == 0
    for phase in (xhc.XHC_PHASE_FWD, xhc.XHC_PHASE_BWD):
        assert xhc.workspace_size(desc16(route=2), phase) > xhc.workspace_size(desc16(), phase)


def test_route_forward_error_paths():
    d = desc16(route=2)
    a, _ = routed_fwd(d)
    a.W_route = None
    assert xhc.validate(d, a, xhc.XHC_PHASE_FWD) == xhc.XHC_ERR_NULL
    # only the fixed prefix of `active` is read: repeats past it are fine
    a, act = routed_fwd(d)
    act[2] = act[3] = act[0]
    assert xhc.validate(d, a, xhc.XHC_PHASE_FWD) == xhc.XHC_OK
    act[1] = act[0]
    assert xhc.validate(d, a, xhc.XHC_PHASE_FWD) == xhc.XHC_ERR_INDEX
    a, _ = routed_fwd(d)
    a.route_idx = fake(22, 4)
    assert xhc.validate(d, a, xhc.XHC_PHASE_FWD) == xhc.XHC_ERR_ALIGN
    a, _ = routed_fwd(d)
    a.route_idx = a.h_in                            # an output overlapping another
    assert xhc.validate(d, a, xhc.XHC_PHASE_FWD) == xhc.XHC_ERR_ALIAS
    a, _ = routed_fwd(d)
    a.route_idx = a.W_route                         # an output overlapping an input
    assert xhc.validate(d, a, xhc.XHC_PHASE_FWD) == xhc.XHC_ERR_ALIAS
    # the router needs neither b_route nor route_idx
    a, _ = routed_fwd(d)
    a.b_route, a.route_idx = None, None
    assert xhc.validate(d, a, xhc.XHC_PHASE_FWD) == xhc.XHC_OK


def test_route_backward_error_paths():
    d = desc16(route=2)
    assert xhc.validate(d, routed_bwd(d)[0], xhc.XHC_PHASE_BWD) == xhc.XHC_OK
    for field in ("route_idx", "W_route", "dW_route"):
        a, _ = routed_bwd(d)
        setattr(a, field, None)
        assert xhc.validate(d, a, xhc.XHC_PHASE_BWD) == xhc.XHC_ERR_NULL, field
    a, _ = routed_bwd(d)
    a.z_save = None                                 # recomputed: needs the forward's b_route
    assert xhc.validate(d, a, xhc.XHC_PHASE_BWD) == xhc.XHC_ERR_NULL
    a.b_route = fake(25)
    assert xhc.validate(d, a, xhc.XHC_PHASE_BWD) == xhc.XHC_OK
    a.xact = fake(2)                                # but not from saved rows
    assert xhc.validate(d, a, xhc.XHC_PHASE_BWD) == xhc.XHC_ERR_UNSUPPORTED
    a, _ = routed_bwd(d)
    a.db_route = None
    assert xhc.validate(d, a, xhc.XHC_PHASE_BWD) == xhc.XHC_OK
    a, _ = routed_bwd(d)
    a.xact = fake(2)                                # after an in-place forward
    assert xhc.validate(d, a, xhc.XHC_PHASE_BWD) == xhc.XHC_OK
    a, _ = routed_bwd(d)
    a.dW_route = a.dW
    assert xhc.validate(d, a, xhc.XHC_PHASE_BWD) == xhc.XHC_ERR_ALIAS
    a, _ = routed_bwd(d)
    a.db_route = a.route_idx
    assert xhc.validate(d, a, xhc.XHC_PHASE_BWD) == xhc.XHC_ERR_ALIAS


def test_route_chain_validation():
    W, NUL, UNS, WS = xhc.XHC_OK, xhc.XHC_ERR_NULL, xhc.XHC_ERR_UNSUPPORTED, xhc.XHC_ERR_WORKSPACE
    nxt = (ctypes.c_int32 * 4)(4, 9, 0, 0)
    nxt_p = ctypes.cast(nxt, ctypes.POINTER(ctypes.c_int32))
    d = desc16(route=2)
    # out of place: the routed pass rewrites each token's own rows in place only
    a, _ = routed_fwd(d)
    c = xhc.xhc_chain_args(None, fake(30), fake(31), None, fake(32), nxt_p)
    assert chain_call(d, a, c) == UNS
    a.X_new = a.X
    # a valid routed chain passes validation and stops at the missing workspace
    assert chain_call(d, a, c) == WS
    c.W_route_next = None                            # the next router's columns are required
    assert chain_call(d, a, c) == NUL
    c.W_route_next = fake(32)
    c.active_next = None                             # and its fixed streams
    assert chain_call(d, a, c) == NUL
    dup = (ctypes.c_int32 * 4)(3, 3, 0, 0)
    c.active_next = ctypes.cast(dup, ctypes.POINTER(ctypes.c_int32))
    assert chain_call(d, a, c) == xhc.XHC_ERR_INDEX
    c.active_next = nxt_p
    c.W_route_next = a.X_new + 64                    # an input overlapping an output
    assert chain_call(d, a, c) == xhc.XHC_ERR_ALIAS
    # two or four per-token slots at N = 16, k = 4 only
    for kw in (dict(route=1), dict(route=3), dict(route=2, N=12)):
        dd = desc16(**kw)
        a, _ = routed_fwd(dd)
        a.X_new = a.X
        c = xhc.xhc_chain_args(None, fake(30), fake(31), None, fake(32), nxt_p)
        assert chain_call(dd, a, c) == UNS, kw
    # a fixed-list sublayer whose next sublayer routes
    a, _ = good_fwd(desc16())
    c = xhc.xhc_chain_args(None, fake(30), fake(31), ctypes.pointer(desc16(route=2)), None, nxt_p)
    assert chain_call(desc16(), a, c) == NUL
    c.W_route_next = fake(32)
    assert chain_call(desc16(), a, c) == WS
    # given lists chain too (four per-token slots)
    dg = desc16(per_token_active=True)
    a, _ = good_fwd(dg)
    a.route_idx = fake(22)
    c = xhc.xhc_chain_args(None, fake(30), fake(31), None, None, None)
    assert chain_call(dg, a, c) == WS


def test_route_kernel_names():
    names = xhc.kernel_names()
    assert {"route_colsum", "route_pass", "route_dwr"} <= set(names)


def test_given_lists_validation():
    d = desc16(per_token_active=1)
    a, _ = good_fwd(d, inplace=False)
    assert xhc.validate(d, a, xhc.XHC_PHASE_FWD) == xhc.XHC_ERR_NULL          # the lists are required
    a.route_idx = fake(22)
    a.active = None                                                          # the host list is not read
    assert xhc.validate(d, a, xhc.XHC_PHASE_FWD) == xhc.XHC_OK
    a.route_idx = a.X_new                                                    # an input overlapping an output
    assert xhc.validate(d, a, xhc.XHC_PHASE_FWD) == xhc.XHC_ERR_ALIAS
    assert xhc.validate(desc16(per_token_active=1, route=2), a, xhc.XHC_PHASE_FWD) == xhc.XHC_ERR_UNSUPPORTED
    assert xhc.validate(desc16(per_token_active=2), a, xhc.XHC_PHASE_FWD) == xhc.XHC_ERR_UNSUPPORTED
    b, _ = good_bwd(d)
    assert xhc.validate(d, b, xhc.XHC_PHASE_BWD) == xhc.XHC_ERR_NULL
    b.route_idx = fake(22)
    assert xhc.validate(d, b, xhc.XHC_PHASE_BWD) == xhc.XHC_OK
    b.z_save = None                                                          # xact without saved logits
    assert xhc.validate(d, b, xhc.XHC_PHASE_BWD) == xhc.XHC_ERR_UNSUPPORTED
    b.xact = None
    assert xhc.validate(d, b, xhc.XHC_PHASE_BWD) == xhc.XHC_OK
    a, _ = good_fwd(d, inplace=False)
    a.route_idx = fake(22)
    c = xhc.xhc_chain_args(None, fake(30), fake(31), None)
    assert chain_call(d, a, c) == xhc.XHC_ERR_UNSUPPORTED


def test_hres_active_descriptions():
    # H_res from the active rows: fixed lists only, not chained; z_save holds r_act too
    d = desc16(hres_active=True)
    a, keep = good_fwd(d)
    assert xhc.validate(d, a, xhc.XHC_PHASE_FWD) == xhc.XHC_OK
    b, keep2 = good_bwd(d)
    assert xhc.validate(d, b, xhc.XHC_PHASE_BWD) == xhc.XHC_OK
    P = 16 + 4 * 4 + 16
    assert xhc.zsave_stride(d) == P + 2 and xhc.zsave_stride(desc16()) == P + 1
    assert xhc.workspace_size(d, 0) == xhc.workspace_size(desc16(), 0)
    for kw in (dict(route=2), dict(per_token_active=True)):
        dd = desc16(hres_active=True, **kw)
        assert xhc.workspace_size(dd, 0) == 0, kw
        assert xhc.validate(dd, a, xhc.XHC_PHASE_FWD) == xhc.XHC_ERR_UNSUPPORTED, kw
    bad = desc16()
    bad.hres_active = 2
    assert xhc.validate(bad, a, xhc.XHC_PHASE_FWD) == xhc.XHC_ERR_UNSUPPORTED
    # the carried partials sum every stream: no chain
    a, keep = good_fwd(d, inplace=False)
    c = good_chain()
    # (no workspace: a call that passes every check stops at XHC_ERR_WORKSPACE)
    assert chain_call(d, a, c) == xhc.XHC_ERR_UNSUPPORTED
    dn = desc16()
    assert chain_call(dn, a, c) == xhc.XHC_ERR_WORKSPACE
    c.desc_next = ctypes.pointer(desc16(hres_active=True))
    assert chain_call(dn, a, c) == xhc.XHC_ERR_UNSUPPORTED


def good_pre(desc, chained=False):
    act = (ctypes.c_int32 * desc.k)(*range(desc.k))
    a = xhc.xhc_pre_args(X=fake(1), W=fake(2), bias=None, active=ctypes.cast(act, ctypes.POINTER(ctypes.c_int32)),
                         h_in=fake(3), z_save=fake(4), carry_in=fake(5) if chained else None,
                         W_next=fake(6) if chained else None, carry_out=fake(7) if chained else None)
    return a, act


def good_post(desc, chained=False):
    act = (ctypes.c_int32 * desc.k)(*range(desc.k))
    c4 = desc.ncomp == 4
    a = xhc.xhc_post_args(X=fake(1), out=fake(8), w4=fake(9) if c4 else None, w8=fake(10) if c4 else None,
                          w12=fake(11) if c4 else None, active=ctypes.cast(act, ctypes.POINTER(ctypes.c_int32)),
                          z_save=fake(4), xact_save=fake(12), W_next=fake(6) if chained else None,
                          carry_out=fake(7) if chained else None)
    return a, act


def test_split_forward_validation():
    d = desc16()
    PRE, POST = xhc.XHC_PHASE_PRE, xhc.XHC_PHASE_POST
    for chained in (False, True):
        a, keep = good_pre(d, chained)
        assert xhc.validate(d, a, PRE) == xhc.XHC_OK, chained
        b, keep2 = good_post(d, chained)
        assert xhc.validate(d, b, POST) == xhc.XHC_OK, chained
    # z_save is required by both calls; W only without carry_in
    a, keep = good_pre(d)
    a.z_save = None
    assert xhc.validate(d, a, PRE) == xhc.XHC_ERR_NULL
    a, keep = good_pre(d)
    a.W = None
    assert xhc.validate(d, a, PRE) == xhc.XHC_ERR_NULL
    a, keep = good_pre(d, chained=True)
    a.W = None
    assert xhc.validate(d, a, PRE) == xhc.XHC_OK
    a.carry_out = None                                   # W_next without carry_out
    assert xhc.validate(d, a, PRE) == xhc.XHC_ERR_NULL
    a, keep = good_pre(d, chained=True)
    a.carry_out = a.carry_in                             # the coefficients consume carry_in first
    assert xhc.validate(d, a, PRE) == xhc.XHC_OK
    a.carry_out = a.h_in
    assert xhc.validate(d, a, PRE) == xhc.XHC_ERR_ALIAS
    a, keep = good_pre(d)
    a.h_in = a.X
    assert xhc.validate(d, a, PRE) == xhc.XHC_ERR_ALIAS
    b, keep = good_post(d)
    b.z_save = None
    assert xhc.validate(d, b, POST) == xhc.XHC_ERR_NULL
    b, keep = good_post(d)
    b.out = b.X
    assert xhc.validate(d, b, POST) == xhc.XHC_ERR_ALIAS
    b, keep = good_post(d, chained=True)
    b.carry_out = b.z_save
    assert xhc.validate(d, b, POST) == xhc.XHC_ERR_ALIAS
    b, keep = good_post(d)
    b.w8 = None
    assert xhc.validate(d, b, POST) == xhc.XHC_ERR_NULL
    # per-token lists (a router or given lists) and hres_active only without a carry
    for kw in (dict(route=2), dict(route=4), dict(per_token_active=True)):
        dd = desc16(**kw)
        a, keep = good_pre(dd)
        assert xhc.validate(dd, a, PRE) == xhc.XHC_ERR_NULL, kw            # no route_idx
        a.route_idx = fake(22)
        if kw.get("route"):
            assert xhc.validate(dd, a, PRE) == xhc.XHC_ERR_NULL, kw        # no W_route
            a.W_route = fake(20)
        assert xhc.validate(dd, a, PRE) == xhc.XHC_OK, kw
        a.route_idx = a.h_in                                            # lists overlapping h_in
        assert xhc.validate(dd, a, PRE) == xhc.XHC_ERR_ALIAS, kw
        a, keep = good_pre(dd, chained=True)
        a.route_idx, a.W_route = fake(22), fake(20)
        assert xhc.validate(dd, a, PRE) == xhc.XHC_ERR_UNSUPPORTED, kw
        b, keep = good_post(dd)
        assert xhc.validate(dd, b, POST) == xhc.XHC_ERR_NULL, kw
        b.route_idx = fake(22)
        assert xhc.validate(dd, b, POST) == xhc.XHC_OK, kw
        b.route_idx = b.X + 64                                          # the lists are an input
        assert xhc.validate(dd, b, POST) == xhc.XHC_ERR_ALIAS, kw
        b, keep = good_post(dd, chained=True)
        b.route_idx = fake(22)
        assert xhc.validate(dd, b, POST) == xhc.XHC_ERR_UNSUPPORTED, kw
    # given lists with a status word (the router's lists are its own output)
    dg = desc16(per_token_active=True)
    a, keep = good_pre(dg)
    a.route_idx, a.status = fake(22), fake(30)
    assert xhc.validate(dg, a, PRE) == xhc.XHC_OK
    a.status = fake(30, 4)
    assert xhc.validate(dg, a, PRE) == xhc.XHC_ERR_ALIGN
    dh = desc16(hres_active=True)
    assert xhc.validate(dh, good_pre(dh)[0], PRE) == xhc.XHC_OK
    assert xhc.validate(dh, good_pre(dh, chained=True)[0], PRE) == xhc.XHC_ERR_UNSUPPORTED
    assert xhc.validate(dh, good_post(dh, chained=True)[0], POST) == xhc.XHC_ERR_UNSUPPORTED
    # the next description must describe the same state
    a, keep = good_pre(d, chained=True)
    a.desc_next = ctypes.pointer(desc16(C=128))
    assert xhc.validate(d, a, PRE) == xhc.XHC_ERR_SHAPE
    a.desc_next = ctypes.pointer(desc16(ncomp=1))
    assert xhc.validate(d, a, PRE) == xhc.XHC_OK
    # calls stop before any launch without a workspace
    a, keep = good_pre(d)
    assert xhc.lib.xhc_forward_pre(ctypes.byref(d), ctypes.byref(a), None, 0, None) == xhc.XHC_ERR_WORKSPACE
    b, keep = good_post(d)
    assert xhc.lib.xhc_forward_post(ctypes.byref(d), ctypes.byref(b), None, 0, None) == xhc.XHC_ERR_WORKSPACE


def good_bwd_post(desc):
    act = (ctypes.c_int32 * desc.k)(*range(desc.k))
    c4 = desc.ncomp == 4
    a = xhc.xhc_bwd_post_args(
        out=fake(3), w4=fake(4) if c4 else None, w8=fake(5) if c4 else None, w12=fake(6) if c4 else None,
        active=ctypes.cast(act, ctypes.POINTER(ctypes.c_int32)), z_save=fake(8), dX_new=fake(9), dout=fake(12),
        dw4=fake(15) if c4 else None, dw8=fake(16) if c4 else None, dw12=fake(17) if c4 else None,
        bwd_state=fake(20), accumulate=0, timer=None)
    return a, act


def good_bwd_pre(desc):
    act = (ctypes.c_int32 * desc.k)(*range(desc.k))
    a = xhc.xhc_bwd_pre_args(
        X=fake(1), xact=fake(2), W=fake(7), bias=None, active=ctypes.cast(act, ctypes.POINTER(ctypes.c_int32)),
        z_save=fake(8), dX_new=fake(9), dh_in=fake(10), bwd_state=fake(20), dX=fake(11), dW=fake(13), db=fake(14),
        accumulate=0, timer=None)
    return a, act


def test_split_backward_validation():
    d = desc16()
    BP, BR = xhc.XHC_PHASE_BWD_POST, xhc.XHC_PHASE_BWD_PRE
    a, keep = good_bwd_post(d)
    assert xhc.validate(d, a, BP) == xhc.XHC_OK
    b, keep2 = good_bwd_pre(d)
    assert xhc.validate(d, b, BR) == xhc.XHC_OK
    # the state: dot partials per channel block of the dots pass, token and dot slot
    T = d.B * d.S
    st = xhc.bwd_state_size(d)
    assert st > 0 and st % (T * 48 * 4) == 0
    assert xhc.bwd_state_size(desc16(C=4096)) > st
    bad = desc16()
    bad.N = 17
    assert xhc.bwd_state_size(bad) == 0
    # required pointers
    for field in ("z_save", "dX_new", "dout", "bwd_state", "out", "dw8"):
        a, keep = good_bwd_post(d)
        setattr(a, field, None)
        assert xhc.validate(d, a, BP) == xhc.XHC_ERR_NULL, field
    for field in ("X", "W", "z_save", "dX_new", "dh_in", "bwd_state", "dX", "dW"):
        b, keep = good_bwd_pre(d)
        setattr(b, field, None)
        assert xhc.validate(d, b, BR) == xhc.XHC_ERR_NULL, field
    # xact and db are optional
    b, keep = good_bwd_pre(d)
    b.xact = None
    b.db = None
    assert xhc.validate(d, b, BR) == xhc.XHC_OK
    # the state is an output of the first call and an input of the second
    a, keep = good_bwd_post(d)
    a.bwd_state = a.dX_new
    assert xhc.validate(d, a, BP) == xhc.XHC_ERR_ALIAS
    a, keep = good_bwd_post(d)
    a.dout = fake(20, 64)
    assert xhc.validate(d, a, BP) == xhc.XHC_ERR_ALIAS
    b, keep = good_bwd_pre(d)
    b.dW = fake(20, 256)
    assert xhc.validate(d, b, BR) == xhc.XHC_ERR_ALIAS
    # dX may be dX_new itself but not a part of it
    b, keep = good_bwd_pre(d)
    b.dX = b.dX_new
    assert xhc.validate(d, b, BR) == xhc.XHC_OK
    b.dX = fake(9, 256)
    assert xhc.validate(d, b, BR) == xhc.XHC_ERR_ALIAS
    # alignment, accumulate, indices
    a, keep = good_bwd_post(d)
    a.bwd_state = fake(20, 4)
    assert xhc.validate(d, a, BP) == xhc.XHC_ERR_ALIGN
    a, keep = good_bwd_post(d)
    a.accumulate = 2
    assert xhc.validate(d, a, BP) == xhc.XHC_ERR_UNSUPPORTED
    b, keep = good_bwd_pre(d)
    keep[1] = keep[0]
    assert xhc.validate(d, b, BR) == xhc.XHC_ERR_INDEX
    # ncomp = 1: no conv weights or their gradients
    d1 = desc16(ncomp=1)
    a, keep = good_bwd_post(d1)
    assert xhc.validate(d1, a, BP) == xhc.XHC_OK
    a.dw4 = fake(15)
    assert xhc.validate(d1, a, BP) == xhc.XHC_ERR_UNSUPPORTED
    # Gram-Schmidt, a router, per-token lists and hres_active are split
    dd = desc16(gram_schmidt=True)
    assert xhc.validate(dd, good_bwd_post(dd)[0], BP) == xhc.XHC_OK
    assert xhc.validate(dd, good_bwd_pre(dd)[0], BR) == xhc.XHC_OK
    for kw in (dict(route=2), dict(per_token_active=True)):
        dd = desc16(**kw)
        a, keep = good_bwd_post(dd)
        assert xhc.validate(dd, a, BP) == xhc.XHC_ERR_NULL, kw             # no route_idx
        a.route_idx = fake(22)
        assert xhc.validate(dd, a, BP) == xhc.XHC_OK, kw
        a.status = fake(30)
        assert xhc.validate(dd, a, BP) == xhc.XHC_OK, kw
        a.status = a.route_idx
        assert xhc.validate(dd, a, BP) == xhc.XHC_ERR_ALIAS, kw
        b, keep = good_bwd_pre(dd)
        assert xhc.validate(dd, b, BR) == xhc.XHC_ERR_NULL, kw
        b.route_idx = fake(22)
        if kw.get("route"):
            assert xhc.validate(dd, b, BR) == xhc.XHC_ERR_NULL, kw         # no W_route, dW_route
            b.W_route, b.dW_route = fake(20), fake(23)
        assert xhc.validate(dd, b, BR) == xhc.XHC_OK, kw
        if kw.get("route"):
            b.db_route = b.dW_route                                     # two outputs overlapping
            assert xhc.validate(dd, b, BR) == xhc.XHC_ERR_ALIAS, kw
    dh = desc16(hres_active=True)
    assert xhc.validate(dh, good_bwd_post(dh)[0], BP) == xhc.XHC_OK
    assert xhc.validate(dh, good_bwd_pre(dh)[0], BR) == xhc.XHC_OK
    # both need the backward's workspace and stop before any launch without it
    assert xhc.workspace_size(d, BP) == 0 and xhc.workspace_size(d, BR) == 0
    a, keep = good_bwd_post(d)
    assert xhc.lib.xhc_backward_post(ctypes.byref(d), ctypes.byref(a), None, 0, None) == xhc.XHC_ERR_WORKSPACE
    b, keep = good_bwd_pre(d)
    assert xhc.lib.xhc_backward_pre(ctypes.byref(d), ctypes.byref(b), None, 0, None) == xhc.XHC_ERR_WORKSPACE
    assert xhc.lib.xhc_backward_pre(ctypes.byref(d), None, None, 0, None) == xhc.XHC_ERR_NULL


def test_status_word_of_given_lists():
    F, Bw = xhc.XHC_PHASE_FWD, xhc.XHC_PHASE_BWD
    d = desc16(per_token_active=True)
    a, keep = good_fwd(d)
    a.route_idx = fake(22)
    assert xhc.validate(d, a, F) == xhc.XHC_OK
    a.status = fake(30)
    assert xhc.validate(d, a, F) == xhc.XHC_OK
    a.status = fake(30, 4)
    assert xhc.validate(d, a, F) == xhc.XHC_ERR_ALIGN
    for other in ("route_idx", "X_new", "h_in", "z_save"):
        a.status = getattr(a, other) + 16
        assert xhc.validate(d, a, F) == xhc.XHC_ERR_ALIAS, other
    b, keep2 = good_bwd(d)
    b.route_idx = fake(22)
    b.status = fake(30)
    assert xhc.validate(d, b, Bw) == xhc.XHC_OK
    b.status = b.route_idx
    assert xhc.validate(d, b, Bw) == xhc.XHC_ERR_ALIAS
    b.status = b.dW + 64
    assert xhc.validate(d, b, Bw) == xhc.XHC_ERR_ALIAS
    # with one list for every token the word is not read
    d0 = desc16()
    a, keep = good_fwd(d0)
    a.status = fake(1, 4)
    assert xhc.validate(d0, a, F) == xhc.XHC_OK
    # the router's lists are its own in the forward and an input of the backward
    dr = desc16(route=2)
    a, keep = good_fwd(dr)
    a.W_route, a.route_idx, a.status = fake(20), fake(22), fake(1, 4)
    assert xhc.validate(dr, a, F) == xhc.XHC_OK
    b, keep = good_bwd(dr)
    b.W_route, b.route_idx, b.dW_route, b.status = fake(20), fake(22), fake(23), fake(30, 8)
    assert xhc.validate(dr, b, Bw) == xhc.XHC_ERR_ALIGN
    b.status = fake(30)
    assert xhc.validate(dr, b, Bw) == xhc.XHC_OK
    assert "check_lists" in xhc.kernel_names()

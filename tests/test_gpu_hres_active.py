"""GPU parity of the active-row form of H_res (desc.hres_active = 1: the res
logits are the RMS-normed projection of the k active rows alone; the oracle's
O9) against the oracle with hres_active=True, forward and backward, through
the C ABI.  Backward from the forward's saved logits and rows, and with the
logits recomputed from the original state; dW's res columns on the untouched
streams' rows must be exactly zero (or keep their value with accumulate).

Tolerances as in the other parity tests: fp32 max|err| <= 1e-4 + 1e-4 |ref|,
bf16 <= 1e-2 + 1e-2 |ref|; pass-through rows and saved rows bit-exact."""
import numpy as np
import pytest
import torch

from oracle import xhc_oracle as xo
from residual_stream_architecture_amd import synth
from residual_stream_architecture_amd import xhc
from tests.gpu_util import check_close, device_inputs, host_inputs, say, to_host

pytestmark = pytest.mark.gpu
W_ = synth.Workload
GS_EPS = 1e-6

# name, workload, active list
CASES = [
    ("tiny_f32", W_("h", 1, 64, 64, 16, 4, 4, "f32", "fwdbwd"), [0, 1, 2, 3]),
    ("ragged_bf16", W_("h", 2, 77, 136, 16, 4, 4, "bf16", "fwdbwd"), [5, 12, 0, 9]),
    ("n8_k3_f32", W_("h", 3, 30, 40, 8, 3, 4, "f32", "fwdbwd"), [6, 1, 4]),
    ("nc1_bf16", W_("h", 2, 50, 64, 16, 4, 1, "bf16", "fwdbwd"), [3, 9, 1, 14]),
    ("k2_wide_bf16", W_("h", 1, 130, 1040, 16, 2, 4, "bf16", "fwdbwd"), [7, 2]),
    ("gs_f32", W_("h", 2, 40, 72, 16, 4, 4, "f32", "fwdbwd", gs=True), [15, 3, 8, 1]),
    ("all_active_n4_f32", W_("h", 2, 33, 48, 4, 4, 1, "f32", "fwdbwd"), [2, 0, 3, 1]),
]


def tol(w):
    return (1e-4, 1e-4) if w.dtype == "f32" else (1e-2, 1e-2)


def convs(h, w):
    return (h["w4"], h["w8"], h["w12"]) if w.ncomp == 4 else ()


def conv_kw(dev, w):
    return dict(w4=dev["w4"], w8=dev["w8"], w12=dev["w12"]) if w.ncomp == 4 else {}


def make_desc(w):
    return xhc.make_desc(w.B, w.S, w.C, w.N, w.k, w.ncomp, xhc.XHC_BF16 if w.dtype == "bf16" else xhc.XHC_F32,
                         w.iters, w.eps, gram_schmidt=w.gs, gs_eps=GS_EPS, hres_active=True)


def host_kw(w):
    return dict(B=w.B, S=w.S, iters=w.iters, eps=w.eps, gram_schmidt_on=w.gs, gs_eps=GS_EPS, hres_active=True)


def run_forward(w, dev, active):
    T, C, P = w.T, w.C, w.P
    desc = make_desc(w)
    assert xhc.zsave_stride(desc) == P + 2
    X = dev["X"].clone()
    h_in = torch.empty(T, C, dtype=X.dtype, device=X.device)
    z_save = torch.empty(T, P + 2, device=X.device)
    xact = torch.empty(T, w.k, C, dtype=X.dtype, device=X.device)
    xhc.forward(X, dev["out"], dev["W"], active, X, h_in, B=w.B, S=w.S, bias=dev["bias"], z_save=z_save,
                xact_save=xact, desc=desc, **conv_kw(dev, w))
    torch.cuda.synchronize()
    return X, h_in, z_save, xact


def run_backward(w, dev, active, X, xact, z_save, accumulate=False, init=None):
    T, N, C, P = w.T, w.N, w.C, w.P
    f32 = dict(dtype=torch.float32, device=X.device)
    o = dict(dX=torch.empty_like(dev["dX_new"]), dout=torch.empty(T, C, dtype=X.dtype, device=X.device),
             dW=torch.empty((N * C, P), **f32), db=torch.empty((P,), **f32))
    if w.ncomp == 4:
        o.update({key: torch.empty((C, K), **f32) for key, K in (("dw4", 4), ("dw8", 8), ("dw12", 12))})
    if init is not None:
        for key, v in init.items():
            o[key].copy_(v)
    grads = {key: o[key] for key in ("dw4", "dw8", "dw12") if key in o}
    xhc.backward(X, dev["out"], dev["W"], active, dev["dX_new"], dev["dh_in"], o["dX"], o["dout"], o["dW"],
                 B=w.B, S=w.S, xact=xact, bias=dev["bias"], z_save=z_save, db=o["db"], desc=make_desc(w),
                 accumulate=accumulate, **conv_kw(dev, w), **grads)
    torch.cuda.synchronize()
    return o


def inputs(w, seed):
    d = synth.make_inputs(w, seed=seed, grads=True)
    d["bias"] = (np.random.default_rng(seed + 40).standard_normal(w.P) * 0.3).astype(np.float32)
    return d


@pytest.mark.parametrize("name,w,active", CASES, ids=[c[0] for c in CASES])
def test_hres_active_forward_and_backward(name, w, active):
    say(f"[hres_active] {name} B={w.B} S={w.S} C={w.C} N={w.N} k={w.k} nc={w.ncomp} gs={w.gs} {w.dtype}")
    d = inputs(w, 0)
    h = host_inputs(d)
    dev = device_inputs(d, w.dtype == "bf16")
    atol, rtol = tol(w)
    T, N, C, P = w.T, w.N, w.C, w.P
    ref = xo.forward(h["X"], h["out"], h["W"], h["bias"], active, convs(h, w), **host_kw(w))
    X, h_in, z_save, xact = run_forward(w, dev, active)
    Xn_h = to_host(X)
    inactive = [i for i in range(N) if i not in active]
    assert np.array_equal(Xn_h[:, inactive], h["X"][:, inactive]), "pass-through rows differ"
    assert np.array_equal(to_host(xact), h["X"][:, active]), "saved rows differ"
    check_close("X_new[active]", Xn_h[:, active], ref["X_new"][:, active], atol, rtol)
    check_close("h_in", to_host(h_in), ref["h_in"], atol, rtol)
    zs = to_host(z_save)
    check_close("z", zs[:, :P], ref["z"], atol, rtol)
    check_close("r", zs[:, P], ref["r"], 1e-5, 1e-5)
    check_close("r_act", zs[:, P + 1], ref["r_act"], 1e-5, 1e-5)

    g = xo.backward(h["X"], h["out"], h["W"], h["bias"], active, convs(h, w), h["dX_new"], h["dh_in"],
                    **host_kw(w))
    res0 = N + w.k * w.ncomp
    for label, args in (("saved", (X, xact, z_save)), ("recomputed", (dev["X"], None, None))):
        o = run_backward(w, dev, active, *args)
        for key, rf in (("dX", g["dX"]), ("dout", g["dout"]), ("dW", g["dW"]), ("db", g["db"])):
            check_close(f"{label} {key}", to_host(o[key]), rf, atol, rtol)
        for m, key in enumerate(["dw4", "dw8", "dw12"][:w.ncomp - 1]):
            check_close(f"{label} {key}", to_host(o[key]), g["dconv"][m], atol, rtol)
        dW = to_host(o["dW"]).reshape(N, C, P)
        assert np.count_nonzero(dW[inactive, :, res0:]) == 0, f"{label}: dW on untouched rows' res columns"
    # with accumulate the untouched rows' res columns keep what they held
    init = {key: torch.full_like(o[key], 0.25) for key in ("dW", "db")}
    o = run_backward(w, dev, active, X, xact, z_save, accumulate=True, init=init)
    dW = to_host(o["dW"]).reshape(N, C, P)
    assert (dW[inactive, :, res0:] == 0.25).all()
    check_close("accumulated dW", dW.reshape(N * C, P), g["dW"] + 0.25, atol, rtol)

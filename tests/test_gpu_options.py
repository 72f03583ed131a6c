"""GPU parity of the options the main parity cases leave at their defaults:
k = 3 active streams, a nonzero logit bias (it enters z, and the backward's
gamma = dz.(z - bias)/(N C r^2) and db), unit gates together with the TFA
components, other Sinkhorn iteration counts and RMS epsilons, and gradient
accumulation into existing parameter-gradient buffers.  Every comparison is
against the oracle on the same seeded inputs, with the tolerances of the
main parity tests."""
import numpy as np
import pytest
import torch

from oracle import xhc_oracle as xo
from residual_stream_architecture_amd import synth
from residual_stream_architecture_amd import xhc
from tests.gpu_util import check_close, device_inputs, host_inputs, say, to_host

pytestmark = pytest.mark.gpu


def tol(w):
    return (1e-4, 1e-4) if w.dtype == "f32" else (1e-2, 1e-2)


# name, workload, active, gate, bias scale
OPTION_CASES = [
    ("k3_bf16", synth.Workload("k3", 2, 45, 96, 11, 3, 4, "bf16", "fwd"), [9, 0, 4], "sigmoid", 0.0),
    ("bias_f32", synth.Workload("b", 2, 40, 72, 16, 4, 4, "f32", "fwd"), [2, 7, 11, 13], "sigmoid", 0.5),
    ("bias_bf16", synth.Workload("bb", 1, 70, 128, 16, 4, 4, "bf16", "fwd"), [0, 5, 10, 15], "sigmoid", 0.5),
    ("unit_tfa_f32", synth.Workload("u", 2, 33, 64, 16, 4, 4, "f32", "fwd"), [1, 2, 3, 4], "unit", 0.0),
    ("iters1_f32", synth.Workload("i1", 1, 50, 64, 8, 4, 4, "f32", "fwd", iters=1), [7, 6, 5, 4], "sigmoid", 0.0),
    ("iters64_eps_f32", synth.Workload("i64", 1, 50, 64, 16, 4, 1, "f32", "fwd", iters=64, eps=1e-3),
     [0, 1, 2, 3], "sigmoid", 0.3),
    # H_res logits from the k active rows only: W's res columns are zero on
    # the rows of the untouched streams (the pages' O(k^3 C) generation)
    ("hres_active_bf16", synth.Workload("ha", 2, 60, 136, 16, 4, 4, "bf16", "fwd"), [3, 9, 12, 14], "sigmoid", 0.2),
    ("hres_active_f32", synth.Workload("hf", 1, 50, 40, 9, 3, 1, "f32", "fwd"), [8, 0, 5], "sigmoid", 0.0),
]
RES_FROM_ACTIVE = {"hres_active_bf16", "hres_active_f32"}


def zero_res_rows(d, w, active):
    """Zero the res-logit columns of W on the rows of the untouched streams."""
    P0 = w.N + w.k * w.ncomp
    for i in range(w.N):
        if i not in active:
            d["W"][i * w.C:(i + 1) * w.C, P0:] = 0       # +0 in fp32 and in bf16 bits


def _inputs(w, bias_scale, seed):
    d = synth.make_inputs(w, seed=seed, grads=True)
    if bias_scale:
        d["bias"] = (np.random.default_rng(seed + 100).standard_normal(w.P) * bias_scale).astype(np.float32)
    return d


def _convs(h, w):
    return (h["w4"], h["w8"], h["w12"]) if w.ncomp == 4 else ()


def _conv_kw(dev, w):
    return dict(w4=dev["w4"], w8=dev["w8"], w12=dev["w12"]) if w.ncomp == 4 else {}


def _gate(gate):
    return xhc.XHC_GATE_UNIT if gate == "unit" else xhc.XHC_GATE_SIGMOID


@pytest.mark.parametrize("name,w,active,gate,bias_scale", OPTION_CASES, ids=[c[0] for c in OPTION_CASES])
def test_options_forward_backward(name, w, active, gate, bias_scale):
    say(f"[options] {name} B={w.B} S={w.S} C={w.C} N={w.N} k={w.k} nc={w.ncomp} iters={w.iters} eps={w.eps}")
    d = _inputs(w, bias_scale, seed=11)
    if name in RES_FROM_ACTIVE:
        zero_res_rows(d, w, active)
    h = host_inputs(d)
    dev = device_inputs(d, w.dtype == "bf16")
    T, N, C, P = w.T, w.N, w.C, w.P
    atol, rtol = tol(w)
    ref = xo.forward(h["X"], h["out"], h["W"], h["bias"], active, _convs(h, w), B=w.B, S=w.S,
                     iters=w.iters, eps=w.eps, gate_mode=gate)
    X = dev["X"].clone()
    h_in = torch.empty(T, C, dtype=X.dtype, device=X.device)
    z_save = torch.empty(T, P + 1, device=X.device)
    xact = torch.empty(T, w.k, C, dtype=X.dtype, device=X.device)
    xhc.forward(X, dev["out"], dev["W"], active, X, h_in, B=w.B, S=w.S, bias=dev["bias"], z_save=z_save,
                xact_save=xact, iters=w.iters, eps=w.eps, gate_mode=_gate(gate), **_conv_kw(dev, w))
    torch.cuda.synchronize()
    Xh = to_host(X)
    inactive = [i for i in range(N) if i not in active]
    assert np.array_equal(Xh[:, inactive], h["X"][:, inactive]), "pass-through rows differ"
    check_close("X_new[active]", Xh[:, active], ref["X_new"][:, active], atol, rtol)
    check_close("h_in", to_host(h_in), ref["h_in"], atol, rtol)
    check_close("z", to_host(z_save)[:, :P], ref["z"], atol, rtol)

    g = xo.backward(h["X"], h["out"], h["W"], h["bias"], active, _convs(h, w), h["dX_new"], h["dh_in"],
                    B=w.B, S=w.S, iters=w.iters, eps=w.eps, gate_mode=gate)
    dX = torch.empty_like(dev["dX_new"])
    dout = torch.empty(T, C, dtype=dX.dtype, device=dX.device)
    dW = torch.empty(N * C, P, device=dX.device)
    db = torch.empty(P, device=dX.device)
    dws = dict(dw4=torch.empty(C, 4, device=dX.device), dw8=torch.empty(C, 8, device=dX.device),
               dw12=torch.empty(C, 12, device=dX.device)) if w.ncomp == 4 else {}
    xhc.backward(X, dev["out"], dev["W"], active, dev["dX_new"], dev["dh_in"], dX, dout, dW, B=w.B, S=w.S,
                 xact=xact, bias=dev["bias"], z_save=z_save, db=db, iters=w.iters, eps=w.eps,
                 gate_mode=_gate(gate), **_conv_kw(dev, w), **dws)
    torch.cuda.synchronize()
    check_close("dX", to_host(dX), g["dX"], atol, rtol)
    check_close("dout", to_host(dout), g["dout"], atol, rtol)
    check_close("dW", to_host(dW), g["dW"], atol, rtol)
    check_close("db", to_host(db), g["db"], atol, rtol)
    for m, key in enumerate(["dw4", "dw8", "dw12"][:w.ncomp - 1]):
        check_close(key, to_host(dws[key]), g["dconv"][m], atol, rtol)


def test_backward_accumulates_into_parameter_gradients():
    # accumulate = 1 adds this call's parameter gradients to the buffers'
    # contents: start from known values and compare with start + oracle
    w = synth.Workload("acc", 2, 37, 72, 16, 4, 4, "f32", "fwd")
    active = [3, 8, 1, 12]
    say("[options] accumulate f32 B=2 S=37 C=72")
    d = _inputs(w, 0.2, seed=21)
    h = host_inputs(d)
    dev = device_inputs(d, False)
    T, N, C, P = w.T, w.N, w.C, w.P
    g = xo.backward(h["X"], h["out"], h["W"], h["bias"], active, _convs(h, w), h["dX_new"], h["dh_in"],
                    B=w.B, S=w.S)
    rng = np.random.default_rng(5)
    start = {"dW": rng.standard_normal((N * C, P)), "db": rng.standard_normal(P),
             "dw4": rng.standard_normal((C, 4)), "dw8": rng.standard_normal((C, 8)),
             "dw12": rng.standard_normal((C, 12))}
    bufs = {k: torch.from_numpy(v.astype(np.float32)).cuda() for k, v in start.items()}
    dX = torch.empty_like(dev["dX_new"])
    dout = torch.empty(T, C, device=dX.device)
    xhc.backward(dev["X"], dev["out"], dev["W"], active, dev["dX_new"], dev["dh_in"], dX, dout, bufs["dW"],
                 B=w.B, S=w.S, bias=dev["bias"], db=bufs["db"], w4=dev["w4"], w8=dev["w8"], w12=dev["w12"],
                 dw4=bufs["dw4"], dw8=bufs["dw8"], dw12=bufs["dw12"], accumulate=True)
    torch.cuda.synchronize()
    want = {"dW": g["dW"], "db": g["db"], "dw4": g["dconv"][0], "dw8": g["dconv"][1], "dw12": g["dconv"][2]}
    for key in start:
        ref = start[key].astype(np.float32).astype(np.float64) + want[key]
        check_close(f"{key} (accumulated)", to_host(bufs[key]), ref, 1e-4, 1e-4)
    check_close("dX", to_host(dX), g["dX"], 1e-4, 1e-4)

"""GPU parity of the Gram-Schmidt form (desc.gram_schmidt = 1: the write-back
components orthogonalised per token by modified Gram-Schmidt before the
write) against the oracle with gram_schmidt_on=True, forward and backward,
through the C ABI.  The conv weights are made large and leaning on the
current token, so that the components are strongly correlated with the
output and the orthogonalisation changes them a lot.

Tolerances as in the other parity tests: fp32 max|err| <= 1e-4 + 1e-4 |ref|,
bf16 <= 1e-2 + 1e-2 |ref|; pass-through rows bit-exact."""
import numpy as np
import pytest
import torch

from oracle import xhc_oracle as xo
from residual_stream_architecture_amd import synth
from residual_stream_architecture_amd import xhc
from tests.gpu_util import check_close, device_inputs, host_inputs, say, to_dev, to_host

pytestmark = pytest.mark.gpu
W_ = synth.Workload
GS_EPS = 1e-6

# name, workload, active list, gate mode, conv weights (synthetic | leaning | zero)
CASES = [
    ("tiny_f32", W_("g", 1, 64, 64, 16, 4, 4, "f32", "fwd"), [0, 1, 2, 3], "sigmoid", "leaning"),
    ("ragged_bf16", W_("g", 2, 77, 136, 16, 4, 4, "bf16", "fwd"), [5, 12, 0, 9], "sigmoid", "leaning"),
    ("ragged_f32", W_("g", 2, 61, 72, 16, 4, 4, "f32", "fwd"), [15, 3, 8, 1], "sigmoid", "synthetic"),
    ("k3_n7_f32", W_("g", 3, 30, 40, 7, 3, 4, "f32", "fwd"), [6, 1, 4], "sigmoid", "leaning"),
    ("wide_bf16", W_("g", 1, 130, 1040, 16, 4, 4, "bf16", "fwd"), [4, 5, 6, 7], "sigmoid", "leaning"),
    ("unit_f32", W_("g", 2, 25, 48, 6, 2, 4, "f32", "fwd"), [2, 5], "unit", "leaning"),
    ("edge_c8_s1_f32", W_("g", 4, 1, 8, 16, 4, 4, "f32", "fwd"), [0, 1, 2, 3], "sigmoid", "leaning"),
    ("edge_c8_s5_bf16", W_("g", 3, 5, 8, 4, 3, 4, "bf16", "fwd"), [3, 1, 2], "sigmoid", "leaning"),
    # near-collinear components (the regime the retrospective's section on
    # Gram-Schmidt is about): each conv component is the output plus a
    # little of its neighbours, cosine with the output about 0.99 / 0.999
    ("collinear99_f32", W_("g", 2, 96, 1024, 16, 4, 4, "f32", "fwd"), [0, 5, 10, 15], "sigmoid", "cos0.99"),
    ("collinear999_f32", W_("g", 2, 96, 1024, 16, 4, 4, "f32", "fwd"), [2, 3, 4, 5], "sigmoid", "cos0.999"),
    ("collinear99_bf16", W_("g", 2, 96, 1024, 16, 4, 4, "bf16", "fwd"), [1, 6, 11, 14], "sigmoid", "cos0.99"),
    ("collinear999_bf16", W_("g", 2, 96, 1024, 16, 4, 4, "bf16", "fwd"), [8, 9, 10, 11], "sigmoid", "cos0.999"),
]


def tol(w):
    return (1e-4, 1e-4) if w.dtype == "f32" else (1e-2, 1e-2)


def make_case(w, seed, grads, convs_kind):
    d = synth.make_inputs(w, seed=seed, grads=grads)
    if convs_kind == "leaning":
        r = np.random.default_rng(seed + 100)
        for key, K in (("w4", 4), ("w8", 8), ("w12", 12)):
            v = (r.standard_normal((w.C, K)) * 0.3).astype(np.float32)
            v[:, K - 1] += 0.6                   # the tap on the current token
            d[key] = v
    elif convs_kind == "zero":
        for key in ("w4", "w8", "w12"):
            d[key] = np.zeros_like(d[key])
    elif convs_kind.startswith("cos"):
        # tap 1 on the current token, the others N(0, e^2) with e such that
        # for independent tokens cos(U_0, U_m) = 1 / sqrt(1 + e^2 (K - 1))
        cos = float(convs_kind[3:])
        r = np.random.default_rng(seed + 200)
        for key, K in (("w4", 4), ("w8", 8), ("w12", 12)):
            e = np.sqrt((1.0 / cos ** 2 - 1.0) / (K - 1))
            v = (r.standard_normal((w.C, K)) * e).astype(np.float32)
            v[:, K - 1] = 1.0
            d[key] = v
    return d


def component_cosines(h, w):
    """Largest and median cosine over tokens between the output and each conv
    component (the oracle's TFA of the case's inputs)."""
    U = xo.tfa_components(h["out"], w.B, w.S, conv_tuple(h))
    cs = [np.sum(U[:, 0] * U[:, m], axis=1)
          / (np.linalg.norm(U[:, 0], axis=1) * np.linalg.norm(U[:, m], axis=1) + 1e-30) for m in range(1, 4)]
    return [(float(np.median(c)), float(np.max(c))) for c in cs]


def gate_code(gate):
    return xhc.XHC_GATE_UNIT if gate == "unit" else xhc.XHC_GATE_SIGMOID


def run_forward(w, dev, active, gate, gs=True, in_place=True):
    T, C, P = w.T, w.C, w.P
    X = dev["X"].clone()
    Xn = X if in_place else torch.empty_like(X)
    h_in = torch.empty(T, C, dtype=X.dtype, device=X.device)
    z_save = torch.empty(T, P + 1, dtype=torch.float32, device=X.device)
    xact = torch.empty(T, w.k, C, dtype=X.dtype, device=X.device)
    xhc.forward(X, dev["out"], dev["W"], active, Xn, h_in, B=w.B, S=w.S, bias=dev["bias"], z_save=z_save,
                xact_save=xact, iters=w.iters, eps=w.eps, gate_mode=gate_code(gate), w4=dev["w4"],
                w8=dev["w8"], w12=dev["w12"], gram_schmidt=gs, gs_eps=GS_EPS)
    torch.cuda.synchronize()
    return Xn, h_in, z_save, xact


def conv_tuple(h):
    return (h["w4"], h["w8"], h["w12"])


@pytest.mark.parametrize("name,w,active,gate,cv", CASES, ids=[c[0] for c in CASES])
def test_gs_forward_parity(name, w, active, gate, cv):
    say(f"[gs forward] {name} B={w.B} S={w.S} C={w.C} N={w.N} k={w.k} {w.dtype} convs={cv}")
    d = make_case(w, 0, False, cv)
    h = host_inputs(d)
    dev = device_inputs(d, w.dtype == "bf16")
    ref = xo.forward(h["X"], h["out"], h["W"], h["bias"], active, conv_tuple(h), B=w.B, S=w.S, iters=w.iters,
                     eps=w.eps, gate_mode=gate, gram_schmidt_on=True, gs_eps=GS_EPS)
    if cv.startswith("cos"):
        say(f"  cos(out, conv_m) median/max: {component_cosines(h, w)}")
    Xn, h_in, z_save, _ = run_forward(w, dev, active, gate)
    atol, rtol = tol(w)
    Xn_h = to_host(Xn)
    inactive = [i for i in range(w.N) if i not in active]
    assert np.array_equal(Xn_h[:, inactive], h["X"][:, inactive]), "pass-through rows differ"
    check_close("X_new[active]", Xn_h[:, active], ref["X_new"][:, active], atol, rtol)
    check_close("h_in", to_host(h_in), ref["h_in"], atol, rtol)
    check_close("z", to_host(z_save)[:, :w.P], ref["z"], atol, rtol)
    # the orthogonalisation matters here: the form without it is far off
    if cv == "leaning":
        plain = xo.forward(h["X"], h["out"], h["W"], h["bias"], active, conv_tuple(h), B=w.B, S=w.S,
                           iters=w.iters, eps=w.eps, gate_mode=gate)
        assert np.max(np.abs(plain["X_new"][:, active] - ref["X_new"][:, active])) > 20 * atol


@pytest.mark.parametrize("name,w,active,gate,cv", CASES, ids=[c[0] for c in CASES])
def test_gs_backward_parity(name, w, active, gate, cv):
    say(f"[gs backward] {name} B={w.B} S={w.S} C={w.C} N={w.N} k={w.k} {w.dtype} convs={cv}")
    d = make_case(w, 1, True, cv)
    h = host_inputs(d)
    dev = device_inputs(d, w.dtype == "bf16")
    g = xo.backward(h["X"], h["out"], h["W"], h["bias"], active, conv_tuple(h), h["dX_new"], h["dh_in"],
                    B=w.B, S=w.S, iters=w.iters, eps=w.eps, gate_mode=gate, gram_schmidt_on=True, gs_eps=GS_EPS)
    Xn, _, z_save, xact = run_forward(w, dev, active, gate)
    T, N, C, P = w.T, w.N, w.C, w.P

    def run(X, xact_, zsave):
        dXn = dev["dX_new"].clone()
        dX = torch.empty_like(dXn)
        dout = torch.empty(T, C, dtype=dXn.dtype, device=dXn.device)
        dW = torch.empty((N * C, P), dtype=torch.float32, device=dXn.device)
        db = torch.empty((P,), dtype=torch.float32, device=dXn.device)
        dws = {key: torch.empty((C, K), device=dXn.device) for key, K in (("dw4", 4), ("dw8", 8), ("dw12", 12))}
        xhc.backward(X, dev["out"], dev["W"], active, dXn, dev["dh_in"], dX, dout, dW, B=w.B, S=w.S, xact=xact_,
                     bias=dev["bias"], z_save=zsave, db=db, iters=w.iters, eps=w.eps, gate_mode=gate_code(gate),
                     w4=dev["w4"], w8=dev["w8"], w12=dev["w12"], gram_schmidt=True, gs_eps=GS_EPS, **dws)
        torch.cuda.synchronize()
        return dict(dX=dX, dout=dout, dW=dW, db=db, **dws)

    atol, rtol = tol(w)
    res = run(Xn, xact, z_save)
    check_close("dX", to_host(res["dX"]), g["dX"], atol, rtol)
    check_close("dout", to_host(res["dout"]), g["dout"], atol, rtol)
    if cv.startswith("cos") and w.dtype == "f32":
        # The stated limit of the coefficient form with nearly collinear
        # components in fp32: the triangle T comes from the fp32 Gram record,
        # and its error (about eps_fp32 cond(g)) times <G_a, U_m> reaches the
        # post logits' gradient, and through Ht and Sg the components'
        # gradient, of every token.  dX and dout stay at 1e-4; the sums over
        # tokens dW, db and the conv-weight gradients are held to 1e-3 of each
        # column's largest magnitude (db: of its largest entry) instead of
        # element by element (measured: about 1e-4 at cosine 0.999).
        for key, ref in (("dW", g["dW"]), ("db", g["db"]), ("dw4", g["dconv"][0]), ("dw8", g["dconv"][1]),
                         ("dw12", g["dconv"][2])):
            got = to_host(res[key])
            if ref.ndim == 1:                 # db: one sum per logit, held to the largest
                scale = np.abs(ref).max(keepdims=True)
                err = np.abs(got - ref).max(keepdims=True)
            else:
                scale = np.abs(ref).reshape(-1, ref.shape[-1]).max(axis=0)
                err = np.abs(got - ref).reshape(-1, ref.shape[-1]).max(axis=0)
            say(f"  {key}: max err / column scale = {np.max(err / scale):.3e}")
            assert (err <= 1e-3 * scale).all(), key
    else:
        check_close("dW", to_host(res["dW"]), g["dW"], atol, rtol)
        check_close("db", to_host(res["db"]), g["db"], atol, rtol)
        for m, key in enumerate(["dw4", "dw8", "dw12"]):
            check_close(key, to_host(res[key]), g["dconv"][m], atol, rtol)
    # recomputed coefficients give the same gradients; a rerun is bitwise identical
    res2 = run(dev["X"], None, None)
    for key in res:
        assert np.allclose(to_host(res[key]), to_host(res2[key]), rtol=1e-6, atol=1e-7), key
    res3 = run(Xn, xact, z_save)
    for key in res:
        assert torch.equal(res[key], res3[key]), f"{key} not deterministic"


def test_gs_with_zero_conv_weights_is_bitwise_the_plain_forward():
    # zero-initialised conv branches: the components past the output are 0,
    # the triangle is the identity, and the write is the one without it
    w = W_("z", 2, 50, 96, 16, 4, 4, "bf16", "fwd")
    d = make_case(w, 2, False, "zero")
    dev = device_inputs(d, True)
    a = run_forward(w, dev, [1, 2, 3, 4], "sigmoid", gs=True, in_place=False)
    b = run_forward(w, dev, [1, 2, 3, 4], "sigmoid", gs=False, in_place=False)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_gs_single_component_is_ignored():
    w = W_("s", 1, 40, 64, 4, 4, 1, "bf16", "fwd")
    d = synth.make_inputs(w, seed=3)
    dev = device_inputs(d, True)
    outs = []
    for gs in (False, True):
        X = dev["X"].clone()
        h_in = torch.empty(w.T, w.C, dtype=X.dtype, device=X.device)
        xhc.forward(X, dev["out"], dev["W"], [0, 1, 2, 3], X, h_in, B=w.B, S=w.S, bias=dev["bias"],
                    gram_schmidt=gs)
        torch.cuda.synchronize()
        outs.append((X, h_in))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_gs_chained_forward_matches_the_oracle_per_layer():
    # two chained sublayers with Gram-Schmidt: the carried projection and the
    # Gram pass of the second call's output
    w = W_("c", 2, 45, 200, 16, 4, 4, "bf16", "stack", layers=2)
    T, N, C, P = w.T, w.N, w.C, w.P
    d0 = make_case(w, 5, False, "leaning")
    X = to_dev(d0["X"], True).clone()
    layers = []
    for l in range(2):
        dl = make_case(w, 10 + l, False, "leaning")
        layers.append((device_inputs({k: dl[k] for k in ("out", "W", "w4", "w8", "w12", "bias")}, True),
                       host_inputs({k: dl[k] for k in ("out", "W", "w4", "w8", "w12", "bias")})))
    carry = torch.empty(xhc.carry_size(xhc.make_desc(w.B, w.S, C, N, 4, 4, xhc.XHC_BF16, gram_schmidt=True))
                        // 4, dtype=torch.float32, device=X.device)
    atol, rtol = tol(w)
    for l in range(2):
        dev, h = layers[l]
        active = synth.active_streams(l, N, 4)
        X_before = to_host(X)
        h_in = torch.empty(T, C, dtype=X.dtype, device=X.device)
        kw = dict(carry_in=carry if l > 0 else None, W_next=layers[1][0]["W"] if l == 0 else None,
                  carry_out=carry if l == 0 else None)
        xhc.forward(X, dev["out"], dev["W"], active, X, h_in, B=w.B, S=w.S, bias=dev["bias"], w4=dev["w4"],
                    w8=dev["w8"], w12=dev["w12"], gram_schmidt=True, gs_eps=GS_EPS, **kw)
        torch.cuda.synchronize()
        ref = xo.forward(X_before, h["out"], h["W"], h["bias"], active, conv_tuple(h), B=w.B, S=w.S,
                         gram_schmidt_on=True, gs_eps=GS_EPS)
        say(f"  layer {l}")
        Xh = to_host(X)
        check_close("X_new[active]", Xh[:, active], ref["X_new"][:, active], atol, rtol)
        check_close("h_in", to_host(h_in), ref["h_in"], atol, rtol)

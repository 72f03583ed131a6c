"""Pins of the oracle's modified Gram-Schmidt over the write-back components
(retrospective section "Conv 带来了新信息，也带来了新的麻烦"), no GPU.

The forward is pinned to numpy's QR factorisation (without the epsilon,
modified Gram-Schmidt without normalisation gives u~_c = R[c, c] q_c), to
the facts the pages fix (the output component is kept as it is, later
components lose their projections on earlier ones) and to closed forms; the
hand-written backward to central differences and to torch.autograd through
a separately written float64 forward."""

import numpy as np
import pytest
import torch

from oracle import xhc_oracle as xo

from test_oracle_backward import case, torch_forward


def rand_components(T=6, m=4, C=9, seed=0, corr=0.0):
    r = np.random.default_rng(seed)
    U = r.standard_normal((T, m, C))
    U[:, 1:] += corr * U[:, :1]          # conv-like components leaning on the output
    return U


def test_without_epsilon_equals_qr_columns_times_diagonal():
    U = rand_components(corr=0.8, seed=1)
    Ut, _ = xo.gram_schmidt(U, 0.0)
    for t in range(U.shape[0]):
        Q, R = np.linalg.qr(U[t].T)              # [C, 4] = Q R
        ref = (Q * np.diag(R)[None, :]).T        # row c = R[c, c] q_c
        np.testing.assert_allclose(Ut[t], ref, rtol=1e-11, atol=1e-11)


def test_output_component_is_kept_bitwise_and_spans_are_nested():
    U = rand_components(seed=2, corr=0.5)
    Ut, _ = xo.gram_schmidt(U, 1e-6)
    assert np.array_equal(Ut[:, 0], U[:, 0])
    for t in range(U.shape[0]):
        for c in range(1, 4):
            # u~_c - U_c lies in the span of U_0 .. U_{c-1}
            A = U[t, :c].T
            d = Ut[t, c] - U[t, c]
            coef, *_ = np.linalg.lstsq(A, d, rcond=None)
            assert np.linalg.norm(A @ coef - d) <= 1e-10 * max(1.0, np.linalg.norm(d))


def test_components_come_out_orthogonal():
    U = rand_components(T=20, C=64, seed=3, corr=1.5)
    Ut, _ = xo.gram_schmidt(U, 1e-6)
    for i in range(4):
        for j in range(i):
            cos = np.sum(Ut[:, i] * Ut[:, j], axis=1) / (
                np.linalg.norm(Ut[:, i], axis=1) * np.linalg.norm(Ut[:, j], axis=1))
            assert np.max(np.abs(cos)) < 1e-5


def test_collinear_component_closed_form():
    # U_1 = 2 U_0: u~_1 = 2 U_0 - 2|U_0|^2 / (|U_0|^2 + C eps) U_0 = 2 C eps / (|U_0|^2 + C eps) U_0
    U = rand_components(T=3, m=2, C=7, seed=4)
    U[:, 1] = 2.0 * U[:, 0]
    eps = 1e-3
    Ut, _ = xo.gram_schmidt(U, eps)
    n0 = np.sum(U[:, 0] ** 2, axis=1)
    ref = (2.0 * 7 * eps / (n0 + 7 * eps))[:, None] * U[:, 0]
    np.testing.assert_allclose(Ut[:, 1], ref, rtol=1e-9, atol=1e-15)


def test_zero_conv_branches_leave_the_forward_unchanged():
    # zero-initialised conv branches: every later component is 0 and stays 0
    c = case(seed=5)
    c["convs"] = [np.zeros_like(w) for w in c["convs"]]
    kw = dict(B=c["B"], S=c["S"])
    a = xo.forward(c["X"], c["out"], c["W"], c["bias"], c["active"], tuple(c["convs"]), **kw)
    b = xo.forward(c["X"], c["out"], c["W"], c["bias"], c["active"], tuple(c["convs"]),
                   gram_schmidt_on=True, **kw)
    assert np.array_equal(a["X_new"], b["X_new"]) and np.array_equal(a["U"], b["U"])
    assert np.all(np.isfinite(b["X_new"]))


def test_single_component_is_left_alone():
    c = case(ncomp=1, seed=6)
    kw = dict(B=c["B"], S=c["S"])
    a = xo.forward(c["X"], c["out"], c["W"], c["bias"], c["active"], (), **kw)
    b = xo.forward(c["X"], c["out"], c["W"], c["bias"], c["active"], (), gram_schmidt_on=True, **kw)
    assert np.array_equal(a["X_new"], b["X_new"])


def test_scaling_the_components_scales_the_result_without_epsilon():
    U = rand_components(seed=7, corr=0.6)
    a, _ = xo.gram_schmidt(U, 0.0)
    b, _ = xo.gram_schmidt(3.0 * U, 0.0)
    np.testing.assert_allclose(b, 3.0 * a, rtol=1e-12, atol=1e-12)


def test_gs_backward_is_the_adjoint_of_the_forward():
    U = rand_components(T=5, C=6, seed=8, corr=0.7)
    r = np.random.default_rng(9)
    dUt = r.standard_normal(U.shape)
    dU = xo.gram_schmidt_backward(U, 1e-3, dUt)
    h = 1e-6
    for _ in range(4):
        V = r.standard_normal(U.shape)
        fp, _ = xo.gram_schmidt(U + h * V, 1e-3)
        fm, _ = xo.gram_schmidt(U - h * V, 1e-3)
        fd = np.sum(dUt * (fp - fm)) / (2 * h)
        assert abs(fd - np.sum(dU * V)) <= 1e-7 * max(1.0, abs(fd))


@pytest.mark.parametrize("gate_mode", ["sigmoid", "unit"])
def test_backward_with_gs_matches_central_differences(gate_mode):
    c = case(seed=10)
    kw = dict(B=c["B"], S=c["S"], gate_mode=gate_mode, gram_schmidt_on=True, gs_eps=1e-4)

    def loss(cc):
        f = xo.forward(cc["X"], cc["out"], cc["W"], cc["bias"], cc["active"], tuple(cc["convs"]), **kw)
        return np.sum(f["X_new"] * cc["dX_new"]) + np.sum(f["h_in"] * cc["dh_in"])

    g = xo.backward(c["X"], c["out"], c["W"], c["bias"], c["active"], tuple(c["convs"]),
                    c["dX_new"], c["dh_in"], **kw)
    r = np.random.default_rng(11)
    h = 1e-5
    targets = [("X", g["dX"]), ("out", g["dout"]), ("W", g["dW"])]
    targets += [(("convs", m), g["dconv"][m]) for m in range(3)]
    for name, grad in targets:
        for _ in range(2):
            V = r.standard_normal(grad.shape)
            cp, cm = dict(c), dict(c)
            if isinstance(name, tuple):
                m = name[1]
                cp["convs"] = list(c["convs"]); cm["convs"] = list(c["convs"])
                cp["convs"][m] = c["convs"][m] + h * V
                cm["convs"][m] = c["convs"][m] - h * V
            else:
                cp[name] = c[name] + h * V
                cm[name] = c[name] - h * V
            fd = (loss(cp) - loss(cm)) / (2 * h)
            an = np.sum(grad * V)
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_backward_with_gs_matches_torch_autograd():
    c = case(B=2, S=15, C=6, N=16, k=4, seed=12, scale_w=0.6)
    g = xo.backward(c["X"], c["out"], c["W"], c["bias"], c["active"], tuple(c["convs"]),
                    c["dX_new"], c["dh_in"], B=c["B"], S=c["S"], gram_schmidt_on=True, gs_eps=1e-3)
    t = {n: torch.tensor(c[n], requires_grad=True) for n in ("X", "out", "W", "bias")}
    tc = [torch.tensor(w, requires_grad=True) for w in c["convs"]]
    Xn, h = torch_forward(t["X"], t["out"], t["W"], t["bias"], c["active"], tc, c["B"], c["S"], gs_eps=1e-3)
    (Xn * torch.tensor(c["dX_new"])).sum().add((h * torch.tensor(c["dh_in"])).sum()).backward()
    np.testing.assert_allclose(g["dX"], t["X"].grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(g["dout"], t["out"].grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(g["dW"], t["W"].grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(g["db"], t["bias"].grad.numpy(), rtol=1e-9, atol=1e-10)
    for m in range(3):
        np.testing.assert_allclose(g["dconv"][m], tc[m].grad.numpy(), rtol=1e-9, atol=1e-10)

"""Pins of the oracle's hand-derived backward pass (no GPU): central finite
differences of the oracle's own forward, torch.autograd through a separately
written float64 forward, adjoint identities and the invariances of Sinkhorn."""

import numpy as np
import pytest
import torch

from oracle import xhc_oracle as xo


def case(B=2, S=13, C=4, N=5, k=3, ncomp=4, seed=0, scale_w=0.4):
    r = np.random.default_rng(seed)
    T = B * S
    P = xo.n_logits(N, k, ncomp)
    return dict(
        X=r.standard_normal((T, N, C)), out=r.standard_normal((T, C)),
        W=r.standard_normal((N * C, P)) * scale_w, bias=r.standard_normal(P) * 0.3,
        convs=[r.standard_normal((C, K)) * 0.4 for K in (4, 8, 12)[:ncomp - 1]],
        active=list(r.permutation(N)[:k]), B=B, S=S,
        dX_new=r.standard_normal((T, N, C)), dh_in=r.standard_normal((T, C)))


def loss(c, **kw):
    f = xo.forward(c["X"], c["out"], c["W"], c["bias"], c["active"], tuple(c["convs"]),
                   B=c["B"], S=c["S"], **kw)
    return np.sum(f["X_new"] * c["dX_new"]) + np.sum(f["h_in"] * c["dh_in"])


def grads(c, **kw):
    return xo.backward(c["X"], c["out"], c["W"], c["bias"], c["active"], tuple(c["convs"]),
                       c["dX_new"], c["dh_in"], B=c["B"], S=c["S"], **kw)


@pytest.mark.parametrize("ncomp,gate_mode", [(4, "sigmoid"), (1, "sigmoid"), (4, "unit")])
def test_backward_matches_central_differences(ncomp, gate_mode):
    c = case(ncomp=ncomp, seed=1)
    g = grads(c, gate_mode=gate_mode)
    r = np.random.default_rng(2)
    h = 1e-5
    targets = [("X", g["dX"]), ("out", g["dout"]), ("W", g["dW"]), ("bias", g["db"])]
    targets += [(("convs", m), g["dconv"][m]) for m in range(ncomp - 1)]
    for name, grad in targets:
        for _ in range(3):
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
            fd = (loss(cp, gate_mode=gate_mode) - loss(cm, gate_mode=gate_mode)) / (2 * h)
            an = np.sum(grad * V)
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def torch_mgs(U, gs_eps):
    """Modified Gram-Schmidt over dim 1 of [T, m, C], written apart from the oracle."""
    C = U.shape[2]
    done = [U[:, 0]]
    for c in range(1, U.shape[1]):
        v = U[:, c]
        for q in done:
            v = v - ((v * q).sum(dim=1) / ((q * q).sum(dim=1) + C * gs_eps))[:, None] * q
        done.append(v)
    return torch.stack(done, dim=1)


def torch_forward(X, out, W, bias, active, convs, B, S, iters=20, eps=1e-6, gs_eps=None):
    """A separately written float64 forward in torch, for autograd (gs_eps:
    None, or the epsilon of Gram-Schmidt over the components)."""
    T, N, C = X.shape
    k = len(active)
    nc = 1 + len(convs)
    flat = X.reshape(T, N * C)
    rms = torch.sqrt((flat ** 2).mean(dim=1, keepdim=True) + eps)
    z = (flat / rms) @ W + bias
    hpre = torch.sigmoid(z[:, :N])
    hpost = torch.sigmoid(z[:, N:N + k * nc]).reshape(T, k, nc)
    M = torch.exp(z[:, N + k * nc:].reshape(T, k, k))
    for _ in range(iters):
        M = M / M.sum(dim=2, keepdim=True)
        M = M / M.sum(dim=1, keepdim=True)
    h_in = (hpre[:, :, None] * X).sum(dim=1)
    seq = out.reshape(B, S, C).permute(0, 2, 1)
    comps = [out]
    for w in convs:
        K = w.shape[1]
        y = torch.nn.functional.conv1d(torch.nn.functional.pad(seq, (K - 1, 0)), w[:, None, :], groups=C)
        comps.append(y.permute(0, 2, 1).reshape(T, C))
    U = torch.stack(comps, dim=1)
    if gs_eps is not None:
        U = torch_mgs(U, gs_eps)
    rows = []
    idx = list(active)
    for i in range(N):
        if i in idx:
            a = idx.index(i)
            rows.append(torch.einsum("tb,tbc->tc", M[:, a], X[:, idx]) +
                        torch.einsum("tm,tmc->tc", hpost[:, a], U))
        else:
            rows.append(X[:, i])
    return torch.stack(rows, dim=1), h_in


def test_backward_matches_torch_autograd():
    c = case(B=2, S=17, C=6, N=16, k=4, seed=3, scale_w=0.6)
    g = grads(c)
    t = {n: torch.tensor(c[n], requires_grad=True) for n in ("X", "out", "W", "bias")}
    tc = [torch.tensor(w, requires_grad=True) for w in c["convs"]]
    Xn, h = torch_forward(t["X"], t["out"], t["W"], t["bias"], c["active"], tc, c["B"], c["S"])
    (Xn * torch.tensor(c["dX_new"])).sum().add((h * torch.tensor(c["dh_in"])).sum()).backward()
    np.testing.assert_allclose(g["dX"], t["X"].grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(g["dout"], t["out"].grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(g["dW"], t["W"].grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(g["db"], t["bias"].grad.numpy(), rtol=1e-9, atol=1e-10)
    for m in range(3):
        np.testing.assert_allclose(g["dconv"][m], tc[m].grad.numpy(), rtol=1e-9, atol=1e-10)


def test_sinkhorn_gradient_is_shift_invariant():
    # The iterations start with a row step, so H_res does not change when a
    # constant is added to a row of the logits: the logit gradient sums to
    # zero along each row, for any iteration count.
    r = np.random.default_rng(4)
    L = r.standard_normal((40, 4, 4)) * 2.5
    dH = r.standard_normal((40, 4, 4))
    for iters in (1, 20):
        dL = xo.sinkhorn_backward(L, iters, dH)
        np.testing.assert_allclose(dL.sum(axis=2), 0.0, atol=1e-12)
        assert np.abs(dL).max() > 1e-3


def test_conv_backward_is_the_adjoint():
    r = np.random.default_rng(5)
    B, S, C = 2, 19, 3
    o = r.standard_normal((B, S, C))
    for K in (4, 8, 12):
        w = r.standard_normal((C, K))
        dy = r.standard_normal((B, S, C))
        y = xo.causal_depthwise_conv(o, w)
        d_o, d_w = xo.causal_depthwise_conv_backward(o, w, dy)
        # <conv(o), dy> = <o, conv^T dy>, and the loss is bilinear in (o, w)
        np.testing.assert_allclose(np.sum(y * dy), np.sum(o * d_o), rtol=1e-12)
        np.testing.assert_allclose(np.sum(y * dy), np.sum(w * d_w), rtol=1e-12)


def test_unit_gates_give_no_gate_gradient():
    c = case(seed=6)
    g = grads(c, gate_mode="unit")
    N, k = c["X"].shape[1], len(c["active"])
    assert np.count_nonzero(g["dz"][:, :N + k * 4]) == 0

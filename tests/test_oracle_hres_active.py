"""Pins of the oracle's O9 (H_res generated from the k active rows, normed by
their own RMS; the retrospective's section on the dense read and sparse
write credits the sparse write with cutting H_res's generation cost from
N^3 C to k^3 C).  None restates the oracle's formula:
  - with every stream active it is the full-state form (O1), which has its
    own pins;
  - H_res does not depend on the untouched rows, nor on the res columns of
    W on their rows, while H_pre still does;
  - the res logits are invariant to scaling the active rows (their own
    RMS), which the full-state normaliser is not;
  - the backward against central differences and against torch.autograd
    through a separately written torch forward."""
import numpy as np
import pytest
import torch

from oracle import xhc_oracle as xo
from tests.test_oracle_backward import case


def fwd(c, **kw):
    return xo.forward(c["X"], c["out"], c["W"], c["bias"], c["active"], tuple(c["convs"]), B=c["B"], S=c["S"],
                      **kw)


def bwd(c, **kw):
    return xo.backward(c["X"], c["out"], c["W"], c["bias"], c["active"], tuple(c["convs"]), c["dX_new"],
                       c["dh_in"], B=c["B"], S=c["S"], **kw)


@pytest.mark.parametrize("perm", [False, True])
def test_every_stream_active_is_the_full_state_form(perm):
    c = case(N=4, k=4, seed=11)
    c["active"] = [2, 0, 3, 1] if perm else [0, 1, 2, 3]
    a, b = fwd(c, hres_active=True), fwd(c)
    for key in ("X_new", "h_in", "z"):
        np.testing.assert_allclose(a[key], b[key], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a["r_act"], b["r"], rtol=1e-14)
    ga, gb = bwd(c, hres_active=True), bwd(c)
    for key in ("dX", "dout", "dW", "db"):
        np.testing.assert_allclose(ga[key], gb[key], rtol=1e-10, atol=1e-11)


def test_res_logits_ignore_the_untouched_rows():
    c = case(N=7, k=3, seed=12)
    N, k, C, P = 7, 3, c["X"].shape[2], c["W"].shape[1]
    res0 = N + k * 4
    base = fwd(c, hres_active=True)
    inactive = [i for i in range(N) if i not in c["active"]]
    r = np.random.default_rng(13)
    c2 = dict(c)
    c2["X"] = c["X"].copy()
    c2["X"][:, inactive] = r.standard_normal(c2["X"][:, inactive].shape) * 3.0
    c2["W"] = c["W"].copy()
    Wv = c2["W"].reshape(N, C, P)
    Wv[inactive, :, res0:] = r.standard_normal(Wv[inactive, :, res0:].shape)
    other = fwd(c2, hres_active=True)
    np.testing.assert_allclose(other["H_res"], base["H_res"], rtol=1e-13, atol=1e-14)
    assert np.abs(other["H_pre"] - base["H_pre"]).max() > 1e-3
    # the full-state form does see them
    assert np.abs(fwd(c2)["H_res"] - fwd(c)["H_res"]).max() > 1e-3
    # and the gradient never reaches W's res columns on those rows
    g = bwd(c, hres_active=True)
    assert np.count_nonzero(g["dW"].reshape(N, C, P)[inactive, :, res0:]) == 0
    assert np.abs(g["dW"].reshape(N, C, P)[c["active"], :, res0:]).max() > 1e-3


def test_res_logits_follow_the_active_rows_own_scale():
    c = case(N=6, k=2, seed=14)
    c["bias"] = np.zeros_like(c["bias"])
    N, k = 6, 2
    res0 = N + k * 4
    c2 = dict(c)
    c2["X"] = c["X"].copy()
    c2["X"][:, c["active"]] *= 7.0
    a = fwd(c, hres_active=True, eps=0.0)
    b = fwd(c2, hres_active=True, eps=0.0)
    np.testing.assert_allclose(b["z"][:, res0:], a["z"][:, res0:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b["r_act"], 7.0 * a["r_act"], rtol=1e-13)
    # the full-state normaliser changes its res logits under the same scaling
    assert np.abs(fwd(c2, eps=0.0)["z"][:, res0:] - fwd(c, eps=0.0)["z"][:, res0:]).max() > 1e-2


@pytest.mark.parametrize("ncomp", [4, 1])
def test_backward_matches_central_differences(ncomp):
    c = case(N=6, k=3, ncomp=ncomp, seed=15)
    g = bwd(c, hres_active=True)

    def loss(cc):
        f = fwd(cc, hres_active=True)
        return np.sum(f["X_new"] * c["dX_new"]) + np.sum(f["h_in"] * c["dh_in"])

    r = np.random.default_rng(16)
    h = 1e-5
    for name, grad in (("X", g["dX"]), ("W", g["dW"]), ("bias", g["db"]), ("out", g["dout"])):
        for _ in range(3):
            V = r.standard_normal(grad.shape)
            cp, cm = dict(c), dict(c)
            cp[name] = c[name] + h * V
            cm[name] = c[name] - h * V
            fd = (loss(cp) - loss(cm)) / (2 * h)
            an = np.sum(grad * V)
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def torch_forward_hres_active(X, out, W, bias, active, convs, B, S, eps=1e-6):
    """The res logits of torch_forward's computation replaced by a
    projection of the active rows alone (written apart from the oracle):
    the rows' own RMS, and W's rows of those streams."""
    T, N, C = X.shape
    k = len(active)
    nc = 1 + len(convs)
    res0 = N + k * nc
    xa = torch.cat([X[:, i] for i in active], dim=1)                    # [T, k*C]
    ra = torch.sqrt((xa ** 2).mean(dim=1, keepdim=True) + eps)
    Wa = torch.cat([W[i * C:(i + 1) * C, res0:] for i in active], dim=0)  # [k*C, k*k]
    La = (xa / ra) @ Wa + bias[res0:]
    # the full-state logits, with the res part taken from La
    Wz = torch.cat([W[:, :res0], torch.zeros_like(W[:, res0:])], dim=1)
    bz = torch.cat([bias[:res0], torch.zeros_like(bias[res0:])])

    flat = X.reshape(T, N * C)
    rms = torch.sqrt((flat ** 2).mean(dim=1, keepdim=True) + eps)
    z = (flat / rms) @ Wz + bz
    z = torch.cat([z[:, :res0], La], dim=1)
    return z


def test_backward_matches_torch_autograd():
    c = case(B=2, S=11, C=5, N=16, k=4, seed=17, scale_w=0.6)
    g = bwd(c, hres_active=True)
    t = {n: torch.tensor(c[n], requires_grad=True) for n in ("X", "out", "W", "bias")}
    tc = [torch.tensor(w, requires_grad=True) for w in c["convs"]]
    z = torch_forward_hres_active(t["X"], t["out"], t["W"], t["bias"], c["active"], tc, c["B"], c["S"])
    # the rest of the sublayer (gates, Sinkhorn, TFA, write) in torch too
    np.testing.assert_allclose(fwd(c, hres_active=True)["z"], z.detach().numpy(), rtol=1e-12, atol=1e-12)
    Xn, h = _sublayer_from_logits(z, t["X"], t["out"], c["active"], tc, c["B"], c["S"])
    (Xn * torch.tensor(c["dX_new"])).sum().add((h * torch.tensor(c["dh_in"])).sum()).backward()
    np.testing.assert_allclose(g["dX"], t["X"].grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(g["dout"], t["out"].grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(g["dW"], t["W"].grad.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(g["db"], t["bias"].grad.numpy(), rtol=1e-9, atol=1e-10)
    for m in range(3):
        np.testing.assert_allclose(g["dconv"][m], tc[m].grad.numpy(), rtol=1e-9, atol=1e-10)


def _sublayer_from_logits(z, X, out, active, convs, B, S, iters=20):
    """Gates, Sinkhorn, TFA and the write from given logits (torch)."""
    T, N, C = X.shape
    k = len(active)
    nc = 1 + len(convs)
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
    rows = []
    idx = list(active)
    for i in range(N):
        if i in idx:
            a = idx.index(i)
            rows.append(torch.einsum("tb,tbc->tc", M[:, a], X[:, idx]) + torch.einsum("tm,tmc->tc", hpost[:, a], U))
        else:
            rows.append(X[:, i])
    return torch.stack(rows, dim=1), h_in

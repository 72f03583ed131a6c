"""Pins of the oracle's router (reading O7: fixed + routed streams chosen per
token from a LayerNorm'd flattened state, sigmoid scores scaling the routed
write-back), against torch's layer_norm, brute-force ordering, the fixed-list
forward it must reduce to, torch.autograd through a separately written
routed forward, and central differences.  No GPU."""

import itertools

import numpy as np
import pytest
import torch

from oracle import xhc_oracle as xo


def case(B=2, S=11, C=4, N=8, k=4, R=2, ncomp=4, seed=0, scale_w=0.4, scale_r=0.6):
    r = np.random.default_rng(seed)
    T = B * S
    P = xo.n_logits(N, k, ncomp)
    return dict(
        X=r.standard_normal((T, N, C)), out=r.standard_normal((T, C)),
        W=r.standard_normal((N * C, P)) * scale_w, bias=r.standard_normal(P) * 0.3,
        Wr=r.standard_normal((N * C, N)) * scale_r, br=r.standard_normal(N) * 0.5,
        convs=[r.standard_normal((C, K)) * 0.4 for K in (4, 8, 12)[:ncomp - 1]],
        active=list(r.permutation(N)[:k]), R=R, B=B, S=S,
        dX_new=r.standard_normal((T, N, C)), dh_in=r.standard_normal((T, C)))


def fwd(c, **kw):
    return xo.forward(c["X"], c["out"], c["W"], c["bias"], c["active"], tuple(c["convs"]), B=c["B"], S=c["S"],
                      route=c["R"], W_route=c["Wr"], b_route=c["br"], **kw)


def bwd(c, **kw):
    return xo.backward(c["X"], c["out"], c["W"], c["bias"], c["active"], tuple(c["convs"]), c["dX_new"],
                       c["dh_in"], B=c["B"], S=c["S"], route=c["R"], W_route=c["Wr"], b_route=c["br"], **kw)


def test_layer_norm_matches_torch():
    r = np.random.default_rng(1)
    Xf = r.standard_normal((37, 96)) * 3.0 + 1.7
    y, mu, sd = xo.layer_norm_flat(Xf, 1e-6)
    ref = torch.nn.functional.layer_norm(torch.tensor(Xf), (96,), eps=1e-6).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mu, Xf.mean(axis=1), rtol=1e-13)
    np.testing.assert_allclose(sd, np.sqrt(Xf.var(axis=1) + 1e-6), rtol=1e-13)


@pytest.mark.parametrize("N,fixed,R", [(16, [3, 9], 2), (8, [0, 1, 2], 1), (6, [], 4), (5, [4], 3)])
def test_route_select_matches_brute_force(N, fixed, R):
    # integer scores so that ties are frequent; order by (-score, stream id)
    r = np.random.default_rng(2)
    rho = r.integers(-3, 4, size=(200, N)).astype(np.float64)
    idx = xo.route_select(rho, fixed, R)
    for t in range(rho.shape[0]):
        cand = [i for i in range(N) if i not in fixed]
        best = sorted(cand, key=lambda i: (-rho[t, i], i))[:R]
        assert list(idx[t]) == list(fixed) + best, t
        # and the chosen set has the largest score sum of all R-subsets
        top = max(sum(rho[t, list(sub)]) for sub in itertools.combinations(cand, R))
        assert sum(rho[t, best]) == top


def test_router_with_saturated_scores_is_the_fixed_list():
    # W_route = 0: every token chooses the same two streams, and scores of
    # +40 / +39 give s == 1 exactly in float64, so the update is the
    # fixed-list update with active = fixed + chosen (in score order)
    c = case(N=16, seed=3)
    fixed = c["active"][:2]
    rest = [i for i in range(16) if i not in fixed]
    c["Wr"] = np.zeros_like(c["Wr"])
    c["br"] = np.full(16, -40.0)
    c["br"][rest[5]], c["br"][rest[2]] = 40.0, 39.0
    f = fwd(c)
    assert (f["idx"] == np.array(fixed + [rest[5], rest[2]])).all()
    assert (f["s"] == 1.0).all()
    ref = xo.forward(c["X"], c["out"], c["W"], c["bias"], fixed + [rest[5], rest[2]], tuple(c["convs"]),
                     B=c["B"], S=c["S"])
    np.testing.assert_allclose(f["X_new"], ref["X_new"], rtol=0, atol=1e-13)
    np.testing.assert_array_equal(f["h_in"], ref["h_in"])


def test_router_scale_multiplies_the_write_back_only():
    c = case(N=16, seed=4)
    fixed = c["active"][:2]
    rest = [i for i in range(16) if i not in fixed]
    c["Wr"] = np.zeros_like(c["Wr"])
    c["br"] = np.linspace(-2.0, 1.0, 16)
    c["br"][rest[0]] = 0.3                      # a mid-sized score for one chosen stream
    f = fwd(c)
    idx = f["idx"][0]
    assert (f["idx"] == idx).all()
    want_s = 1.0 / (1.0 + np.exp(-c["br"][idx[2:]]))
    np.testing.assert_allclose(f["s"][:, 2:], np.broadcast_to(want_s, (f["s"].shape[0], 2)), rtol=1e-15)
    ref = xo.forward(c["X"], c["out"], c["W"], c["bias"], list(idx), tuple(c["convs"]), B=c["B"], S=c["S"])
    mix = np.einsum("tab,tbc->tac", ref["H_res"], c["X"][:, list(idx)])
    wb = ref["X_new"][:, list(idx)] - mix       # the unscaled write-back
    got = f["X_new"][:, list(idx)] - mix
    np.testing.assert_allclose(got[:, :2], wb[:, :2], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got[:, 2:], want_s[None, :, None] * wb[:, 2:], rtol=1e-12, atol=1e-13)
    others = [i for i in range(16) if i not in idx]
    np.testing.assert_array_equal(f["X_new"][:, others], c["X"][:, others])


def torch_routed_forward(X, out, W, bias, Wr, br, idx, R, convs, B, S, iters=20, eps=1e-6):
    """A separately written float64 routed forward in torch; idx [T, k] is
    the per-token active list (fixed streams first, then the routed ones)."""
    T, N, C = X.shape
    k = idx.shape[1]
    nc = 1 + len(convs)
    flat = X.reshape(T, N * C)
    z = flat / torch.sqrt((flat ** 2).mean(dim=1, keepdim=True) + eps) @ W + bias
    hpre = torch.sigmoid(z[:, :N])
    hpost = torch.sigmoid(z[:, N:N + k * nc]).reshape(T, k, nc)
    M = torch.exp(z[:, N + k * nc:].reshape(T, k, k))
    for _ in range(iters):
        M = M / M.sum(dim=2, keepdim=True)
        M = M / M.sum(dim=1, keepdim=True)
    rho = torch.nn.functional.layer_norm(flat, (N * C,), eps=eps) @ Wr + br
    s = torch.cat([torch.ones(T, k - R, dtype=X.dtype), torch.sigmoid(torch.gather(rho, 1, idx[:, k - R:]))], 1)
    h_in = (hpre[:, :, None] * X).sum(dim=1)
    seq = out.reshape(B, S, C).permute(0, 2, 1)
    comps = [out]
    for w in convs:
        K = w.shape[1]
        y = torch.nn.functional.conv1d(torch.nn.functional.pad(seq, (K - 1, 0)), w[:, None, :], groups=C)
        comps.append(y.permute(0, 2, 1).reshape(T, C))
    U = torch.stack(comps, dim=1)
    gi = idx[:, :, None].expand(T, k, C)
    Xa = torch.gather(X, 1, gi)
    new = torch.einsum("tab,tbc->tac", M, Xa) + s[:, :, None] * torch.einsum("tam,tmc->tac", hpost, U)
    return X.scatter(1, gi, new), h_in


@pytest.mark.parametrize("N,k,R", [(16, 4, 2), (8, 3, 1), (6, 4, 4)])
def test_router_backward_matches_torch_autograd(N, k, R):
    c = case(N=N, k=k, R=R, C=5, seed=5)
    f = fwd(c)
    g = bwd(c)
    names = ("X", "out", "W", "bias", "Wr", "br")
    t = {n: torch.tensor(c[n], requires_grad=True) for n in names}
    tc = [torch.tensor(w, requires_grad=True) for w in c["convs"]]
    Xn, h = torch_routed_forward(t["X"], t["out"], t["W"], t["bias"], t["Wr"], t["br"],
                                 torch.tensor(f["idx"]), R, tc, c["B"], c["S"])
    np.testing.assert_allclose(Xn.detach().numpy(), f["X_new"], rtol=1e-12, atol=1e-12)
    (Xn * torch.tensor(c["dX_new"])).sum().add((h * torch.tensor(c["dh_in"])).sum()).backward()
    for n, gk in zip(names, ("dX", "dout", "dW", "db", "dW_route", "db_route")):
        np.testing.assert_allclose(g[gk], t[n].grad.numpy(), rtol=1e-9, atol=1e-10, err_msg=n)
    for m in range(3):
        np.testing.assert_allclose(g["dconv"][m], tc[m].grad.numpy(), rtol=1e-9, atol=1e-10)


def test_router_backward_matches_central_differences():
    # well separated scores, so that no step of size h changes a choice
    c = case(N=8, k=4, R=2, C=3, seed=6, scale_r=0.05)
    c["br"] = np.arange(8, dtype=np.float64) * 1.5 - 4.0
    g = bwd(c)

    def loss(cc):
        f = fwd(cc)
        assert (f["idx"] == g["idx"]).all()
        return np.sum(f["X_new"] * cc["dX_new"]) + np.sum(f["h_in"] * cc["dh_in"])

    r = np.random.default_rng(7)
    h = 1e-5
    for name, grad in [("X", g["dX"]), ("Wr", g["dW_route"]), ("br", g["db_route"]), ("W", g["dW"])]:
        for _ in range(3):
            V = r.standard_normal(grad.shape)
            cp, cm = dict(c), dict(c)
            cp[name] = c[name] + h * V
            cm[name] = c[name] - h * V
            fd = (loss(cp) - loss(cm)) / (2 * h)
            an = np.sum(grad * V)
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_only_chosen_scores_receive_gradient():
    c = case(N=16, seed=8)
    g = bwd(c)
    T = c["X"].shape[0]
    chosen = np.zeros((T, 16), dtype=bool)
    chosen[np.arange(T)[:, None], g["idx"][:, 2:]] = True
    assert (g["drho"][~chosen] == 0).all()
    assert (np.abs(g["drho"][chosen]) > 0).all()
    # the fixed streams are never scored, so their router columns get nothing
    fixed = c["active"][:2]
    assert (g["db_route"][fixed] == 0).all() and (g["dW_route"][:, fixed] == 0).all()
    # and the per-token active lists hold distinct streams, fixed ones first
    assert (g["idx"][:, :2] == fixed).all()
    assert all(len(set(row)) == 4 for row in g["idx"])


def test_given_lists_are_each_tokens_fixed_list():
    # O8: a per-token list makes token t's update the fixed-list update with
    # that list (the write of a token depends on its own list only; the TFA
    # components and the dense read do not depend on the lists at all)
    c = case(N=8, k=3, R=0, C=4, seed=9)
    T = c["X"].shape[0]
    r = np.random.default_rng(10)
    lists = np.stack([r.permutation(8)[:3] for _ in range(T)])
    f = xo.forward(c["X"], c["out"], c["W"], c["bias"], [0, 1, 2], tuple(c["convs"]), B=c["B"], S=c["S"],
                   active_tok=lists)
    g = xo.backward(c["X"], c["out"], c["W"], c["bias"], [0, 1, 2], tuple(c["convs"]), c["dX_new"], c["dh_in"],
                    B=c["B"], S=c["S"], active_tok=lists)
    dW = np.zeros_like(g["dW"])
    for t in range(T):
        lt = list(lists[t])
        ft = xo.forward(c["X"], c["out"], c["W"], c["bias"], lt, tuple(c["convs"]), B=c["B"], S=c["S"])
        np.testing.assert_array_equal(f["X_new"][t], ft["X_new"][t])
        # the gradient of token t's own terms: token t's upstream gradient only
        cc = dict(c)
        cc["dX_new"] = np.zeros_like(c["dX_new"]); cc["dX_new"][t] = c["dX_new"][t]
        cc["dh_in"] = np.zeros_like(c["dh_in"]); cc["dh_in"][t] = c["dh_in"][t]
        gt = xo.backward(c["X"], c["out"], c["W"], c["bias"], lt, tuple(c["convs"]), cc["dX_new"], cc["dh_in"],
                         B=c["B"], S=c["S"])
        np.testing.assert_allclose(g["dX"][t], gt["dX"][t], rtol=1e-12, atol=1e-12)
        dW += gt["dW"]
    np.testing.assert_array_equal(f["h_in"], xo.forward(c["X"], c["out"], c["W"], c["bias"], [0, 1, 2],
                                                       tuple(c["convs"]), B=c["B"], S=c["S"])["h_in"])
    np.testing.assert_allclose(g["dW"], dW, rtol=1e-10, atol=1e-10)

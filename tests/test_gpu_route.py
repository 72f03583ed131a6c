"""GPU parity of the router (desc.route = R > 0: the first k - R active
streams fixed, the other R slots chosen per token by sigmoid scores over the
LayerNorm'd flattened state, the routed write-back scaled by the score)
against the oracle, through the C ABI.

The choice is an integer decided by floating point.  The library decides on
fp32 scores, the oracle on fp64 ones, so near ties may go either way; the
tests therefore check that every GPU choice is a valid top-R under the
oracle's scores within a score tolerance, that it agrees with the oracle's
own choice on all but a small share of tokens, and then compare every
output with the oracle run on the GPU's choice.  With W_route = 0 the scores
are exactly b_route in both, and the choice (ties included) must match bit
for bit.

Tolerances as in the other parity tests: fp32 max|err| <= 1e-4 + 1e-4 |ref|,
bf16 <= 1e-2 + 1e-2 |ref|; pass-through rows bit-exact."""
import numpy as np
import pytest
import torch

from oracle import xhc_oracle as xo
from residual_stream_architecture_amd import synth
from residual_stream_architecture_amd import xhc
from tests.gpu_util import check_close, device_inputs, host_inputs, say, to_host

pytestmark = pytest.mark.gpu
W_ = synth.Workload

# name, workload (route = R), fixed streams
CASES = [
    ("tiny_f32", W_("r", 1, 64, 64, 16, 4, 4, "f32", "fwdbwd", route=2), [0, 1]),
    ("ragged_bf16", W_("r", 2, 77, 136, 16, 4, 4, "bf16", "fwdbwd", route=2), [5, 12]),
    ("n8_k3_r1_f32", W_("r", 3, 30, 40, 8, 3, 4, "f32", "fwdbwd", route=1), [6, 1]),
    ("all_routed_n6_f32", W_("r", 2, 25, 48, 6, 4, 4, "f32", "fwdbwd", route=4), []),
    ("fix1_r3_bf16", W_("r", 2, 41, 96, 16, 4, 4, "bf16", "fwdbwd", route=3), [7]),
    ("nc1_bf16", W_("r", 2, 50, 64, 16, 4, 1, "bf16", "fwdbwd", route=2), [3, 9]),
    ("gs_bf16", W_("r", 2, 77, 136, 16, 4, 4, "bf16", "fwdbwd", gs=True, route=2), [5, 12]),
    ("wide_bf16", W_("r", 1, 130, 1040, 16, 4, 4, "bf16", "fwdbwd", route=2), [4, 5]),
    ("edge_c8_s1_f32", W_("r", 4, 1, 8, 16, 4, 4, "f32", "fwdbwd", route=2), [0, 15]),
    # one routed stream and nothing fixed: 15 candidates
    ("k1_n15_r1_f32", W_("r", 2, 37, 48, 15, 1, 4, "f32", "fwdbwd", route=1), []),
    ("nc1_f32", W_("r", 2, 29, 56, 12, 3, 1, "f32", "fwdbwd", route=2), [4]),
    # nothing fixed at N = 16: all 16 streams are candidates (a full router tile)
    ("all_routed_n16_f32", W_("r", 2, 45, 64, 16, 4, 4, "f32", "fwdbwd", route=4), []),
    ("all_routed_n16_bf16", W_("r", 2, 77, 136, 16, 2, 4, "bf16", "fwdbwd", route=2), []),
]
GS_EPS = 1e-6


def tol(w):
    return (1e-4, 1e-4) if w.dtype == "f32" else (1e-2, 1e-2)


def tol_logits(w):
    """Tolerance of the intermediates (logits z, scores rho, and the score
    slack of check_choice): the fp32 path sums in fp32 throughout, the bf16
    one rounds its inputs to bf16 but still accumulates in fp32."""
    return (1e-4, 1e-4) if w.dtype == "f32" else (1e-3, 1e-3)


def slack(w):
    return (2e-4, 1e-4) if w.dtype == "f32" else (2e-3, 1e-3)


def inputs(w, seed, grads):
    d = synth.make_inputs(w, seed=seed, grads=grads)
    d.update(synth.make_router(w, seed))
    return d


def host_kw(h, w, fixed, gate="sigmoid"):
    convs = (h["w4"], h["w8"], h["w12"]) if w.ncomp == 4 else ()
    return dict(args=(h["X"], h["out"], h["W"], h["bias"], list(fixed) + [0] * w.route, convs),
                kw=dict(B=w.B, S=w.S, iters=w.iters, eps=w.eps, gram_schmidt_on=w.gs, gs_eps=GS_EPS,
                        route=w.route, W_route=h["W_route"], b_route=h["b_route"], gate_mode=gate))


def run_forward(w, dev, fixed, in_place=False, xact=None, gate="sigmoid"):
    T, C = w.T, w.C
    X = dev["X"].clone()
    Xn = X if in_place else torch.empty_like(X)
    h_in = torch.empty(T, C, dtype=X.dtype, device=X.device)
    desc = xhc.make_desc(w.B, w.S, C, w.N, w.k, w.ncomp, xhc.XHC_BF16 if w.dtype == "bf16" else xhc.XHC_F32,
                         w.iters, w.eps, gram_schmidt=w.gs, gs_eps=GS_EPS, route=w.route,
                         gate_mode=xhc.XHC_GATE_UNIT if gate == "unit" else xhc.XHC_GATE_SIGMOID)
    z_save = torch.empty(T, xhc.zsave_stride(desc), dtype=torch.float32, device=X.device)
    ridx = torch.full((T, w.k), -1, dtype=torch.int32, device=X.device)
    conv = dict(w4=dev["w4"], w8=dev["w8"], w12=dev["w12"]) if w.ncomp == 4 else {}
    xhc.forward(X, dev["out"], dev["W"], list(fixed) + [0] * w.route, Xn, h_in, B=w.B, S=w.S,
                bias=dev["bias"], z_save=z_save, desc=desc, W_route=dev["W_route"], b_route=dev["b_route"],
                route_idx=ridx, xact_save=xact, **conv)
    torch.cuda.synchronize()
    return Xn, h_in, z_save, ridx.cpu().numpy().astype(np.int64), desc


def check_choice(rho, idx, fixed, R, atol=2e-3, rtol=1e-3):
    """Every token's list: the fixed streams, then R distinct candidates that
    form a top-R (in order) under the reference scores within a tolerance.
    Returns the number of tokens whose list differs from the exact choice."""
    T, N = rho.shape
    k = idx.shape[1]
    nfix = k - R
    assert (idx[:, :nfix] == np.asarray(fixed, dtype=np.int64)[None, :]).all(), "fixed slots"
    cand = np.array([i for i in range(N) if i not in fixed])
    routed = idx[:, nfix:]
    assert np.isin(routed, cand).all(), "a routed slot holds a fixed or invalid stream"
    assert all(len(set(r)) == R for r in routed), "repeated stream in a routed list"
    t_ = np.arange(T)[:, None]
    chosen_rho = rho[t_, routed]
    slack = atol + rtol * np.abs(rho).max(axis=1)
    # in order (non-increasing) within the slack
    assert (np.diff(chosen_rho, axis=1) <= slack[:, None]).all(), "routed slots out of score order"
    # no unchosen candidate scores above the lowest chosen one beyond the slack
    mask = np.zeros((T, N), dtype=bool)
    mask[:, cand] = True
    mask[t_, routed] = False
    best_left = np.where(mask, rho, -np.inf).max(axis=1)
    assert (best_left <= chosen_rho.min(axis=1) + slack).all(), "a better candidate was left out"
    exact = xo.route_select(rho, fixed, R)
    return int((exact != idx).any(axis=1).sum())


def compare_forward(w, h, fixed, Xn, h_in, z_save, idx, ref):
    atol, rtol = tol(w)
    T, N = w.T, w.N
    Xn_h = to_host(Xn)
    act = np.zeros((T, N), dtype=bool)
    act[np.arange(T)[:, None], idx] = True
    assert np.array_equal(Xn_h[~act], h["X"][~act]), "pass-through rows differ"
    check_close("X_new[active]", Xn_h[act], ref["X_new"][act], atol, rtol)
    check_close("h_in", to_host(h_in), ref["h_in"], atol, rtol)
    zs = z_save.cpu().numpy().astype(np.float64)
    P, k, R = w.P, w.k, w.route
    check_close("z", zs[:, :P], ref["z"], *tol_logits(w))
    check_close("mean", zs[:, P + 1], ref["mu"], 1e-5, 1e-4)
    check_close("sd", zs[:, P + 2], ref["sd"], 1e-5, 1e-4)
    rec = zs[:, P + 3:P + 3 + 3 * R].reshape(T, R, 3)
    check_close("rho[routed]", rec[:, :, 0], np.take_along_axis(ref["rho"], idx[:, k - R:], axis=1), *slack(w))


@pytest.mark.parametrize("name,w,fixed", CASES, ids=[c[0] for c in CASES])
def test_route_forward_parity(name, w, fixed):
    say(f"[route forward] {name} B={w.B} S={w.S} C={w.C} N={w.N} k={w.k} R={w.route} nc={w.ncomp} "
        f"gs={w.gs} {w.dtype}")
    d = inputs(w, 0, False)
    h = host_inputs(d)
    dev = device_inputs(d, w.dtype == "bf16")
    Xn, h_in, z_save, idx, _ = run_forward(w, dev, fixed)
    hk = host_kw(h, w, fixed)
    rt = xo.forward(*hk["args"], **hk["kw"])
    differ = check_choice(rt["rho"], idx, fixed, w.route, *slack(w))
    say(f"  tokens whose choice differs from the exact one (near ties): {differ} of {w.T}")
    assert differ <= max(1, w.T // 100)
    ref = xo.forward(*hk["args"], **hk["kw"], route_idx=idx)
    compare_forward(w, h, fixed, Xn, h_in, z_save, idx, ref)


@pytest.mark.parametrize("case", [0, 1, 11], ids=["tiny_f32", "ragged_bf16", "all_routed_n16_f32"])
def test_route_offset_state(case):
    # a state whose tokens have a mean far from zero next to their spread
    # (X + 8): the router's LayerNorm subtracts a large mean, which a
    # one-pass variance or an uncentred score sum would lose in fp32
    name, w, fixed = CASES[case]
    say(f"[route offset state] {name}")
    d = inputs(w, 5, False)
    if w.dtype == "bf16":
        d["X"] = synth.bf16_bits(synth.bf16_to_f32(d["X"]) + np.float32(8.0))
    else:
        d["X"] = d["X"] + np.float32(8.0)
    h = host_inputs(d)
    dev = device_inputs(d, w.dtype == "bf16")
    Xn, h_in, z_save, idx, _ = run_forward(w, dev, fixed)
    hk = host_kw(h, w, fixed)
    rt = xo.forward(*hk["args"], **hk["kw"])
    assert np.abs(rt["mu"]).min() > 7.0
    differ = check_choice(rt["rho"], idx, fixed, w.route, *slack(w))
    say(f"  tokens whose choice differs from the exact one (near ties): {differ} of {w.T}")
    assert differ <= max(1, w.T // 100)
    ref = xo.forward(*hk["args"], **hk["kw"], route_idx=idx)
    compare_forward(w, h, fixed, Xn, h_in, z_save, idx, ref)


def test_route_forward_in_place_matches_out_of_place():
    w = CASES[1][1]
    fixed = CASES[1][2]
    say(f"[route forward in place] B={w.B} S={w.S} C={w.C}")
    d = inputs(w, 1, False)
    dev = device_inputs(d, True)
    a = run_forward(w, dev, fixed, in_place=False)
    b = run_forward(w, dev, fixed, in_place=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and (a[3] == b[3]).all()


def test_route_ties_go_to_the_lower_stream():
    # W_route = 0: every score is exactly b_route, so the choice (ties
    # included) is decided exactly and must equal the oracle's
    w = W_("r", 2, 33, 64, 16, 4, 4, "f32", "fwd", route=2)
    fixed = [2, 11]
    say(f"[route ties] B={w.B} S={w.S} C={w.C}")
    d = inputs(w, 2, False)
    d["W_route"] = np.zeros_like(d["W_route"])
    d["b_route"] = np.array([0.5, 1.0, 9.0, 1.0, 0.25, 1.0, 0.5, 0.75, 1.0, 0.0, 0.5, 9.0, 0.75, 0.5, 1.0, 0.5],
                            dtype=np.float32)
    h = host_inputs(d)
    dev = device_inputs(d, False)
    Xn, h_in, z_save, idx, _ = run_forward(w, dev, fixed)
    assert (idx == np.array([2, 11, 1, 3])[None, :]).all(), idx[:3]
    hk = host_kw(h, w, fixed)
    ref = xo.forward(*hk["args"], **hk["kw"])
    assert (ref["idx"] == idx).all()
    compare_forward(w, h, fixed, Xn, h_in, z_save, idx, ref)


def run_backward(w, dev, fixed, X, z_save, ridx_dev, in_place_dx=False, accumulate=False, init=None, xact=None,
                 gate="sigmoid"):
    T, N, C, P = w.T, w.N, w.C, w.P
    dXn = dev["dX_new"].clone()
    dX = dXn if in_place_dx else torch.empty_like(dXn)
    f32 = dict(dtype=torch.float32, device=dXn.device)
    out = dict(dX=dX, dout=torch.empty(T, C, dtype=dXn.dtype, device=dXn.device),
               dW=torch.empty((N * C, P), **f32), db=torch.empty((P,), **f32),
               dW_route=torch.empty((N * C, N), **f32), db_route=torch.empty((N,), **f32))
    if w.ncomp == 4:
        out.update({key: torch.empty((C, K), **f32) for key, K in (("dw4", 4), ("dw8", 8), ("dw12", 12))})
    if init is not None:
        for key, v in init.items():
            out[key].copy_(v)
    conv = dict(w4=dev["w4"], w8=dev["w8"], w12=dev["w12"]) if w.ncomp == 4 else {}
    grads = {key: out[key] for key in ("dw4", "dw8", "dw12") if key in out}
    xhc.backward(X, dev["out"], dev["W"], list(fixed) + [0] * w.route, dXn, dev["dh_in"], out["dX"], out["dout"],
                 out["dW"], B=w.B, S=w.S, bias=dev["bias"], z_save=z_save, db=out["db"], iters=w.iters, eps=w.eps,
                 gram_schmidt=w.gs, gs_eps=GS_EPS, route=w.route, W_route=dev["W_route"], route_idx=ridx_dev,
                 gate_mode=xhc.XHC_GATE_UNIT if gate == "unit" else xhc.XHC_GATE_SIGMOID, b_route=dev["b_route"],
                 dW_route=out["dW_route"], db_route=out["db_route"], accumulate=accumulate, xact=xact, **conv,
                 **grads)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,w,fixed", CASES, ids=[c[0] for c in CASES])
def test_route_backward_parity(name, w, fixed):
    say(f"[route backward] {name} B={w.B} S={w.S} C={w.C} N={w.N} k={w.k} R={w.route} nc={w.ncomp} "
        f"gs={w.gs} {w.dtype}")
    d = inputs(w, 1, True)
    h = host_inputs(d)
    dev = device_inputs(d, w.dtype == "bf16")
    _, _, z_save, idx, _ = run_forward(w, dev, fixed)
    ridx_dev = torch.from_numpy(idx.astype(np.int32)).to(dev["X"].device)
    hk = host_kw(h, w, fixed)
    g = xo.backward(*hk["args"], h["dX_new"], h["dh_in"], **hk["kw"], route_idx=idx)
    res = run_backward(w, dev, fixed, dev["X"], z_save, ridx_dev)
    atol, rtol = tol(w)
    for key, ref in (("dX", g["dX"]), ("dout", g["dout"]), ("dW", g["dW"]), ("db", g["db"]),
                     ("dW_route", g["dW_route"]), ("db_route", g["db_route"])):
        check_close(key, to_host(res[key]), ref, atol, rtol)
    for m, key in enumerate(["dw4", "dw8", "dw12"][:w.ncomp - 1]):
        check_close(key, to_host(res[key]), g["dconv"][m], atol, rtol)
    # deterministic, and dX may overwrite dX_new
    res2 = run_backward(w, dev, fixed, dev["X"], z_save, ridx_dev)
    for key in res:
        assert torch.equal(res[key], res2[key]), f"{key} not deterministic"
    res3 = run_backward(w, dev, fixed, dev["X"], z_save, ridx_dev, in_place_dx=True)
    for key in res:
        assert torch.equal(res[key], res3[key]), f"{key} differs with dX == dX_new"
    # without z_save the logits and the router's record are recomputed for
    # the forward's choice: the same gradients, bit for bit
    res4 = run_backward(w, dev, fixed, dev["X"], None, ridx_dev)
    for key in res:
        assert torch.equal(res[key], res4[key]), f"{key} differs when recomputed"


def test_route_backward_accumulates():
    name, w, fixed = CASES[1]
    say(f"[route backward accumulate] {name}")
    d = inputs(w, 3, True)
    dev = device_inputs(d, True)
    _, _, z_save, idx, _ = run_forward(w, dev, fixed)
    ridx_dev = torch.from_numpy(idx.astype(np.int32)).to(dev["X"].device)
    base = run_backward(w, dev, fixed, dev["X"], z_save, ridx_dev)
    init = {key: torch.full_like(base[key], 0.25) for key in ("dW", "db", "dW_route", "db_route", "dw4")}
    acc = run_backward(w, dev, fixed, dev["X"], z_save, ridx_dev, accumulate=True, init=init)
    for key in init:
        assert torch.allclose(acc[key], base[key] + 0.25, rtol=1e-6, atol=1e-6), key


@pytest.mark.parametrize("case", [1, 2, 6], ids=[CASES[i][0] for i in (1, 2, 6)])
def test_route_backward_after_in_place_forward(case):
    # the in-place forward keeps each token's old active rows (slot order);
    # the backward from the updated state and those rows equals the one from
    # the forward's input, bit for bit
    name, w, fixed = CASES[case]
    say(f"[route backward in place] {name}")
    d = inputs(w, 4, True)
    dev = device_inputs(d, w.dtype == "bf16")
    _, _, z_save, idx, _ = run_forward(w, dev, fixed)
    ridx_dev = torch.from_numpy(idx.astype(np.int32)).to(dev["X"].device)
    ref = run_backward(w, dev, fixed, dev["X"], z_save, ridx_dev)
    xact = torch.empty(w.T, w.k, w.C, dtype=dev["X"].dtype, device=dev["X"].device)
    Xn, _, z2, idx2, _ = run_forward(w, dev, fixed, in_place=True, xact=xact)
    assert (idx2 == idx).all() and torch.equal(z2, z_save)
    got = run_backward(w, dev, fixed, Xn, z2, ridx_dev, xact=xact)
    for key in ref:
        assert torch.equal(got[key], ref[key]), key


# ---------------------------------------------------------------------------
# per-token lists given by the caller (desc.per_token_active = 1, reading O8)
# ---------------------------------------------------------------------------

GIVEN = [
    ("given_bf16", W_("g", 2, 77, 136, 16, 4, 4, "bf16", "fwdbwd")),
    ("given_k3_n7_f32", W_("g", 3, 30, 40, 7, 3, 4, "f32", "fwdbwd")),
    ("given_gs_bf16", W_("g", 2, 61, 96, 16, 4, 4, "bf16", "fwdbwd", gs=True)),
    ("given_nc1_bf16", W_("g", 2, 50, 64, 16, 4, 1, "bf16", "fwdbwd")),
]


def given_lists(w, seed):
    r = np.random.default_rng(seed)
    return np.stack([r.permutation(w.N)[:w.k] for _ in range(w.T)]).astype(np.int64)


@pytest.mark.parametrize("name,w", GIVEN, ids=[c[0] for c in GIVEN])
def test_given_lists_parity(name, w):
    say(f"[given lists] {name} B={w.B} S={w.S} C={w.C} N={w.N} k={w.k} nc={w.ncomp} gs={w.gs} {w.dtype}")
    d = synth.make_inputs(w, seed=5, grads=True)
    h = host_inputs(d)
    dev = device_inputs(d, w.dtype == "bf16")
    lists = given_lists(w, 6)
    lists_dev = torch.from_numpy(lists.astype(np.int32)).to(dev["X"].device)
    T, N, C, P, k = w.T, w.N, w.C, w.P, w.k
    desc = xhc.make_desc(w.B, w.S, C, N, k, w.ncomp, xhc.XHC_BF16 if w.dtype == "bf16" else xhc.XHC_F32,
                         w.iters, w.eps, gram_schmidt=w.gs, gs_eps=GS_EPS, per_token_active=True)
    conv = dict(w4=dev["w4"], w8=dev["w8"], w12=dev["w12"]) if w.ncomp == 4 else {}
    convs = (h["w4"], h["w8"], h["w12"]) if w.ncomp == 4 else ()
    kw = dict(B=w.B, S=w.S, iters=w.iters, eps=w.eps, gram_schmidt_on=w.gs, gs_eps=GS_EPS, active_tok=lists)
    ref = xo.forward(h["X"], h["out"], h["W"], h["bias"], [0] * k, convs, **kw)
    g = xo.backward(h["X"], h["out"], h["W"], h["bias"], [0] * k, convs, h["dX_new"], h["dh_in"], **kw)
    atol, rtol = tol(w)
    X = dev["X"].clone()
    h_in = torch.empty(T, C, dtype=X.dtype, device=X.device)
    z_save = torch.empty(T, P + 1, device=X.device)
    xact = torch.empty(T, k, C, dtype=X.dtype, device=X.device)
    xhc.forward(X, dev["out"], dev["W"], [0] * k, X, h_in, B=w.B, S=w.S, bias=dev["bias"], z_save=z_save,
                xact_save=xact, desc=desc, route_idx=lists_dev, **conv)
    torch.cuda.synchronize()
    Xn_h = to_host(X)
    act = np.zeros((T, N), dtype=bool)
    act[np.arange(T)[:, None], lists] = True
    assert np.array_equal(Xn_h[~act], h["X"][~act]), "pass-through rows differ"
    check_close("X_new[active]", Xn_h[act], ref["X_new"][act], atol, rtol)
    check_close("h_in", to_host(h_in), ref["h_in"], atol, rtol)
    assert np.array_equal(to_host(xact), h["X"][np.arange(T)[:, None], lists]), "saved rows"

    def run(Xs, xs, zs):
        f32 = dict(dtype=torch.float32, device=X.device)
        o = dict(dX=torch.empty_like(dev["dX_new"]), dout=torch.empty(T, C, dtype=X.dtype, device=X.device),
                 dW=torch.empty((N * C, P), **f32), db=torch.empty((P,), **f32))
        grads = {}
        if w.ncomp == 4:
            grads = {key: torch.empty((C, K), **f32) for key, K in (("dw4", 4), ("dw8", 8), ("dw12", 12))}
        xhc.backward(Xs, dev["out"], dev["W"], [0] * k, dev["dX_new"], dev["dh_in"], o["dX"], o["dout"], o["dW"],
                     B=w.B, S=w.S, xact=xs, bias=dev["bias"], z_save=zs, db=o["db"], desc=desc,
                     route_idx=lists_dev, **conv, **grads)
        torch.cuda.synchronize()
        o.update(grads)
        return o

    res = run(X, xact, z_save)
    for key, rf in (("dX", g["dX"]), ("dout", g["dout"]), ("dW", g["dW"]), ("db", g["db"])):
        check_close(key, to_host(res[key]), rf, atol, rtol)
    for m, key in enumerate(["dw4", "dw8", "dw12"][:w.ncomp - 1]):
        check_close(key, to_host(res[key]), g["dconv"][m], atol, rtol)
    # from the forward's input, with the logits recomputed: the same gradients
    res2 = run(dev["X"], None, None)
    for key in res:
        assert np.allclose(to_host(res[key]), to_host(res2[key]), rtol=1e-5, atol=1e-6), key


def test_route_with_unit_gates():
    # unit gates (H_pre = H_post = 1): the routed write-back is s times the
    # plain sum of the components, and the router still gets its gradient
    name, w, fixed = CASES[0]
    say(f"[route unit gates] {name}")
    d = inputs(w, 11, True)
    h = host_inputs(d)
    dev = device_inputs(d, False)
    Xn, h_in, z_save, idx, _ = run_forward(w, dev, fixed, gate="unit")
    hk = host_kw(h, w, fixed, gate="unit")
    own = xo.forward(*hk["args"], **hk["kw"])
    assert check_choice(own["rho"], idx, fixed, w.route, *slack(w)) <= 1
    ref = xo.forward(*hk["args"], **hk["kw"], route_idx=idx)
    compare_forward(w, h, fixed, Xn, h_in, z_save, idx, ref)
    ridx_dev = torch.from_numpy(idx.astype(np.int32)).to(dev["X"].device)
    g = xo.backward(*hk["args"], h["dX_new"], h["dh_in"], **hk["kw"], route_idx=idx)
    res = run_backward(w, dev, fixed, dev["X"], z_save, ridx_dev, gate="unit")
    for key, rf in (("dX", g["dX"]), ("dout", g["dout"]), ("dW", g["dW"]), ("db", g["db"]),
                    ("dW_route", g["dW_route"]), ("db_route", g["db_route"])):
        check_close(key, to_host(res[key]), rf, 1e-4, 1e-4)
    assert np.abs(g["db_route"]).max() > 1e-3

"""GPU parity of the chained forward with per-token lists (the router,
desc.route > 0, and given lists) through the C ABI.

Every sublayer of the stack routes (two fixed and two routed streams, the
retrospective's setting), or the stack mixes routed and fixed-list
sublayers.  Each call's fused write pass forms the next sublayer's
projection -- with a routed next sublayer also its router's logits and
sum(x') -- from the new state, so every call after the first starts from
the carry.  Checked layer by layer, teacher-forced: the oracle runs sublayer
l from the GPU's state before it, the GPU's choice must be a valid top-R
under the oracle's scores (near ties may differ: the carried sums are taken
in another order), and then every output is compared with the oracle run on
the GPU's lists: active rows and h_in within fp32 1e-4 + 1e-4 |ref| (bf16
1e-2 + 1e-2 |ref|), pass-through rows bitwise, logits as in the router
tests."""
import numpy as np
import pytest
import torch

from oracle import xhc_oracle as xo
from residual_stream_architecture_amd import synth
from residual_stream_architecture_amd import xhc
from tests.gpu_util import check_close, device_inputs, host_inputs, say, to_host
from tests.test_gpu_route import GS_EPS, check_choice, slack, tol, tol_logits

pytestmark = pytest.mark.gpu
W_ = synth.Workload

# name, workload shape, per layer: (route R or "given", fixed streams)
CASES = [
    ("routed3_f32", W_("c", 1, 64, 64, 16, 4, 4, "f32", "fwd", route=2),
     [(2, [0, 1]), (2, [5, 9]), (2, [2, 14])]),
    ("routed3_bf16", W_("c", 2, 45, 136, 16, 4, 4, "bf16", "fwd", route=2),
     [(2, [3, 7]), (2, [11, 0]), (2, [6, 12])]),
    ("mixed_bf16", W_("c", 2, 40, 128, 16, 4, 4, "bf16", "fwd", route=2),
     [(0, [1, 2, 3, 4]), (2, [8, 9]), (0, [12, 13, 14, 15]), (2, [0, 5])]),
    ("all_routed_f32", W_("c", 2, 33, 64, 16, 4, 4, "f32", "fwd", route=4),
     [(4, []), (4, []), (2, [4, 10])]),
    ("given_bf16", W_("c", 2, 41, 96, 16, 4, 4, "bf16", "fwd"),
     [("given", []), ("given", []), (2, [7, 1])]),
    # the stack's channel count (112 chunks of 64 channels in 16 blocks)
    ("stack_c7168_bf16", W_("c", 1, 160, 7168, 16, 4, 4, "bf16", "fwd", route=2),
     [(2, [0, 1]), (2, [4, 5]), (2, [8, 9]), (2, [12, 13])]),
    # Gram-Schmidt over the components in every sublayer
    ("gram_schmidt_bf16", W_("c", 2, 45, 136, 16, 4, 4, "bf16", "fwd", route=2, gs=True),
     [(2, [3, 7]), ("given", []), (2, [6, 12])]),
]


def layer_desc(w, kind):
    dt = xhc.XHC_BF16 if w.dtype == "bf16" else xhc.XHC_F32
    if kind == "given":
        return xhc.make_desc(w.B, w.S, w.C, w.N, w.k, w.ncomp, dt, w.iters, w.eps, per_token_active=True,
                             gram_schmidt=w.gs, gs_eps=GS_EPS)
    return xhc.make_desc(w.B, w.S, w.C, w.N, w.k, w.ncomp, dt, w.iters, w.eps, route=kind, gram_schmidt=w.gs,
                         gs_eps=GS_EPS)


def layer_inputs(w, l):
    d = synth.make_inputs(w, seed=100 + l, state=False)
    d.update(synth.make_router(w, 100 + l))
    return d


@pytest.mark.parametrize("name,w,layers", CASES, ids=[c[0] for c in CASES])
def test_chained_routed_stack(name, w, layers):
    say(f"[chain route] {name} B={w.B} S={w.S} C={w.C} layers={[k for k, _ in layers]} {w.dtype}")
    bf = w.dtype == "bf16"
    T, N, C, k = w.T, w.N, w.C, w.k
    d0 = synth.make_inputs(w, seed=99)
    X = device_inputs({"X": d0["X"]}, bf)["X"].clone()
    L = len(layers)
    host = [host_inputs(layer_inputs(w, l)) for l in range(L)]
    dev = [device_inputs(layer_inputs(w, l), bf) for l in range(L)]
    descs = [layer_desc(w, kind) for kind, _ in layers]
    rng = np.random.default_rng(5)
    given = [np.stack([rng.permutation(N)[:k] for _ in range(T)]).astype(np.int32) if kind == "given" else None
             for kind, _ in layers]
    carry = None
    for l, (kind, fixed) in enumerate(layers):
        desc = descs[l]
        x_before = to_host(X)
        h_in = torch.empty(T, C, dtype=X.dtype, device=X.device)
        z_save = torch.empty(T, xhc.zsave_stride(desc), dtype=torch.float32, device=X.device)
        if kind == "given":
            ridx = torch.from_numpy(given[l]).to(X.device)
        else:
            ridx = torch.full((T, k), -1, dtype=torch.int32, device=X.device)
        active = list(fixed) + [0] * (k - len(fixed))
        kw = {}
        if l + 1 < L:
            kn, fn = layers[l + 1]
            carry_out = torch.empty(xhc.carry_size(descs[l + 1]) // 4, dtype=torch.float32, device=X.device)
            kw = dict(W_next=dev[l + 1]["W"], carry_out=carry_out, desc_next=descs[l + 1])
            if kn not in (0, "given"):
                kw.update(W_route_next=dev[l + 1]["W_route"], active_next=list(fn) + [0] * (k - len(fn)))
        if carry is not None:
            kw["carry_in"] = carry
        rkw = {}
        if kind == "given" or kind:
            rkw = dict(route_idx=ridx)
            if kind != "given":
                rkw.update(W_route=dev[l]["W_route"], b_route=dev[l]["b_route"])
        if kind == 0:
            rkw = {}
        conv = dict(w4=dev[l]["w4"], w8=dev[l]["w8"], w12=dev[l]["w12"])
        xhc.forward(X, dev[l]["out"], dev[l]["W"] if carry is None else None, active, X, h_in, B=w.B, S=w.S,
                    bias=dev[l]["bias"], z_save=z_save, desc=desc, **conv, **rkw, **kw)
        torch.cuda.synchronize()
        carry = kw.get("carry_out")
        # the oracle from the GPU's state before the sublayer
        h = host[l]
        convs = (h["w4"], h["w8"], h["w12"])
        base = dict(B=w.B, S=w.S, iters=w.iters, eps=w.eps, gram_schmidt_on=w.gs, gs_eps=GS_EPS)
        if kind == "given":
            idx = given[l].astype(np.int64)
            ref = xo.forward(x_before, h["out"], h["W"], h["bias"], [0] * k, convs, active_tok=idx, **base)
        elif kind == 0:
            idx = np.tile(np.array(fixed, dtype=np.int64), (T, 1))
            ref = xo.forward(x_before, h["out"], h["W"], h["bias"], fixed, convs, **base)
        else:
            rkw_o = dict(route=kind, W_route=h["W_route"], b_route=h["b_route"], **base)
            own = xo.forward(x_before, h["out"], h["W"], h["bias"], active, convs, **rkw_o)
            idx = ridx.cpu().numpy().astype(np.int64)
            differ = check_choice(own["rho"], idx, fixed, kind, *slack(w))
            say(f"  layer {l}: tokens whose choice differs from the exact one (near ties): {differ} of {T}")
            assert differ <= max(1, T // 100)
            ref = xo.forward(x_before, h["out"], h["W"], h["bias"], active, convs, route_idx=idx, **rkw_o)
        atol, rtol = tol(w)
        Xh = to_host(X)
        act = np.zeros((T, N), dtype=bool)
        act[np.arange(T)[:, None], idx] = True
        assert np.array_equal(Xh[~act], x_before[~act]), f"layer {l}: pass-through rows differ"
        check_close(f"layer {l} X_new[active]", Xh[act], ref["X_new"][act], atol, rtol)
        check_close(f"layer {l} h_in", to_host(h_in), ref["h_in"], atol, rtol)
        check_close(f"layer {l} z", z_save.cpu().numpy().astype(np.float64)[:, :w.P], ref["z"], *tol_logits(w))

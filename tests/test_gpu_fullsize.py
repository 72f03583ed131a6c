"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.  The forward of the single-sublayer workloads (fwd2048 at
every layer of its rotation, mhc4, fwdbwd4096) is checked on every token
against the oracle run sequence by sequence, and pass-through rows bitwise
over the whole state; the backward of the fwd+bwd workload is checked in
full the same way.  The Gram-Schmidt form and the 48-layer stack are checked
on sampled token blocks that the oracle computes on their own (a block
carries an 11-token lead-in, so its outputs are exact: tokens interact only
through the 11-token TFA window), the stack layer by layer, teacher-forced
from the GPU's own state."""
import time

import numpy as np
import pytest
import torch

from oracle import xhc_oracle as xo
from residual_stream_architecture_amd import synth
from residual_stream_architecture_amd import xhc
from tests.gpu_util import check_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu
LEAD = 11


def dev_params(d):
    p = {}
    for key in ("out", "W"):
        p[key] = to_dev(d[key], True)
    for key in ("w4", "w8", "w12", "bias"):
        if key in d:
            p[key] = torch.from_numpy(d[key]).cuda()
    return p


def conv_kw(p, nc):
    return dict(w4=p["w4"], w8=p["w8"], w12=p["w12"]) if nc == 4 else {}


def sample_blocks(w, n=24):
    """(sequence, start) of sampled blocks: sequence starts, ends, segment
    boundaries and a middle block."""
    out = []
    last = w.S - n
    for b in sorted({0, w.B - 1}):
        for s in sorted({0, 36, min(w.S // 2, last), last}):
            out.append((b, max(0, min(s, last))))
    return out


def check_forward_full(w, Xh, outh, hW, bias, convs, active, Xn_dev, hin_dev):
    """Every token's rewritten rows and h_in against the oracle, one sequence
    at a time."""
    for b in range(w.B):
        rows = slice(b * w.S, (b + 1) * w.S)
        ref = xo.forward(Xh[rows], outh[rows], hW, bias, active, convs, B=1, S=w.S, iters=w.iters, eps=w.eps)
        check_close(f"X_new[seq {b}]", to_host(Xn_dev[rows][:, active]), ref["X_new"][:, active], 1e-2, 1e-2)
        check_close(f"h_in[seq {b}]", to_host(hin_dev[rows]), ref["h_in"], 1e-2, 1e-2)
        del ref


@pytest.mark.timeout(900)
def test_fwd2048_rotating_layers():
    w = synth.WORKLOADS["fwd2048"]
    say(f"[fullsize] fwd2048 B={w.B} S={w.S} C={w.C}")
    d = synth.make_inputs(w, seed=0)
    Xh = synth.bf16_to_f32(d["X"])
    outh, hW = synth.as_float(d, "out"), synth.as_float(d, "W")
    convs = (d["w4"], d["w8"], d["w12"])
    p = dev_params(d)
    X0 = to_dev(d["X"], True)
    for layer in range(4):
        active = synth.active_streams(layer, w.N, w.k)
        X = X0.clone()
        h_in = torch.empty(w.T, w.C, dtype=torch.bfloat16, device="cuda")
        xhc.forward(X, p["out"], p["W"], active, X, h_in, B=w.B, S=w.S, bias=p["bias"], **conv_kw(p, 4))
        torch.cuda.synchronize()
        inactive = [i for i in range(w.N) if i not in active]
        assert torch.equal(X[:, inactive], X0[:, inactive]), f"layer {layer}: pass-through rows differ"
        say(f" layer {layer} active={active}")
        check_forward_full(w, Xh, outh, hW, d["bias"], convs, active, X, h_in)


@pytest.mark.timeout(600)
def test_mhc4_dense_update():
    w = synth.WORKLOADS["mhc4"]
    say(f"[fullsize] mhc4 B={w.B} S={w.S} C={w.C} N={w.N}")
    d = synth.make_inputs(w, seed=0)
    Xh = synth.bf16_to_f32(d["X"])
    outh, hW = synth.as_float(d, "out"), synth.as_float(d, "W")
    p = dev_params(d)
    X = to_dev(d["X"], True)
    h_in = torch.empty(w.T, w.C, dtype=torch.bfloat16, device="cuda")
    xhc.forward(X, p["out"], p["W"], [0, 1, 2, 3], X, h_in, B=w.B, S=w.S, bias=p["bias"])
    torch.cuda.synchronize()
    check_forward_full(w, Xh, outh, hW, d["bias"], (), [0, 1, 2, 3], X, h_in)


@pytest.mark.timeout(1200)
def test_fwdbwd4096_full_backward():
    w = synth.WORKLOADS["fwdbwd4096"]
    say(f"[fullsize] fwdbwd4096 B={w.B} S={w.S} C={w.C}")
    t_start = time.time()
    d = synth.make_inputs(w, seed=0, grads=True)
    p = dev_params(d)
    X = to_dev(d["X"], True)
    dXn = to_dev(d["dX_new"], True)
    dhin = to_dev(d["dh_in"], True)
    active = [0, 1, 2, 3]
    T, N, C, P = w.T, w.N, w.C, w.P
    h_in = torch.empty(T, C, dtype=torch.bfloat16, device="cuda")
    z_save = torch.empty(T, P + 1, device="cuda")
    xact = torch.empty(T, 4, C, dtype=torch.bfloat16, device="cuda")
    X_before = X.clone()
    xhc.forward(X, p["out"], p["W"], active, X, h_in, B=w.B, S=w.S, bias=p["bias"], z_save=z_save,
                xact_save=xact, **conv_kw(p, 4))
    dX = torch.empty_like(dXn)
    dout = torch.empty(T, C, dtype=torch.bfloat16, device="cuda")
    dW = torch.empty(N * C, P, device="cuda")
    db = torch.empty(P, device="cuda")
    dws = dict(dw4=torch.empty(C, 4, device="cuda"), dw8=torch.empty(C, 8, device="cuda"),
               dw12=torch.empty(C, 12, device="cuda"))
    xhc.backward(X, p["out"], p["W"], active, dXn, dhin, dX, dout, dW, B=w.B, S=w.S, xact=xact, bias=p["bias"],
                 z_save=z_save, db=db, **conv_kw(p, 4), **dws)
    torch.cuda.synchronize()
    assert torch.equal(xact, X_before[:, :4])
    del X_before
    say(f" gpu done in {time.time() - t_start:.1f}s")

    Xh = synth.bf16_to_f32(d["X"])
    outh, hW = synth.as_float(d, "out"), synth.as_float(d, "W")
    convs = (d["w4"], d["w8"], d["w12"])
    check_forward_full(w, Xh, outh, hW, d["bias"], convs, active, X, h_in)
    dW_ref = np.zeros((N * C, P))
    db_ref = np.zeros(P)
    dconv_ref = [np.zeros((C, K)) for K in (4, 8, 12)]
    for b in range(w.B):
        rows = slice(b * w.S, (b + 1) * w.S)
        g = xo.backward(Xh[rows], outh[rows], hW, d["bias"], active, convs,
                        synth.bf16_to_f32(d["dX_new"][rows]), synth.bf16_to_f32(d["dh_in"][rows]),
                        B=1, S=w.S, iters=w.iters, eps=w.eps)
        check_close(f"dX[seq {b}]", to_host(dX[rows]), g["dX"], 1e-2, 1e-2)
        check_close(f"dout[seq {b}]", to_host(dout[rows]), g["dout"], 1e-2, 1e-2)
        dW_ref += g["dW"]
        db_ref += g["db"]
        for m in range(3):
            dconv_ref[m] += g["dconv"][m]
        del g
        say(f" oracle sequence {b} done at {time.time() - t_start:.1f}s")
    check_close("dW", to_host(dW), dW_ref, 1e-2, 1e-2)
    check_close("db", to_host(db), db_ref, 1e-2, 1e-2)
    for m, key in enumerate(("dw4", "dw8", "dw12")):
        check_close(key, to_host(dws[key]), dconv_ref[m], 1e-2, 1e-2)


@pytest.mark.timeout(600)
def test_fwdbwd4096_gs_sampled():
    # the Gram-Schmidt form at the full fwd+bwd size, in the launch
    # configuration the benchmark times.  Tokens interact only through the
    # 11-token TFA window: a block with 11 tokens of lead-in gives exact
    # forward outputs and dX; one with 11 more tokens after it gives exact
    # dout (the gradients of later positions flow back through the window).
    w = synth.WORKLOADS["fwdbwd4096_gs"]
    say(f"[fullsize] fwdbwd4096_gs B={w.B} S={w.S} C={w.C}")
    d = synth.make_inputs(w, seed=7, grads=True)
    r = np.random.default_rng(8)
    for key, K in (("w4", 4), ("w8", 8), ("w12", 12)):       # components leaning on the output
        v = (r.standard_normal((w.C, K)) * 0.3).astype(np.float32)
        v[:, K - 1] += 0.6
        d[key] = v
    p = dev_params(d)
    X = to_dev(d["X"], True)
    dXn = to_dev(d["dX_new"], True)
    dhin = to_dev(d["dh_in"], True)
    active = [0, 1, 2, 3]
    T, N, C, P = w.T, w.N, w.C, w.P
    h_in = torch.empty(T, C, dtype=torch.bfloat16, device="cuda")
    z_save = torch.empty(T, P + 1, device="cuda")
    xact = torch.empty(T, 4, C, dtype=torch.bfloat16, device="cuda")
    xhc.forward(X, p["out"], p["W"], active, X, h_in, B=w.B, S=w.S, bias=p["bias"], z_save=z_save,
                xact_save=xact, gram_schmidt=True, **conv_kw(p, 4))
    dX = torch.empty_like(dXn)
    dout = torch.empty(T, C, dtype=torch.bfloat16, device="cuda")
    dW = torch.empty(N * C, P, device="cuda")
    dws = dict(dw4=torch.empty(C, 4, device="cuda"), dw8=torch.empty(C, 8, device="cuda"),
               dw12=torch.empty(C, 12, device="cuda"))
    xhc.backward(X, p["out"], p["W"], active, dXn, dhin, dX, dout, dW, B=w.B, S=w.S, xact=xact, bias=p["bias"],
                 z_save=z_save, gram_schmidt=True, **conv_kw(p, 4), **dws)
    torch.cuda.synchronize()
    Xh = synth.bf16_to_f32(d["X"])
    outh, hW = synth.as_float(d, "out"), synth.as_float(d, "W")
    dXnh, dhinh = synth.bf16_to_f32(d["dX_new"]), synth.bf16_to_f32(d["dh_in"])
    convs = (d["w4"], d["w8"], d["w12"])
    n = 24
    for (b, s) in sample_blocks(w, n):
        lo, hi = max(0, s - LEAD), min(w.S, s + n + LEAD)
        rows = slice(b * w.S + lo, b * w.S + hi)
        kw = dict(B=1, S=hi - lo, iters=w.iters, eps=w.eps, gram_schmidt_on=True)
        ref = xo.forward(Xh[rows], outh[rows], hW, d["bias"], active, convs, **kw)
        g = xo.backward(Xh[rows], outh[rows], hW, d["bias"], active, convs, dXnh[rows], dhinh[rows], **kw)
        k0, t0 = s - lo, b * w.S + s
        check_close(f"X_new[b={b},s={s}]", to_host(X[t0:t0 + n])[:, active], ref["X_new"][k0:k0 + n, active],
                    1e-2, 1e-2)
        check_close(f"h_in[b={b},s={s}]", to_host(h_in[t0:t0 + n]), ref["h_in"][k0:k0 + n], 1e-2, 1e-2)
        check_close(f"dX[b={b},s={s}]", to_host(dX[t0:t0 + n]), g["dX"][k0:k0 + n], 1e-2, 1e-2)
        check_close(f"dout[b={b},s={s}]", to_host(dout[t0:t0 + n]), g["dout"][k0:k0 + n], 1e-2, 1e-2)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("chained", [True, False], ids=["chained", "two_pass"])
def test_stack48_teacher_forced(chained):
    """All 48 sublayers of the stack, in the launch configuration the
    benchmark times (chained: every sublayer after the first starts from the
    projection partials the previous write pass carried out, and every
    sublayer but the last carries them on).  Each layer is checked on
    sampled blocks, teacher-forced from the GPU's own state before it: the
    active rows and h_in within tolerance, the other rows bitwise, and the
    saved logits and RMS (for a chained layer these come from the carry).
    The first, a middle and the last layer are checked on every token the
    same way."""
    w = synth.WORKLOADS["stack48"]
    say(f"[fullsize] stack48 S={w.S} C={w.C} layers={w.layers} chained={chained}")
    t_start = time.time()
    T, N, C, P = w.T, w.N, w.C, w.P
    X = to_dev(synth.make_inputs(w, seed=0)["X"], True)
    blocks = [(0, 0), (0, 4096), (0, w.S - 16)]
    n = 16
    h_in = torch.empty(T, C, dtype=torch.bfloat16, device="cuda")
    z_save = torch.empty(T, P + 1, device="cuda")
    desc = xhc.make_desc(w.B, w.S, C, N, w.k, 4, xhc.XHC_BF16)
    carries = [torch.empty(xhc.carry_size(desc) // 4, device="cuda") for _ in range(2)] if chained else None

    def params(layer):
        d = synth.make_inputs(w, seed=synth.stack_layer_seed(layer), state=False)
        return d, dev_params(d)

    cur = params(0)
    for layer in range(w.layers):
        d, p = cur
        nxt = params(layer + 1) if layer + 1 < w.layers else None
        active = synth.active_streams(layer, w.N, w.k)
        before = {}
        for (_, s) in blocks:
            lo = max(0, s - LEAD)
            before[s] = to_host(X[lo:s + n])
        full = layer in (0, w.layers // 2, w.layers - 1)
        X_full = X.clone() if full else None
        extra = {}
        if chained:
            extra = dict(carry_in=carries[layer % 2] if layer > 0 else None,
                         W_next=None if nxt is None else nxt[1]["W"],
                         carry_out=None if nxt is None else carries[(layer + 1) % 2])
        xhc.forward(X, p["out"], None if (chained and layer > 0) else p["W"], active, X, h_in, B=w.B, S=w.S,
                    bias=p["bias"], z_save=z_save, desc=desc, **conv_kw(p, 4), **extra)
        torch.cuda.synchronize()
        outh, hW = synth.as_float(d, "out"), synth.as_float(d, "W")
        convs = (d["w4"], d["w8"], d["w12"])
        for (_, s) in blocks:
            lo = max(0, s - LEAD)
            ref = xo.forward(before[s], outh[lo:s + n], hW, d["bias"], active, convs, B=1, S=s + n - lo,
                             iters=w.iters, eps=w.eps)
            k0 = s - lo
            got = to_host(X[s:s + n])
            inactive = [i for i in range(w.N) if i not in active]
            assert np.array_equal(got[:, inactive], before[s][k0:, inactive]), f"layer {layer}: pass-through"
            check_close(f"L{layer} X_new[s={s}]", got[:, active], ref["X_new"][k0:, active], 1e-2, 1e-2)
            check_close(f"L{layer} h_in[s={s}]", to_host(h_in[s:s + n]), ref["h_in"][k0:], 1e-2, 1e-2)
            zs = to_host(z_save[s:s + n])
            check_close(f"L{layer} z[s={s}]", zs[:, :P], ref["z"][k0:], 1e-3, 1e-3)
            check_close(f"L{layer} r[s={s}]", zs[:, P], ref["r"][k0:], 1e-5, 1e-4)
        if full:
            inactive = [i for i in range(w.N) if i not in active]
            assert torch.equal(X[:, inactive], X_full[:, inactive]), f"layer {layer}: pass-through"
            ref = xo.forward(to_host(X_full), outh, hW, d["bias"], active, convs, B=1, S=w.S, iters=w.iters,
                             eps=w.eps)
            del X_full
            check_close(f"L{layer} X_new[all]", to_host(X[:, active]), ref["X_new"][:, active], 1e-2, 1e-2)
            check_close(f"L{layer} h_in[all]", to_host(h_in), ref["h_in"], 1e-2, 1e-2)
            zs = to_host(z_save)
            check_close(f"L{layer} z[all]", zs[:, :P], ref["z"], 1e-3, 1e-3)
            check_close(f"L{layer} r[all]", zs[:, P], ref["r"], 1e-5, 1e-4)
            del ref, zs
        say(f" layer {layer} ok at {time.time() - t_start:.1f}s")
        cur = nxt


@pytest.mark.timeout(600)
def test_fwdbwd4096_route_sampled():
    # the router at the full fwd+bwd size, in the launch configuration the
    # benchmark times (in-place forward with the saved rows, then the
    # backward).  Sampled blocks as in the Gram-Schmidt test; each block's
    # choice is checked against the oracle's scores, then its outputs against
    # the oracle run on the GPU's choice.
    from tests.test_gpu_route import check_choice
    w = synth.WORKLOADS["fwdbwd4096_route"]
    say(f"[fullsize] fwdbwd4096_route B={w.B} S={w.S} C={w.C} R={w.route}")
    d = synth.make_inputs(w, seed=0, grads=True)
    d.update(synth.make_router(w, 0))
    p = dev_params(d)
    Wr = to_dev(d["W_route"], True)
    br = torch.from_numpy(d["b_route"]).cuda()
    X = to_dev(d["X"], True)
    dXn = to_dev(d["dX_new"], True)
    dhin = to_dev(d["dh_in"], True)
    fixed = synth.active_streams(0, w.N, w.k)[:w.k - w.route]
    active = fixed + [0] * w.route
    T, N, C, P, k = w.T, w.N, w.C, w.P, w.k
    desc = xhc.make_desc(w.B, w.S, C, N, k, 4, xhc.XHC_BF16, w.iters, w.eps, route=w.route)
    h_in = torch.empty(T, C, dtype=torch.bfloat16, device="cuda")
    z_save = torch.empty(T, xhc.zsave_stride(desc), device="cuda")
    xact = torch.empty(T, k, C, dtype=torch.bfloat16, device="cuda")
    ridx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    xhc.forward(X, p["out"], p["W"], active, X, h_in, B=w.B, S=w.S, bias=p["bias"], z_save=z_save, xact_save=xact,
                desc=desc, W_route=Wr, b_route=br, route_idx=ridx, **conv_kw(p, 4))
    dX = torch.empty_like(dXn)
    dout = torch.empty(T, C, dtype=torch.bfloat16, device="cuda")
    dW = torch.empty(N * C, P, device="cuda")
    dWr = torch.empty(N * C, N, device="cuda")
    dws = dict(dw4=torch.empty(C, 4, device="cuda"), dw8=torch.empty(C, 8, device="cuda"),
               dw12=torch.empty(C, 12, device="cuda"))
    xhc.backward(X, p["out"], p["W"], active, dXn, dhin, dX, dout, dW, B=w.B, S=w.S, xact=xact, bias=p["bias"],
                 z_save=z_save, desc=desc, W_route=Wr, route_idx=ridx, dW_route=dWr, **conv_kw(p, 4), **dws)
    torch.cuda.synchronize()
    idx = ridx.cpu().numpy().astype(np.int64)
    Xh = synth.bf16_to_f32(d["X"])
    outh, hW, hWr = synth.as_float(d, "out"), synth.as_float(d, "W"), synth.as_float(d, "W_route")
    dXnh, dhinh = synth.bf16_to_f32(d["dX_new"]), synth.bf16_to_f32(d["dh_in"])
    convs = (d["w4"], d["w8"], d["w12"])
    Xn_h = None
    n = 24
    for (b, s) in sample_blocks(w, n):
        lo, hi = max(0, s - LEAD), min(w.S, s + n + LEAD)
        rows = slice(b * w.S + lo, b * w.S + hi)
        kw = dict(B=1, S=hi - lo, iters=w.iters, eps=w.eps, route=w.route, W_route=hWr, b_route=d["b_route"])
        own = xo.forward(Xh[rows], outh[rows], hW, d["bias"], active, convs, **kw)
        differ = check_choice(own["rho"], idx[rows], fixed, w.route)
        assert differ <= 1, f"block (b={b}, s={s}): {differ} tokens chose otherwise"
        ref = xo.forward(Xh[rows], outh[rows], hW, d["bias"], active, convs, route_idx=idx[rows], **kw)
        g = xo.backward(Xh[rows], outh[rows], hW, d["bias"], active, convs, dXnh[rows], dhinh[rows],
                        route_idx=idx[rows], **kw)
        k0, t0 = s - lo, b * w.S + s
        got = to_host(X[t0:t0 + n])
        act = np.zeros((n, N), dtype=bool)
        act[np.arange(n)[:, None], idx[t0:t0 + n]] = True
        assert np.array_equal(got[~act], Xh[t0:t0 + n][~act]), f"pass-through rows (b={b}, s={s})"
        check_close(f"X_new[b={b},s={s}]", got[act], ref["X_new"][k0:k0 + n][act], 1e-2, 1e-2)
        check_close(f"h_in[b={b},s={s}]", to_host(h_in[t0:t0 + n]), ref["h_in"][k0:k0 + n], 1e-2, 1e-2)
        check_close(f"dX[b={b},s={s}]", to_host(dX[t0:t0 + n]), g["dX"][k0:k0 + n], 1e-2, 1e-2)
        check_close(f"dout[b={b},s={s}]", to_host(dout[t0:t0 + n]), g["dout"][k0:k0 + n], 1e-2, 1e-2)
    # the saved rows are the old active rows of each token's own list
    xs = to_host(xact[:64])
    assert np.array_equal(xs, Xh[np.arange(64)[:, None], idx[:64]])
    # every fixed slot holds its stream, every routed list is valid
    assert (idx[:, :w.k - w.route] == np.array(fixed)).all()
    assert ((idx >= 0) & (idx < N)).all() and all(len(set(r)) == k for r in idx[::97])

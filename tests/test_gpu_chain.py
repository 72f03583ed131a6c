"""GPU parity of the chained forward (xhc_forward_chain).  Each sublayer's
write pass also forms the next sublayer's projection partials from the state
it writes, and the next call starts from those partials (carry_in) instead of
projecting its state again.  Checked layer by layer, teacher-forced from the
GPU's own state, against the oracle forward of that state: X_new (active rows
within tolerance, the other rows bitwise), h_in, xact_save (bitwise) and the
saved logits and RMS, which for every layer after the first come from the
carried partials."""
import time

import numpy as np
import pytest
import torch

from oracle import xhc_oracle as xo
from residual_stream_architecture_amd import synth
from residual_stream_architecture_amd import xhc
from tests.gpu_util import check_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu
W_ = synth.Workload


def tol(w):
    return (1e-4, 1e-4) if w.dtype == "f32" else (1e-2, 1e-2)


# name, workload (phase "stack", layers), in place, save the old active rows,
# one carry buffer for in and out, bias scale
CHAIN_CASES = [
    ("f32_tiny", W_("c32", 1, 64, 64, 16, 4, 4, "f32", "stack", layers=3), True, True, False, 0.0),
    ("bf16_ragged_c", W_("cb", 2, 45, 200, 16, 4, 4, "bf16", "stack", layers=3), True, False, True, 0.3),
    ("bf16_out_of_place", W_("co", 1, 150, 128, 16, 4, 4, "bf16", "stack", layers=2), False, True, False, 0.0),
    ("bf16_n11_k3", W_("cn", 2, 70, 96, 11, 3, 4, "bf16", "stack", layers=3), True, True, False, 0.2),
    ("bf16_mhc_n4", W_("cm", 2, 40, 136, 4, 4, 1, "bf16", "stack", layers=3), True, False, True, 0.0),
    ("f32_n6_k2_nc1", W_("cf", 3, 33, 72, 6, 2, 1, "f32", "stack", layers=2), False, False, False, 0.5),
    ("f32_n16_many_blocks", W_("cg", 1, 300, 608, 16, 4, 4, "f32", "stack", layers=2), True, True, False, 0.0),
    # N = 16 with k < 4: a chunk's first step holds active and untouched rows
    ("bf16_n16_k2", W_("ck", 2, 70, 192, 16, 2, 4, "bf16", "stack", layers=3), True, True, False, 0.1),
    ("bf16_n16_k3_nc1", W_("cl", 1, 100, 128, 16, 3, 1, "bf16", "stack", layers=2), False, False, True, 0.0),
    ("bf16_n16_k1", W_("cu", 2, 60, 128, 16, 1, 4, "bf16", "stack", layers=3), True, True, False, 0.2),
    # edge shapes: the smallest C, one-token sequences
    ("f32_c8_s1", W_("cs", 6, 1, 8, 16, 4, 4, "f32", "stack", layers=3), True, True, False, 0.0),
    ("bf16_c8_s2", W_("ct", 3, 2, 8, 5, 2, 4, "bf16", "stack", layers=2), False, True, True, 0.1),
]


def layer_params(w, layer, bias_scale):
    d = synth.make_inputs(w, seed=synth.stack_layer_seed(layer), state=False)
    if bias_scale:
        d["bias"] = (np.random.default_rng(50 + layer).standard_normal(w.P) * bias_scale).astype(np.float32)
    bf16 = w.dtype == "bf16"
    p = {"out": to_dev(d["out"], bf16), "W": to_dev(d["W"], bf16), "bias": torch.from_numpy(d["bias"]).cuda()}
    if w.ncomp == 4:
        for key in ("w4", "w8", "w12"):
            p[key] = torch.from_numpy(d[key]).cuda()
    h = {"out": synth.as_float(d, "out"), "W": synth.as_float(d, "W"), "bias": d["bias"],
         "convs": (d["w4"], d["w8"], d["w12"]) if w.ncomp == 4 else ()}
    return p, h


def conv_kw(p, w):
    return dict(w4=p["w4"], w8=p["w8"], w12=p["w12"]) if w.ncomp == 4 else {}


@pytest.mark.parametrize("name,w,in_place,save_rows,one_carry,bias_scale", CHAIN_CASES,
                         ids=[c[0] for c in CHAIN_CASES])
def test_chain_matches_oracle_per_layer(name, w, in_place, save_rows, one_carry, bias_scale):
    say(f"[chain] {name} B={w.B} S={w.S} C={w.C} N={w.N} k={w.k} nc={w.ncomp} layers={w.layers}")
    bf16 = w.dtype == "bf16"
    dt = torch.bfloat16 if bf16 else torch.float32
    T, N, C, P = w.T, w.N, w.C, w.P
    atol, rtol = tol(w)
    X = to_dev(synth.make_inputs(w, seed=0)["X"], bf16)
    desc = xhc.make_desc(w.B, w.S, C, N, w.k, w.ncomp, xhc.XHC_BF16 if bf16 else xhc.XHC_F32)
    nbytes = xhc.carry_size(desc)
    assert nbytes > 0
    carries = [torch.empty(nbytes // 4, device="cuda") for _ in range(1 if one_carry else 2)]
    params = [layer_params(w, layer, bias_scale) for layer in range(w.layers)]
    h_in = torch.empty(T, C, dtype=dt, device="cuda")
    z_save = torch.empty(T, P + 1, device="cuda")
    xact = torch.empty(T, w.k, C, dtype=dt, device="cuda") if save_rows else None
    for layer in range(w.layers):
        p, h = params[layer]
        active = synth.active_streams(layer, N, w.k)
        carry_in = carries[layer % len(carries)] if layer > 0 else None
        last = layer + 1 == w.layers
        W_next = None if last else params[layer + 1][0]["W"]
        carry_out = None if last else carries[(layer + 1) % len(carries)]
        Xh = to_host(X)
        X_new = X if in_place else torch.empty_like(X)
        xhc.forward(X, p["out"], None if carry_in is not None else p["W"], active, X_new, h_in, B=w.B, S=w.S,
                    bias=p["bias"], z_save=z_save, xact_save=xact, desc=desc, carry_in=carry_in,
                    W_next=W_next, carry_out=carry_out, **conv_kw(p, w))
        torch.cuda.synchronize()
        ref = xo.forward(Xh, h["out"], h["W"], h["bias"], active, h["convs"], B=w.B, S=w.S)
        got = to_host(X_new)
        inactive = [i for i in range(N) if i not in active]
        assert np.array_equal(got[:, inactive], Xh[:, inactive]), f"layer {layer}: pass-through rows differ"
        check_close(f"L{layer} X_new[active]", got[:, active], ref["X_new"][:, active], atol, rtol)
        check_close(f"L{layer} h_in", to_host(h_in), ref["h_in"], atol, rtol)
        check_close(f"L{layer} z", to_host(z_save)[:, :P], ref["z"], atol, rtol)
        check_close(f"L{layer} r", to_host(z_save)[:, P], ref["r"], atol, rtol)
        if save_rows:
            assert np.array_equal(to_host(xact), Xh[:, active]), f"layer {layer}: saved rows differ"
        X = X_new


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wname", ["stack48", "stack48_alt"])
def test_chain_stack48_shape_sampled(wname):
    """The stacked workloads' shape (S = 8192, C = 7168) for four chained
    layers, teacher-forced, on sampled token blocks (an 11-token lead-in
    makes each block's outputs exact).  stack48_alt alternates sublayers with
    one component and with TFA."""
    import dataclasses
    w = synth.WORKLOADS[wname]
    layers, n, lead = 4, 16, 11
    say(f"[chain] {wname} shape S={w.S} C={w.C} layers={layers}")
    t_start = time.time()
    T, N, C = w.T, w.N, w.C
    X = to_dev(synth.make_inputs(w, seed=0)["X"], True)
    lw = [dataclasses.replace(w, ncomp=synth.layer_ncomp(w, layer), layers=1) for layer in range(layers)]
    descs = [xhc.make_desc(w.B, w.S, C, N, w.k, wl.ncomp, xhc.XHC_BF16) for wl in lw]
    carries = [torch.empty(max(xhc.carry_size(dsc) for dsc in descs) // 4, device="cuda") for _ in range(2)]
    params = [layer_params(lw[layer], layer, 0.0) for layer in range(layers)]
    h_in = torch.empty(T, C, dtype=torch.bfloat16, device="cuda")
    blocks = [0, 4096 - 5, w.S - n]
    for layer in range(layers):
        p, h = params[layer]
        P = lw[layer].P
        z_save = torch.empty(T, P + 1, device="cuda")
        active = synth.active_streams(layer, N, w.k)
        before = {s: to_host(X[max(0, s - lead):s + n]) for s in blocks}
        last = layer + 1 == layers
        xhc.forward(X, p["out"], p["W"], active, X, h_in, B=w.B, S=w.S, bias=p["bias"], z_save=z_save,
                    desc=descs[layer], carry_in=carries[layer % 2] if layer > 0 else None,
                    W_next=None if last else params[layer + 1][0]["W"],
                    carry_out=None if last else carries[(layer + 1) % 2],
                    desc_next=None if last else descs[layer + 1], **conv_kw(p, lw[layer]))
        torch.cuda.synchronize()
        for s in blocks:
            lo = max(0, s - lead)
            ref = xo.forward(before[s], h["out"][lo:s + n], h["W"], h["bias"], active, h["convs"], B=1,
                             S=s + n - lo, iters=w.iters, eps=w.eps)
            k0 = s - lo
            got = to_host(X[s:s + n])
            inactive = [i for i in range(N) if i not in active]
            assert np.array_equal(got[:, inactive], before[s][k0:, inactive]), f"layer {layer}: pass-through"
            check_close(f"L{layer} X_new[s={s}]", got[:, active], ref["X_new"][k0:, active], 1e-2, 1e-2)
            check_close(f"L{layer} h_in[s={s}]", to_host(h_in[s:s + n]), ref["h_in"][k0:], 1e-2, 1e-2)
            check_close(f"L{layer} z[s={s}]", to_host(z_save[s:s + n])[:, :P], ref["z"][k0:], 1e-2, 1e-2)
        say(f" layer {layer} ok at {time.time() - t_start:.1f}s")


# name, base workload, per-layer (k, ncomp): the chain between sublayers of
# different descriptions (attention-side sublayers with one component,
# MLP-side ones with TFA, different k), so P and the tile count change
ALT_CASES = [
    ("bf16_attn_mlp", W_("ca", 2, 45, 200, 16, 4, 4, "bf16", "stack"), [(4, 1), (4, 4), (4, 1), (4, 4)]),
    ("f32_n4_tiles_change", W_("cb", 3, 33, 72, 4, 4, 4, "f32", "stack"), [(4, 4), (4, 1), (2, 4), (3, 1)]),
    ("bf16_k_varies", W_("cc", 1, 130, 128, 16, 4, 4, "bf16", "stack"), [(4, 4), (2, 4), (3, 1)]),
    # MLP-side sublayers with Gram-Schmidt over their four components
    ("bf16_attn_mlp_gs", W_("cd", 2, 40, 136, 16, 4, 4, "bf16", "stack"), [(4, 1), (4, 4, True), (4, 1), (4, 4, True)]),
]


@pytest.mark.parametrize("name,w,spec", ALT_CASES, ids=[c[0] for c in ALT_CASES])
def test_chain_across_different_descriptions(name, w, spec):
    import dataclasses
    say(f"[chain alt] {name} B={w.B} S={w.S} C={w.C} N={w.N} layers={spec}")
    bf16 = w.dtype == "bf16"
    dt = torch.bfloat16 if bf16 else torch.float32
    T, N, C = w.T, w.N, w.C
    code = xhc.XHC_BF16 if bf16 else xhc.XHC_F32
    spec = [tuple(sp) + (False,) * (3 - len(sp)) for sp in spec]
    ws = [dataclasses.replace(w, k=k, ncomp=nc, layers=1, gs=gs) for k, nc, gs in spec]
    descs = [xhc.make_desc(w.B, w.S, C, N, k, nc, code, gram_schmidt=gs) for k, nc, gs in spec]
    params = [layer_params(wl, l, 0.2) for l, wl in enumerate(ws)]
    X = to_dev(synth.make_inputs(w, seed=0)["X"], bf16)
    nbytes = max(xhc.carry_size(dsc) for dsc in descs)
    carries = [torch.empty(nbytes // 4, device="cuda") for _ in range(2)]
    h_in = torch.empty(T, C, dtype=dt, device="cuda")
    for l, wl in enumerate(ws):
        p, h = params[l]
        atol, rtol = tol(wl)
        active = synth.active_streams(l, N, wl.k)
        last = l + 1 == len(ws)
        z_save = torch.empty(T, wl.P + 1, device="cuda")
        Xh = to_host(X)
        xhc.forward(X, p["out"], p["W"], active, X, h_in, B=w.B, S=w.S, bias=p["bias"], z_save=z_save,
                    desc=descs[l], carry_in=carries[l % 2] if l > 0 else None,
                    W_next=None if last else params[l + 1][0]["W"],
                    carry_out=None if last else carries[(l + 1) % 2],
                    desc_next=None if last else descs[l + 1], **conv_kw(p, wl))
        torch.cuda.synchronize()
        ref = xo.forward(Xh, h["out"], h["W"], h["bias"], active, h["convs"], B=w.B, S=w.S,
                         gram_schmidt_on=wl.gs)
        got = to_host(X)
        inactive = [i for i in range(N) if i not in active]
        assert np.array_equal(got[:, inactive], Xh[:, inactive]), f"layer {l}: pass-through rows differ"
        check_close(f"L{l} X_new[active]", got[:, active], ref["X_new"][:, active], atol, rtol)
        check_close(f"L{l} h_in", to_host(h_in), ref["h_in"], atol, rtol)
        check_close(f"L{l} z", to_host(z_save)[:, :wl.P], ref["z"], atol, rtol)

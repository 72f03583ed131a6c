"""The forward and backward captured in a HIP graph (through torch's graph
API) and replayed: the library launches only kernels on the caller's
stream, with no allocation, memset or synchronisation, so a captured step
replays exactly.  Every replay, with eager work and synchronisations
between replays, is compared bitwise with the eager result (the kernels are
deterministic)."""
import numpy as np
import pytest
import torch

from residual_stream_architecture_amd import synth
from residual_stream_architecture_amd import xhc
from tests.gpu_util import device_inputs, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gs,route", [(False, 0), (True, 0), (False, 2)])
def test_forward_backward_graph_replays_match_eager(gs, route):
    w = synth.Workload("g", 2, 96, 256, 16, 4, 4, "bf16", "fwdbwd", route=route)
    say(f"[graph] B={w.B} S={w.S} C={w.C} gram_schmidt={gs} route={route}")
    d = synth.make_inputs(w, seed=21, grads=True)
    if route:
        d.update(synth.make_router(w, 21))
    dev = device_inputs(d, True)
    T, N, C, P = w.T, w.N, w.C, w.P
    active = [3, 7, 11, 15]
    desc = xhc.make_desc(w.B, w.S, C, N, 4, 4, xhc.XHC_BF16, gram_schmidt=gs, route=route)
    ridx = torch.empty(T, 4, dtype=torch.int32, device="cuda")
    rkw_f = dict(W_route=dev["W_route"], b_route=dev["b_route"], route_idx=ridx) if route else {}
    ws_f = torch.empty(xhc.workspace_size(desc, 0), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(xhc.workspace_size(desc, 1), dtype=torch.uint8, device="cuda")
    conv = dict(w4=dev["w4"], w8=dev["w8"], w12=dev["w12"])

    def buffers():
        b = dict(Xn=torch.empty_like(dev["X"]), h_in=torch.empty(T, C, dtype=torch.bfloat16, device="cuda"),
                 z=torch.empty(T, xhc.zsave_stride(desc), device="cuda"), dX=torch.empty_like(dev["X"]),
                 dout=torch.empty(T, C, dtype=torch.bfloat16, device="cuda"),
                 dW=torch.empty(N * C, P, device="cuda"), db=torch.empty(P, device="cuda"),
                 dw4=torch.empty(C, 4, device="cuda"), dw8=torch.empty(C, 8, device="cuda"),
                 dw12=torch.empty(C, 12, device="cuda"))
        if route:
            b.update(dWr=torch.empty(N * C, N, device="cuda"), dbr=torch.empty(N, device="cuda"))
        return b

    def step(b):
        # out of place, so that a replay starts from the same state
        xhc.forward(dev["X"], dev["out"], dev["W"], active, b["Xn"], b["h_in"], B=w.B, S=w.S, bias=dev["bias"],
                    z_save=b["z"], workspace=ws_f, desc=desc, **conv, **rkw_f)
        rkw_b = dict(W_route=dev["W_route"], route_idx=ridx, dW_route=b["dWr"], db_route=b["dbr"]) if route else {}
        xhc.backward(dev["X"], dev["out"], dev["W"], active, dev["dX_new"], dev["dh_in"], b["dX"], b["dout"],
                     b["dW"], B=w.B, S=w.S, bias=dev["bias"], z_save=b["z"], db=b["db"], dw4=b["dw4"],
                     dw8=b["dw8"], dw12=b["dw12"], workspace=ws_b, desc=desc, **conv, **rkw_b)

    eager = buffers()
    step(eager)
    torch.cuda.synchronize()

    static = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm the capture stream, as torch advises
        step(static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(static)
    torch.cuda.synchronize()

    other = buffers()
    for rep in range(3):
        for t in static.values():
            t.zero_()                       # eager work between replays
        step(other)                         # and an eager step on other buffers
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in eager:
            assert torch.equal(static[key], eager[key]), f"replay {rep}: {key} differs from the eager result"
        say(f"  replay {rep} bitwise equal")
    for key in eager:
        assert torch.equal(other[key], eager[key]), key
    assert np.isfinite(eager["dW"].cpu().numpy()).all()


@pytest.mark.parametrize("gs,route", [(False, 0), (False, 2), (True, 0), (True, 2)])
def test_split_calls_graph_replays_match_eager(gs, route):
    """The split forward and backward (pre, post; backward post, pre) captured
    in one graph: the state is copied in first (a copy kernel), since the post
    call rewrites it in place.  Also with Gram-Schmidt and with the router."""
    w = synth.Workload("gs", 2, 96, 256, 16, 4, 4, "bf16", "fwdbwd", route=route)
    say(f"[graph split] B={w.B} S={w.S} C={w.C} gram_schmidt={gs} route={route}")
    d = synth.make_inputs(w, seed=23, grads=True)
    if route:
        d.update(synth.make_router(w, 23))
    dev = device_inputs(d, True)
    T, N, C, P = w.T, w.N, w.C, w.P
    active = [1, 6, 11, 12]
    desc = xhc.make_desc(w.B, w.S, C, N, 4, 4, xhc.XHC_BF16, gram_schmidt=gs, route=route)
    ws_f = torch.empty(xhc.workspace_size(desc, 0), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(xhc.workspace_size(desc, 1), dtype=torch.uint8, device="cuda")
    conv = dict(w4=dev["w4"], w8=dev["w8"], w12=dev["w12"])

    def buffers():
        b = dict(X=torch.empty_like(dev["X"]), h_in=torch.empty(T, C, dtype=torch.bfloat16, device="cuda"),
                 z=torch.empty(T, xhc.zsave_stride(desc), device="cuda"),
                 xact=torch.empty(T, 4, C, dtype=torch.bfloat16, device="cuda"),
                 st=torch.empty(xhc.bwd_state_size(desc) // 4, device="cuda"), dX=torch.empty_like(dev["X"]),
                 dout=torch.empty(T, C, dtype=torch.bfloat16, device="cuda"),
                 dW=torch.empty(N * C, P, device="cuda"), db=torch.empty(P, device="cuda"),
                 dw4=torch.empty(C, 4, device="cuda"), dw8=torch.empty(C, 8, device="cuda"),
                 dw12=torch.empty(C, 12, device="cuda"))
        if route:
            b.update(ridx=torch.empty(T, 4, dtype=torch.int32, device="cuda"),
                     dWr=torch.empty(N * C, N, device="cuda"), dbr=torch.empty(N, device="cuda"))
        return b

    def step(b):
        pre_kw = dict(W_route=dev["W_route"], b_route=dev["b_route"], route_idx=b["ridx"]) if route else {}
        lists = dict(route_idx=b["ridx"]) if route else {}
        bpre_kw = dict(W_route=dev["W_route"], route_idx=b["ridx"], dW_route=b["dWr"], db_route=b["dbr"]) \
            if route else {}
        b["X"].copy_(dev["X"])
        xhc.forward_pre(b["X"], dev["W"], active, b["h_in"], b["z"], desc=desc, bias=dev["bias"], workspace=ws_f,
                        **pre_kw)
        xhc.forward_post(b["X"], dev["out"], active, b["z"], desc=desc, xact_save=b["xact"], workspace=ws_f,
                         **conv, **lists)
        xhc.backward_post(dev["out"], active, b["z"], dev["dX_new"], b["dout"], b["st"], desc=desc, workspace=ws_b,
                          dw4=b["dw4"], dw8=b["dw8"], dw12=b["dw12"], **conv, **lists)
        xhc.backward_pre(b["X"], dev["W"], active, b["z"], dev["dX_new"], dev["dh_in"], b["st"], b["dX"], b["dW"],
                         desc=desc, xact=b["xact"], bias=dev["bias"], db=b["db"], workspace=ws_b, **bpre_kw)

    eager = buffers()
    step(eager)
    torch.cuda.synchronize()
    static = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(static)
    torch.cuda.synchronize()
    other = buffers()
    for rep in range(3):
        for t in static.values():
            t.zero_()
        step(other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in eager:
            if key == "st":
                continue                    # the state's unused dot slots are never written
            assert torch.equal(static[key], eager[key]), f"replay {rep}: {key} differs from the eager result"
        say(f"  replay {rep} bitwise equal")
    assert np.isfinite(eager["dW"].cpu().numpy()).all()

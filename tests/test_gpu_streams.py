"""Calls on a stream other than torch's current one, with the workspace left
to the binding: it allocates the workspace on the current stream and records
it on the launch stream, so the caching allocator cannot hand the block to
other work before the call's kernels have finished.  The side-stream results
must be bitwise those of the same calls on the current stream; between the
calls, other work on the current stream allocates and overwrites memory of
the workspace's size, which would corrupt a workspace freed too early."""
import pytest
import torch

from residual_stream_architecture_amd import synth
from residual_stream_architecture_amd import xhc
from tests.gpu_util import device_inputs, say

pytestmark = pytest.mark.gpu


def step(w, dev, stream):
    T, N, C, P, k = w.T, w.N, w.C, w.P, w.k
    X = dev["X"].clone()
    h_in = torch.empty(T, C, dtype=X.dtype, device="cuda")
    z_save = torch.empty(T, P + 1, device="cuda")
    xact = torch.empty(T, k, C, dtype=X.dtype, device="cuda")
    dX = torch.empty_like(dev["dX_new"])
    dout = torch.empty(T, C, dtype=X.dtype, device="cuda")
    dW = torch.empty(N * C, P, device="cuda")
    dws = {key: torch.empty(C, K, device="cuda") for key, K in (("dw4", 4), ("dw8", 8), ("dw12", 12))}
    conv = dict(w4=dev["w4"], w8=dev["w8"], w12=dev["w12"])
    active = [3, 7, 0, 12]
    if stream is not None:
        stream.wait_stream(torch.cuda.current_stream())
    xhc.forward(X, dev["out"], dev["W"], active, X, h_in, B=w.B, S=w.S, bias=dev["bias"], z_save=z_save,
                xact_save=xact, stream=stream, **conv)
    # other work on the current stream, sized like the freed workspaces
    scratch = [torch.full((xhc.workspace_size(xhc.make_desc(w.B, w.S, C, N, k, 4, xhc.XHC_BF16), ph),),
                          7, dtype=torch.uint8, device="cuda") for ph in (0, 1)]
    xhc.backward(X, dev["out"], dev["W"], active, dev["dX_new"], dev["dh_in"], dX, dout, dW, B=w.B, S=w.S,
                 xact=xact, bias=dev["bias"], z_save=z_save, stream=stream, **conv, **dws)
    scratch += [torch.full((xhc.workspace_size(xhc.make_desc(w.B, w.S, C, N, k, 4, xhc.XHC_BF16), 1),),
                           9, dtype=torch.uint8, device="cuda")]
    del scratch
    if stream is not None:
        torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    return dict(X=X, h_in=h_in, z_save=z_save, dX=dX, dout=dout, dW=dW, **dws)


def test_side_stream_with_automatic_workspace():
    w = synth.Workload("side", 2, 200, 512, 16, 4, 4, "bf16", "fwdbwd")
    say(f"[streams] B={w.B} S={w.S} C={w.C}")
    d = synth.make_inputs(w, seed=3, grads=True)
    dev = device_inputs(d, True)
    ref = step(w, dev, None)
    side = torch.cuda.Stream()
    for rep in range(3):
        got = step(w, dev, side)
        for key in ref:
            a, b = ref[key], got[key]
            iv = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(a.view(iv), b.view(iv)), f"rep {rep}: {key} differs on the side stream"
    say("  side-stream results bitwise equal to the current stream's")

"""xhc_forward_noalloc (the forward with the library's static scratch array
instead of a workspace) against xhc_forward on the same inputs, through the
C ABI: two calls in a row, the second on a smaller problem (the array keeps
the first call's contents), each compared element by element.  The two
entry points run the same kernels in the same launch configuration, so the
results must be bitwise equal -- a stricter bar than the oracle tolerance."""
import numpy as np
import pytest
import torch

from residual_stream_architecture_amd import synth
from residual_stream_architecture_amd import xhc
from tests.gpu_util import device_inputs, say

pytestmark = pytest.mark.gpu
W_ = synth.Workload

# the first problem, then a smaller one in another storage type
CASES = [
    W_("na", 2, 300, 256, 16, 4, 4, "bf16", "fwd"),
    W_("nb", 1, 70, 64, 16, 4, 4, "f32", "fwd"),
]


def run(w, dev, noalloc):
    bf16 = w.dtype == "bf16"
    T, C, k, P = w.T, w.C, w.k, w.P
    X = dev["X"].clone()
    h_in = torch.empty(T, C, dtype=X.dtype, device=X.device)
    z_save = torch.full((T, P + 1), float("nan"), device=X.device)
    xact = torch.empty(T, k, C, dtype=X.dtype, device=X.device)
    active = synth.active_streams(1, w.N, k)
    kw = dict(B=w.B, S=w.S, w4=dev["w4"], w8=dev["w8"], w12=dev["w12"], bias=dev["bias"], z_save=z_save,
              xact_save=xact)
    if noalloc:
        xhc.forward_noalloc(X, dev["out"], dev["W"], active, X, h_in, **kw)
    else:
        xhc.forward(X, dev["out"], dev["W"], active, X, h_in, **kw)
    torch.cuda.synchronize()
    assert bf16 == (X.dtype == torch.bfloat16)
    return {"X_new": X, "h_in": h_in, "z_save": z_save, "xact": xact}


def test_noalloc_matches_forward_twice():
    for i, w in enumerate(CASES):
        say(f"[noalloc] call {i}: B={w.B} S={w.S} C={w.C} N={w.N} k={w.k} {w.dtype}")
        d = synth.make_inputs(w, seed=10 + i)
        dev = device_inputs(d, w.dtype == "bf16")
        ref = run(w, dev, noalloc=False)
        got = run(w, dev, noalloc=True)
        for key in ref:
            a = ref[key].view(torch.int16 if ref[key].dtype == torch.bfloat16 else torch.int32)
            b = got[key].view(torch.int16 if got[key].dtype == torch.bfloat16 else torch.int32)
            same = torch.equal(a, b)
            say(f"  {key}: bitwise equal {same}")
            assert same, f"call {i}: {key} differs"
        assert np.isfinite(got["z_save"].cpu().numpy()).all()

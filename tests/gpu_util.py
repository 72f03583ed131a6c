"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library through its binding, compare with the oracle."""
import sys

import numpy as np
import torch

from residual_stream_architecture_amd import synth

DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, bf16):
    """numpy float32 or uint16-bf16-bits -> device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.to(torch.bfloat16) if bf16 else t


def to_host(t):
    """device tensor -> float64 numpy (exact for bf16 and fp32)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def device_inputs(d, bf16):
    dev = {}
    for key, a in d.items():
        if key in ("w4", "w8", "w12", "bias", "b_route"):
            dev[key] = torch.from_numpy(a).to(DEV)
        else:
            dev[key] = to_dev(a, bf16)
    return dev


def host_inputs(d):
    return {k: synth.as_float(d, k) for k in d}


def check_close(name, got, ref, atol, rtol):
    """max over elements of |got - ref| - (atol + rtol |ref|) must be <= 0."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    excess = err - bound
    worst = np.unravel_index(np.argmax(excess), excess.shape) if excess.size else None
    ok = excess.size == 0 or excess.max() <= 0
    say(f"  {name}: max|err|={err.max() if err.size else 0:.3e} "
        f"max|ref|={np.abs(ref).max() if ref.size else 0:.3e} ok={ok}")
    assert ok, f"{name}: err {err[worst]:.4e} > {bound[worst]:.4e} at {worst} (got {got[worst]}, ref {ref[worst]})"

"""The oracle against its stored regression record (no GPU)."""
import json
import os

import numpy as np

from oracle import xhc_oracle as xo
from residual_stream_architecture_amd import synth

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tiny_forward_matches_golden_record():
    with open(os.path.join(HERE, "tiny_forward_sample.json")) as fh:
        g = json.load(fh)
    w = synth.WORKLOADS[g["workload"]]
    d = synth.make_inputs(w, seed=g["seed"])
    f = xo.forward(d["X"], d["out"], d["W"], d["bias"], g["active"],
                   (d["w4"], d["w8"], d["w12"]), B=w.B, S=w.S, iters=w.iters, eps=w.eps)
    pos, ch = g["positions"], g["channels"]
    np.testing.assert_allclose(f["X_new"][pos][:, :4][:, :, ch], g["X_new_active"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f["h_in"][pos][:, ch], g["h_in"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f["H_res"][pos], g["H_res"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f["r"][pos], g["r"], rtol=1e-12)

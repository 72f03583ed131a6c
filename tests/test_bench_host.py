"""bench.py's host-side contract, no GPU: it refuses more than one GPU, its
algorithmic byte model matches the per-token accounting in units of C, and
a committed HBM-counter record is used only while the kernel's sources keep
the digest the record was taken on."""
import json
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
from residual_stream_architecture_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_byte_model_in_units_of_c():
    w = synth.WORKLOADS["fwdbwd4096"]
    unit = w.T * w.C * 2
    wb = w.N * w.C * w.P * 2
    kb = bench.kernel_bytes(w, 2)
    assert kb["proj"] == 16 * unit + wb
    assert kb["mix"] == 26 * unit
    assert kb["bxdots"] == 21 * unit
    assert kb["bdots"] == 6 * unit
    assert kb["bgrad"] == 49 * unit + wb
    assert kb["mixproj"] == 22 * unit + wb
    assert bench.kernel_bytes(w, 2, save_rows=False)["mix"] == 22 * unit
    g = bench.kernel_bytes(synth.WORKLOADS["fwdbwd4096_gs"], 2)
    assert g["gram"] == unit and g["bdots"] == 5 * unit and g["bdots_gs"] == 6 * unit


def test_traffic_record_follows_the_sources(monkeypatch):
    path = os.path.join(ROOT, "profiles", "pmc_bgrad_fwdbwd4096.md")
    if not os.path.exists(path):
        pytest.skip("no committed counter record")
    rec = json.loads(open(path).read().split("```json\n")[1].split("\n```")[0])
    if rec["source_digest"] != bench.source_digest("bgrad"):
        pytest.skip("the record predates the current sources")
    assert bench.measured_traffic("bgrad", "fwdbwd4096") == rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "source_digest", lambda kernel=None: "0" * 16)
    assert bench.measured_traffic("bgrad", "fwdbwd4096") is None
    assert bench.measured_traffic("bgrad", "no-such-workload") is None

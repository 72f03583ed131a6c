"""GPU check of the status word for per-token active lists
(desc.per_token_active = 1): tokens whose list holds an id outside [0, N)
or an id twice are reported in status[0] (XHC_STATUS_* flags, ORed) and
counted in status[1], by the forward and by the backward; valid lists leave
the word at zero.  Every access stays inside the buffers (such ids read as
stream 0, a repeat writes its row twice), and the tokens with valid lists
get exactly the results of a run in which every list is valid: the forward
computes each token from its own list only."""
import numpy as np
import pytest
import torch

from residual_stream_architecture_amd import synth
from residual_stream_architecture_amd import xhc
from tests.gpu_util import device_inputs, say

pytestmark = pytest.mark.gpu
W_ = synth.Workload

CASES = [
    ("bf16_n16_k4", W_("st", 2, 50, 136, 16, 4, 4, "bf16", "fwdbwd")),
    ("f32_n7_k3", W_("st", 3, 30, 40, 7, 3, 1, "f32", "fwdbwd")),
]


def valid_lists(w, seed):
    r = np.random.default_rng(seed)
    return np.stack([r.permutation(w.N)[:w.k] for _ in range(w.T)]).astype(np.int32)


def corrupt(w, lists):
    """Bad lists at a few tokens: (token, expected flags)."""
    bad = lists.copy()
    R, P = xhc.XHC_STATUS_ID_RANGE, xhc.XHC_STATUS_ID_REPEAT
    cases = [(3, R), (7, R), (11, P), (w.T - 1, R | P)]
    bad[3, 0] = w.N                                   # one past the last stream
    bad[7, w.k - 1] = -1
    bad[11, 1] = bad[11, 0]                           # a repeated stream
    bad[w.T - 1, 0] = 1 << 30
    bad[w.T - 1, 2] = bad[w.T - 1, 1]
    return bad, cases


def run_forward(w, dev, desc, lists, status):
    T, C = w.T, w.C
    X = dev["X"].clone()
    h_in = torch.empty(T, C, dtype=X.dtype, device=X.device)
    z_save = torch.empty(T, xhc.zsave_stride(desc), device=X.device)
    xact = torch.empty(T, w.k, C, dtype=X.dtype, device=X.device)
    conv = dict(w4=dev["w4"], w8=dev["w8"], w12=dev["w12"]) if w.ncomp == 4 else {}
    xhc.forward(X, dev["out"], dev["W"], [0] * w.k, X, h_in, B=w.B, S=w.S, z_save=z_save, xact_save=xact,
                desc=desc, route_idx=lists, status=status, **conv)
    return X, h_in, z_save, xact


def run_backward(w, dev, desc, lists, status, X, xact, z_save):
    T, N, C, P = w.T, w.N, w.C, w.P
    f32 = dict(dtype=torch.float32, device=X.device)
    o = dict(dX=torch.empty_like(dev["dX_new"]), dout=torch.empty(T, C, dtype=X.dtype, device=X.device),
             dW=torch.empty((N * C, P), **f32))
    grads = {}
    conv = {}
    if w.ncomp == 4:
        conv = dict(w4=dev["w4"], w8=dev["w8"], w12=dev["w12"])
        grads = {key: torch.empty((C, K), **f32) for key, K in (("dw4", 4), ("dw8", 8), ("dw12", 12))}
    xhc.backward(X, dev["out"], dev["W"], [0] * w.k, dev["dX_new"], dev["dh_in"], o["dX"], o["dout"], o["dW"],
                 B=w.B, S=w.S, xact=xact, z_save=z_save, desc=desc, route_idx=lists, status=status, **conv,
                 **grads)
    return o


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_bad_lists_are_reported(name, w):
    say(f"[lists status] {name} B={w.B} S={w.S} C={w.C} N={w.N} k={w.k} nc={w.ncomp} {w.dtype}")
    d = synth.make_inputs(w, seed=9, grads=True)
    dev = device_inputs(d, w.dtype == "bf16")
    desc = xhc.make_desc(w.B, w.S, w.C, w.N, w.k, w.ncomp, xhc.XHC_BF16 if w.dtype == "bf16" else xhc.XHC_F32,
                         per_token_active=True)
    good = valid_lists(w, 4)
    bad, cases = corrupt(w, good)
    good_d = torch.from_numpy(good).cuda()
    bad_d = torch.from_numpy(bad).cuda()
    flags = 0
    for _, f in cases:
        flags |= f

    st = torch.zeros(2, dtype=torch.int32, device="cuda")
    Xg, hg, zg, xg = run_forward(w, dev, desc, good_d, st)
    torch.cuda.synchronize()
    assert st.tolist() == [0, 0], "valid lists reported"
    Xb, hb, zb, xb = run_forward(w, dev, desc, bad_d, st)
    torch.cuda.synchronize()
    assert st.tolist() == [flags, len(cases)], st.tolist()
    # the word accumulates: a second call adds its count
    run_forward(w, dev, desc, bad_d, st)
    torch.cuda.synchronize()
    assert st.tolist() == [flags, 2 * len(cases)]

    # tokens with valid lists: bitwise the all-valid results
    ok = np.ones(w.T, dtype=bool)
    ok[[t for t, _ in cases]] = False
    okd = torch.from_numpy(ok).cuda()
    assert torch.equal(Xb[okd], Xg[okd]) and torch.equal(hb[okd], hg[okd])
    assert torch.equal(zb[okd], zg[okd]) and torch.equal(xb[okd], xg[okd])
    # a flagged token's rows stay finite (out-of-range ids read as stream 0)
    assert torch.isfinite(Xb.float()).all()

    st.zero_()
    run_backward(w, dev, desc, good_d, st, Xg, xg, zg)
    torch.cuda.synchronize()
    assert st.tolist() == [0, 0]
    o = run_backward(w, dev, desc, bad_d, st, Xb, xb, zb)
    torch.cuda.synchronize()
    assert st.tolist() == [flags, len(cases)], st.tolist()
    assert torch.isfinite(o["dX"].float()).all() and torch.isfinite(o["dW"]).all()
    # without a status word the calls run as before
    run_forward(w, dev, desc, bad_d, None)
    torch.cuda.synchronize()

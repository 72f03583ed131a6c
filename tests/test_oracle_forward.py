"""Pins of the oracle's forward pass against facts fixed by the pages and by
mathematics (no GPU).  Each test names the passage or the closed form it
checks; a plausible slip in the oracle (a dropped term, a swapped index, a
transposed operand, a wrong tap orientation) fails at least one of them."""

import numpy as np
import pytest
import torch

from oracle import xhc_oracle as xo
from residual_stream_architecture_amd import synth

RNG = np.random.default_rng(1234)


def rand_case(B=1, S=7, C=5, N=6, k=3, ncomp=4, scale_w=0.3, seed=0):
    r = np.random.default_rng(seed)
    T = B * S
    P = xo.n_logits(N, k, ncomp)
    X = r.standard_normal((T, N, C))
    out = r.standard_normal((T, C))
    W = r.standard_normal((N * C, P)) * scale_w
    bias = r.standard_normal(P) * 0.5
    convs = tuple(r.standard_normal((C, K)) * 0.5 for K in xo.TFA_KERNEL_SIZES[:ncomp - 1])
    active = list(r.permutation(N)[:k])
    return dict(X=X, out=out, W=W, bias=bias, convs=convs, active=active, B=B, S=S)


def fwd(c, **kw):
    return xo.forward(c["X"], c["out"], c["W"], c["bias"], c["active"], c["convs"],
                      B=c["B"], S=c["S"], **kw)


# ---------------------------------------------------------------------------
# N = 1 is the ordinary residual (HC and mHC widen the single residual stream;
# retrospective section "从复现 DeepSeek mHC 开始", explainer "解决的真问题")
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_single_stream_unit_gates_is_vanilla_residual(dtype):
    r = np.random.default_rng(7)
    B, S, C = 2, 9, 11
    X = r.standard_normal((B * S, 1, C)).astype(dtype)
    out = r.standard_normal((B * S, C)).astype(dtype)
    W = r.standard_normal((C, 3))
    res = xo.forward(X, out, W, None, [0], (), B=B, S=S, gate_mode="unit")
    # bitwise: x' = x + out, h_in = x
    assert np.array_equal(res["X_new"][:, 0, :], X[:, 0, :].astype(np.float64) + out)
    assert np.array_equal(res["h_in"], X[:, 0, :].astype(np.float64))
    assert np.array_equal(res["H_res"], np.ones((B * S, 1, 1)))


def test_single_stream_sigmoid_gates():
    # With W = 0 the logits equal the bias: x' = x + sigmoid(b_post) out,
    # h_in = sigmoid(b_pre) x.  sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4.
    r = np.random.default_rng(8)
    S, C = 6, 4
    X = r.standard_normal((S, 1, C))
    out = r.standard_normal((S, C))
    bias = np.array([np.log(3.0), -np.log(3.0), 5.0])
    res = xo.forward(X, out, np.zeros((C, 3)), bias, [0], (), B=1, S=S)
    np.testing.assert_allclose(res["h_in"], 0.75 * X[:, 0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(res["X_new"][:, 0], X[:, 0] + 0.25 * out, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# A hand-worked case pinning the bias -> pre/post column layout, the tap
# orientation of the causal convolutions, the dense read and the sparse write
# (retrospective sections on TFA and on Dense Read / Sparse Write).
# ---------------------------------------------------------------------------

def test_hand_worked_two_stream_case():
    S, C, N, k = 3, 2, 2, 1
    X = np.arange(S * N * C, dtype=np.float64).reshape(S, N, C) * 0.5 - 1.0
    out = np.array([[1.0, -2.0], [3.0, 0.5], [-1.0, 4.0]])
    w4 = np.zeros((C, 4)); w4[:, 2] = 1.0      # tap 2 of 4 looks one token back
    w8 = np.zeros((C, 8)); w8[:, 0] = 1.0      # tap 0 of 8 looks seven back: 0 here
    w12 = np.zeros((C, 12)); w12[:, 11] = 2.0  # last tap is the current token
    P = xo.n_logits(N, k, 4)                   # 2 + 4 + 1 = 7
    bias = np.zeros(P)
    bias[0], bias[1] = 0.0, np.log(3.0)        # H_pre = [1/2, 3/4]
    res = xo.forward(X, out, np.zeros((N * C, P)), bias, [1], (w4, w8, w12), B=1, S=S)
    prev = np.vstack([np.zeros((1, C)), out[:-1]])
    # U = [out, out[s-1], 0, 2 out]; H_post = 1/2 each; H_res = [[1]]
    expect_x1 = X[:, 1] + 0.5 * out + 0.5 * prev + 0.0 + 0.5 * 2.0 * out
    np.testing.assert_allclose(res["X_new"][:, 1], expect_x1, rtol=1e-14, atol=1e-14)
    assert np.array_equal(res["X_new"][:, 0], X[:, 0])
    np.testing.assert_allclose(res["h_in"], 0.5 * X[:, 0] + 0.75 * X[:, 1], rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# zero-initialised convolution branches add exactly nothing
# (retrospective section "最便宜的新信息，可能就在相邻 token 里")
# ---------------------------------------------------------------------------

def test_zero_conv_branches_contribute_nothing():
    c = rand_case(seed=3)
    c["convs"] = tuple(np.zeros_like(w) for w in c["convs"])
    base = fwd(c)
    assert np.array_equal(base["U"][:, 1:], np.zeros_like(base["U"][:, 1:]))
    # the post columns of components 1..3 cannot matter any more
    N, k = c["X"].shape[1], len(c["active"])
    W2 = c["W"].copy()
    b2 = c["bias"].copy()
    for a in range(k):
        for m in (1, 2, 3):
            W2[:, N + a * 4 + m] = RNG.standard_normal(W2.shape[0])
            b2[N + a * 4 + m] += 3.0
    other = xo.forward(c["X"], c["out"], W2, b2, c["active"], c["convs"], B=c["B"], S=c["S"])
    assert np.array_equal(other["X_new"], base["X_new"])


# ---------------------------------------------------------------------------
# causality: nothing at a later position changes an earlier output, and the
# sequences of a batch do not see each other
# ---------------------------------------------------------------------------

def test_causality_and_batch_isolation():
    c = rand_case(B=2, S=16, seed=4)
    base = fwd(c)
    S = c["S"]
    for s in (0, 5, 11, 14):
        c2 = dict(c)
        X2, out2 = c["X"].copy(), c["out"].copy()
        X2[s + 1:S] += RNG.standard_normal(X2[s + 1:S].shape)
        out2[s + 1:S] += RNG.standard_normal(out2[s + 1:S].shape)
        c2["X"], c2["out"] = X2, out2
        pert = fwd(c2)
        assert np.array_equal(pert["X_new"][:s + 1], base["X_new"][:s + 1])
        assert np.array_equal(pert["h_in"][:s + 1], base["h_in"][:s + 1])
        # the second sequence starts over: its first positions do not move
        assert np.array_equal(pert["X_new"][S:], base["X_new"][S:])
    # the convolution does reach back: a change 11 positions earlier matters,
    # one 12 positions earlier does not (longest kernel is 12)
    out3 = c["out"].copy(); out3[3] += 1.0
    c3 = dict(c); c3["out"] = out3
    r3 = fwd(c3)
    assert not np.array_equal(r3["X_new"][14], base["X_new"][14])
    assert np.array_equal(r3["X_new"][15], base["X_new"][15])


# ---------------------------------------------------------------------------
# sparse write: inactive streams are bitwise unchanged
# (retrospective "模型可以拥有 16 条 streams，但每层只更新 4 条"; explainer
# "核心方法": the other 12 streams pass through)
# ---------------------------------------------------------------------------

def test_inactive_streams_pass_through_bitwise():
    c = rand_case(N=16, k=4, C=9, seed=5)
    res = fwd(c)
    inactive = [i for i in range(16) if i not in c["active"]]
    assert np.array_equal(res["X_new"][:, inactive], c["X"][:, inactive])
    assert not np.allclose(res["X_new"][:, c["active"]], c["X"][:, c["active"]])


# ---------------------------------------------------------------------------
# dense read: every stream reaches h_in
# ---------------------------------------------------------------------------

def test_dense_read_sees_every_stream():
    c = rand_case(N=16, k=4, C=6, seed=6)
    base = fwd(c)
    for i in range(16):
        X2 = c["X"].copy()
        X2[:, i] += 1.0
        c2 = dict(c); c2["X"] = X2
        assert not np.allclose(fwd(c2)["h_in"], base["h_in"])


# ---------------------------------------------------------------------------
# Sinkhorn (retrospective section "把 N 调大以后…": H_res is made doubly
# stochastic by Sinkhorn normalisation)
# ---------------------------------------------------------------------------

def test_sinkhorn_column_sums_exact_and_rows_close_for_small_logits():
    L = np.random.default_rng(9).standard_normal((4000, 4, 4)) * 0.64
    H, _ = xo.sinkhorn(L, 20)
    np.testing.assert_allclose(H.sum(axis=1), 1.0, atol=1e-14)
    np.testing.assert_allclose(H.sum(axis=2), 1.0, atol=1e-4)
    assert (H > 0).all()


def test_sinkhorn_keeps_cross_ratios():
    # row and column scalings leave every ratio H_ab H_cd / (H_ad H_cb)
    # unchanged, so it equals exp(L_ab + L_cd - L_ad - L_cb) for any
    # iteration count; this pins that H_res is exp(L) rescaled, not L^T or a
    # softmax along the wrong axis.
    L = np.random.default_rng(10).standard_normal((50, 4, 4)) * 3.0
    for iters in (1, 7, 20):
        H, _ = xo.sinkhorn(L, iters)
        lh = np.log(H)
        for (a, c_) in [(0, 1), (1, 3), (2, 0)]:
            for (b, d) in [(0, 2), (3, 1)]:
                got = lh[:, a, b] + lh[:, c_, d] - lh[:, a, d] - lh[:, c_, b]
                want = L[:, a, b] + L[:, c_, d] - L[:, a, d] - L[:, c_, b]
                np.testing.assert_allclose(got, want, atol=1e-9)


def test_sinkhorn_additive_logits_give_uniform():
    r = np.random.default_rng(11)
    alpha, beta = r.standard_normal((30, 4, 1)) * 4, r.standard_normal((30, 1, 4)) * 4
    H, _ = xo.sinkhorn(alpha + beta, 20)
    np.testing.assert_allclose(H, 0.25, atol=1e-12)


def test_sinkhorn_two_by_two_scalar_recurrence():
    # For 2x2, after a column step the matrix is [[p, q], [1-p, 1-q]] with the
    # cross ratio rho = p (1-q) / (q (1-p)) fixed, so one iteration is the
    # scalar map p -> (p/(p+q)) / (p/(p+q) + (1-p)/(2-p-q)),
    # q = p / (p + rho (1-p)).  This pins the iteration count and the order
    # (row step first, column step last).
    L = np.array([[1.3, -0.4], [0.2, 2.1]])
    rho = np.exp(L[0, 0] + L[1, 1] - L[0, 1] - L[1, 0])
    M = np.exp(L)
    # first row step, then the first column step, by hand
    R = M / M.sum(axis=1, keepdims=True)
    p = R[0, 0] / (R[0, 0] + R[1, 0])
    for _ in range(19):
        q = p / (p + rho * (1 - p))
        rp, rq = p / (p + q), (1 - p) / (2 - p - q)
        p = rp / (rp + rq)
    q = p / (p + rho * (1 - p))
    H, _ = xo.sinkhorn(L[None], 20)
    np.testing.assert_allclose(H[0], [[p, q], [1 - p, 1 - q]], atol=1e-14)
    H19, _ = xo.sinkhorn(L[None], 19)
    assert not np.allclose(H19[0], H[0], atol=1e-15, rtol=0)


def test_sinkhorn_tiny_config_is_near_the_limit():
    w = synth.WORKLOADS["tiny"]
    d = synth.make_inputs(w, seed=0)
    res = xo.forward(d["X"], d["out"], d["W"], d["bias"], [0, 1, 2, 3],
                     (d["w4"], d["w8"], d["w12"]), B=w.B, S=w.S)
    L = xo.split_logits(res["z"], w.N, w.k, w.ncomp)[2]
    Hlim, _ = xo.sinkhorn(L, 2000)
    np.testing.assert_allclose(res["H_res"], Hlim, atol=1e-4)
    np.testing.assert_allclose(res["H_res"].sum(axis=2), 1.0, atol=1e-4)
    np.testing.assert_allclose(res["H_res"].sum(axis=1), 1.0, atol=1e-12)


def test_sinkhorn_permutation_equivariant():
    r = np.random.default_rng(12)
    L = r.standard_normal((20, 4, 4)) * 2
    pr, pc = r.permutation(4), r.permutation(4)
    H, _ = xo.sinkhorn(L, 20)
    Hp, _ = xo.sinkhorn(L[:, pr][:, :, pc], 20)
    np.testing.assert_allclose(Hp, H[:, pr][:, :, pc], atol=1e-14)


# ---------------------------------------------------------------------------
# TFA against the library convolution (torch conv1d, cross-correlation)
# ---------------------------------------------------------------------------

def test_tfa_matches_torch_conv1d():
    r = np.random.default_rng(13)
    B, S, C = 3, 20, 7
    out = r.standard_normal((B * S, C))
    ws = tuple(r.standard_normal((C, K)) for K in (4, 8, 12))
    U = xo.tfa_components(out, B, S, ws)
    x = torch.from_numpy(out.reshape(B, S, C)).permute(0, 2, 1)     # [B, C, S]
    assert np.array_equal(U[:, 0], out)
    for m, w in enumerate(ws):
        K = w.shape[1]
        y = torch.nn.functional.conv1d(torch.nn.functional.pad(x, (K - 1, 0)),
                                       torch.from_numpy(w)[:, None, :], groups=C)
        np.testing.assert_allclose(U[:, m + 1], y.permute(0, 2, 1).reshape(B * S, C).numpy(),
                                   atol=1e-12)


def test_tfa_one_hot_reproduces_taps():
    B, S, C = 1, 30, 3
    out = np.zeros((S, C)); s0, c0 = 4, 1
    out[s0, c0] = 1.0
    ws = tuple(np.random.default_rng(14).standard_normal((C, K)) for K in (4, 8, 12))
    U = xo.tfa_components(out, B, S, ws)
    for m, w in enumerate(ws):
        K = w.shape[1]
        for q in range(K):
            assert U[s0 + K - 1 - q, m + 1, c0] == w[c0, q]
        assert np.count_nonzero(U[:, m + 1]) == np.count_nonzero(w[c0])


# ---------------------------------------------------------------------------
# projection: flatten order, RMS normalisation, column layout
# ---------------------------------------------------------------------------

def test_projection_one_hot_rows_pick_state_entries():
    r = np.random.default_rng(15)
    T, N, C = 5, 3, 4
    X = r.standard_normal((T, N, C))
    P = 6
    for (i, c, p) in [(0, 0, 0), (2, 1, 5), (1, 3, 2)]:
        W = np.zeros((N * C, P)); W[i * C + c, p] = 1.0
        z, rr, _ = xo.rms_projection(X.reshape(T, N * C), W, np.zeros(P), 0.0)
        rms = np.sqrt((X ** 2).sum(axis=(1, 2)) / (N * C))
        np.testing.assert_allclose(z[:, p], X[:, i, c] / rms, rtol=1e-14)
        assert np.count_nonzero(np.delete(z, p, axis=1)) == 0


def test_projection_rms_of_constant_state_and_scale_invariance():
    T, N, C = 3, 4, 5
    X = np.full((T, N, C), -2.5)
    _, rr, _ = xo.rms_projection(X.reshape(T, N * C), np.zeros((N * C, 2)), np.zeros(2), 1e-6)
    np.testing.assert_allclose(rr, np.sqrt(6.25 + 1e-6), rtol=1e-15)
    c = rand_case(seed=16)
    z1 = fwd(c, eps=0.0)["z"]
    c2 = dict(c); c2["X"] = c["X"] * 37.0
    np.testing.assert_allclose(fwd(c2, eps=0.0)["z"], z1, rtol=1e-12, atol=1e-12)


def test_column_layout_through_bias():
    # W = 0, logits = bias.  Saturating one post logit routes exactly one
    # component into one active stream; a permutation pattern in the res
    # logits routes the old active rows accordingly.
    r = np.random.default_rng(17)
    B, S, C, N, k = 1, 14, 3, 6, 3
    X = r.standard_normal((S, N, C))
    out = r.standard_normal((S, C))
    ws = tuple(r.standard_normal((C, K)) for K in (4, 8, 12))
    active = [4, 0, 2]
    P = xo.n_logits(N, k, 4)
    U = xo.tfa_components(out, B, S, ws)
    perm = [2, 0, 1]                 # active row a takes old active row perm[a]
    for (a, m) in [(0, 0), (1, 3), (2, 1)]:
        bias = np.full(P, -40.0)
        bias[N + a * 4 + m] = 40.0
        for aa in range(k):
            bias[N + k * 4 + aa * k + perm[aa]] = 40.0
        bias[3] = 40.0               # H_pre ~ e_3
        res = xo.forward(X, out, np.zeros((N * C, P)), bias, active, ws, B=B, S=S)
        for aa in range(k):
            want = X[:, active[perm[aa]]] + (U[:, m] if aa == a else 0.0)
            np.testing.assert_allclose(res["X_new"][:, active[aa]], want, atol=1e-12)
        np.testing.assert_allclose(res["h_in"], X[:, 3], atol=1e-12)


def test_zero_weights_closed_form():
    # W = 0, b = 0: H_pre = H_post = 1/2, H_res = 1/k exactly
    c = rand_case(N=8, k=4, seed=18)
    c["W"] = np.zeros_like(c["W"]); c["bias"] = np.zeros_like(c["bias"])
    res = fwd(c)
    act = c["active"]
    np.testing.assert_allclose(res["h_in"], 0.5 * c["X"].sum(axis=1), atol=1e-13)
    mix = c["X"][:, act].mean(axis=1)
    want = mix[:, None, :] + 0.5 * res["U"].sum(axis=1)[:, None, :]
    np.testing.assert_allclose(res["X_new"][:, act], np.repeat(want, 4, axis=1), atol=1e-13)


def test_mhc_dense_special_case():
    # N = k = 4 with identity index and one component is the mHC update
    # X' = H_res X + H_post out^T (retrospective section "把 N 调大以后…").
    c = rand_case(N=4, k=4, ncomp=1, seed=19)
    c["active"] = [0, 1, 2, 3]
    res = fwd(c)
    T = c["X"].shape[0]
    for t in range(T):
        dense = res["H_res"][t] @ c["X"][t] + np.outer(res["H_post"][t][:, 0], c["out"][t])
        np.testing.assert_allclose(res["X_new"][t], dense, atol=1e-13)


def test_stream_relabelling_equivariance():
    # Relabel the streams with a permutation pi: state rows, projection rows,
    # pre columns and active ids move together, outputs move the same way.
    c = rand_case(N=7, k=3, C=4, seed=20)
    N, C = 7, 4
    pi = np.random.default_rng(21).permutation(N)          # new stream j = old pi[j]
    inv = np.argsort(pi)
    X2 = c["X"][:, pi]
    W2 = c["W"].reshape(N, C, -1)[pi].reshape(N * C, -1).copy()
    b2 = c["bias"].copy()
    W2[:, :N] = W2[:, pi]
    b2[:N] = c["bias"][pi]
    act2 = [int(inv[a]) for a in c["active"]]
    base = fwd(c)
    res = xo.forward(X2, c["out"], W2, b2, act2, c["convs"], B=c["B"], S=c["S"])
    np.testing.assert_allclose(res["X_new"], base["X_new"][:, pi], atol=1e-12)
    np.testing.assert_allclose(res["h_in"], base["h_in"], atol=1e-12)


def test_active_order_equivariance():
    # Reordering the active list together with the post and res columns
    # leaves X' unchanged.
    c = rand_case(N=6, k=3, seed=22)
    N, k = 6, 3
    sig = [2, 0, 1]
    act2 = [c["active"][s] for s in sig]
    W2, b2 = c["W"].copy(), c["bias"].copy()
    for a in range(k):
        for m in range(4):
            W2[:, N + a * 4 + m] = c["W"][:, N + sig[a] * 4 + m]
            b2[N + a * 4 + m] = c["bias"][N + sig[a] * 4 + m]
        for bb in range(k):
            W2[:, N + 4 * k + a * k + bb] = c["W"][:, N + 4 * k + sig[a] * k + sig[bb]]
            b2[N + 4 * k + a * k + bb] = c["bias"][N + 4 * k + sig[a] * k + sig[bb]]
    res = xo.forward(c["X"], c["out"], W2, b2, act2, c["convs"], B=c["B"], S=c["S"])
    np.testing.assert_allclose(res["X_new"], fwd(c)["X_new"], atol=1e-12)


def test_active_rows_mixing_conserves_the_sum():
    # columns of H_res sum to one, so summing the rewritten rows and removing
    # the write-back leaves the sum of the old active rows (a transposed
    # H_res fails this at large logits, where its rows do not sum to one)
    c = rand_case(N=16, k=4, C=6, scale_w=3.0, seed=23)
    res = fwd(c)
    act = c["active"]
    wb = np.einsum("tam,tmc->tc", res["H_post"], res["U"])
    lhs = res["X_new"][:, act].sum(axis=1) - wb
    np.testing.assert_allclose(lhs, c["X"][:, act].sum(axis=1), atol=1e-11)
    assert np.abs(res["H_res"].sum(axis=2) - 1).max() > 1e-3   # the test has teeth


# ---------------------------------------------------------------------------
# H_res generated from the k active rows only (retrospective section
# "模型可以拥有 16 条 streams，但每层只更新 4 条": the cubic generation cost
# falls from N^3 C to k^3 C): with W's res columns zero on the rows of the
# untouched streams, the un-normalised res logits r * (z_res - b) depend on
# the active rows alone, while the pre logits still see every stream
# ---------------------------------------------------------------------------

def test_res_logits_from_active_rows_only():
    c = rand_case(N=10, k=3, C=5, seed=31)
    N, k, C = 10, 3, 5
    P0 = N + k * 4
    inactive = [i for i in range(N) if i not in c["active"]]
    for i in inactive:
        c["W"][i * C:(i + 1) * C, P0:] = 0.0
    a = fwd(c)
    c2 = dict(c)
    c2["X"] = c["X"].copy()
    c2["X"][:, inactive] = RNG.standard_normal(c2["X"][:, inactive].shape)
    b = fwd(c2)
    un_a = a["r"][:, None] * (a["z"][:, P0:] - c["bias"][P0:])
    un_b = b["r"][:, None] * (b["z"][:, P0:] - c["bias"][P0:])
    np.testing.assert_allclose(un_a, un_b, rtol=1e-12, atol=1e-12)
    assert np.abs(a["z"][:, :N] - b["z"][:, :N]).max() > 1e-3

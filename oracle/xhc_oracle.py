"""Plain CPU oracle of one xHC sublayer update (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it and shares no code with it; it imports nothing but numpy.

Everything is computed in float64 from the given inputs (bf16 inputs arrive
already rounded, as float32, and are upcast exactly).  Nothing is blocked,
fused or reordered beyond what the definition states: tokens are processed as
one batch with numpy array operations, one step of the method at a time.

Sources (three web pages on xHC, Expanded Hyper-Connections):

  [R]  "xHC: Expanded Hyper-Connections" research retrospective
       (qingkeai.online/archives/xHC, mirror of the first author's Zhihu post).
       Sections used, by heading:
         R-mHC   "把 N 调大以后，事情开始不太对了"   (the multi-stream state
                  X in R^{N x C}; H_pre reads, H_post writes, H_res mixes;
                  Sinkhorn makes H_res doubly stochastic)
         R-one   "更多 streams，为什么仍然只写入一份信息？" (write-back as
                  H_post times out^T; coefficients are dynamic, per stream)
         R-TFA   "最便宜的新信息，可能就在相邻 token 里" (causal depthwise
                  convolutions with kernel sizes 4, 8, 12 over the sublayer
                  output, stacked with it into 4 components; zero init)
         R-GS    "Conv 带来了新信息，也带来了新的麻烦" (the four components
                  u_0..u_3; optional Gram-Schmidt, dropped under Muon)
         R-cost  "N 从 4 扩展到 16，成本为什么涨得这么快？" (coefficients are
                  generated from the flattened N*C state)
         R-DRSW  "模型可以拥有 16 条 streams，但每层只更新 4 条" (dense read
                  over all N streams, sparse write to k active streams, the
                  xHC write formula, inactive streams unchanged)
  [E]  explainer "xHC：把残差流扩到 N=16 的可扩展超连接"
       (papers.ananclaw.com), section "核心方法" (wide state, narrow write;
       k=4 of N=16 updated, the other 12 pass through).

Readings where the pages are silent or their formulas were lost (each one is
shared with the GPU library and listed in the design notes):

  O1  coefficients: z = rms(xbar) ^-1 * xbar @ W + b, with xbar the token's
      flattened state, xbar[i*C + c] = X[t, i, c], and
      rms(xbar) = sqrt(mean(xbar^2) + eps).  All P = N + k*ncomp + k*k logits
      come from the full N*C state.  Column layout of z:
      [ pre (N) | post (k*ncomp, a-major) | res (k*k, a-major) ].
  O2  gates: H_pre = sigmoid(z_pre), H_post = sigmoid(z_post); in "unit" gate
      mode both are identically 1 (a test mode, used for the N=1 reduction).
  O3  H_res = Sinkhorn(L) with L the k x k res logits: M = exp(L - rowmax(L)),
      then `iters` times: divide each row by its sum, then each column by its
      sum.  No epsilon in the denominators.
  O4  TFA: U_0 = out; U_m[s, c] = sum_q w_m[c, q] * out[s - (K_m - 1) + q, c]
      for K = 4, 8, 12, positions before the start of the sequence read 0 (no
      leak between sequences of a batch); w_m[c, K_m - 1] multiplies the
      current token.
  O5  write: for active stream a (index i_a = active[a]):
        X'[t, i_a] = sum_b H_res[a, b] X[t, i_b] + sum_c H_post[a, c] U_c[t];
      every other stream is copied unchanged.  Dense read:
        h_in[t] = sum_i H_pre[i] X[t, i].
  O6  Gram-Schmidt (optional, [R-GS]; off by default, the form the pages
      keep when the backbone trains with Muon): per token, over the C
      channels, u~_0 = U_0 and for c = 1, 2, 3 in turn the component keeps
      its own direction minus its projections on the components already
      produced, removed one after another (modified Gram-Schmidt):
        v = U_c;  for j < c:  v -= <v, u~_j> / (<u~_j, u~_j> + C*gs_eps) u~_j
        u~_c = v.
      No normalisation (the output keeps its magnitude).  gs_eps (1e-6 by
      default, the RMS epsilon scaled to a sum over C) keeps a zero
      component -- the zero-initialised conv branches at the start of
      training -- from dividing 0 by 0; with it such a component stays 0.
      The write uses u~ in place of U.
  O7  router (optional, [R-DRSW], the paragraphs on fixed and routed
      streams, the sigmoid router and its gradient): the first k - R
      entries of `active` are fixed streams, written at every token; the
      other R slots are chosen per token.  The router reads the flattened
      state through a LayerNorm without affine parameters (a gain and a
      shift fold into W_route and b_route):
        y = (xbar - mean(xbar)) / sqrt(var(xbar) + eps),  var the population
        variance, eps the RMS epsilon;  rho = y @ W_route + b_route  (N scores)
      and s = sigmoid(rho).  Slot k - R + j (j = 0 .. R-1) takes the stream
      with the (j+1)-th largest rho among the streams that are not fixed;
      equal scores go to the lower stream id first.  A routed slot's
      write-back is scaled by its score:
        X'[t, i_a] = sum_b H_res[a, b] X[t, i_b] + s_a sum_c H_post[a, c] u~_c
      (s_a = 1 for a fixed slot).  The choice itself is discrete: only the
      chosen streams' scores receive a gradient, through s_a.  R = 0 is the
      fixed active list of O5.
  O8  per-token active lists given by the caller (`active_tok`, [T, k]):
      O5's write with token t's own list in place of `active`, s = 1, and
      no router.  It is the form in which another router's choice enters.
  O9  H_res from the active rows (optional, `hres_active`; [R-DRSW] credits
      the sparse write with generating H_res at k^3 C instead of N^3 C, that
      is from the k active rows only): the res logits are the RMS-normed
      projection of the k*C active state alone,
        xa = [X[t, i_0], .., X[t, i_{k-1}]] (length k*C),
        r_act = sqrt(mean(xa^2) + eps),
        L[a, b] = sum_{a'} sum_c X[t, i_{a'}, c] / r_act
                  * W[i_{a'}*C + c, N + k*ncomp + a*k + b] + bias[...]
      -- the rows of W that belong to the active streams, normalised by the
      active state's own RMS.  The pre and post logits stay O1's (full state,
      r).  W's res columns on the other streams' rows are not read, and
      their gradient is zero.  With every stream active (k = N) this is O1.
"""

import numpy as np

TFA_KERNEL_SIZES = (4, 8, 12)


def n_logits(N, k, ncomp):
    """P = N pre logits + k*ncomp post logits + k*k res logits (O1)."""
    return N + k * ncomp + k * k


# --------------------------------------------------------------------------
# forward pieces
# --------------------------------------------------------------------------

def rms_projection(Xf, W, bias, eps):
    """O1 / [R-cost], [R-DRSW]: logits from the RMS-normed flattened state.

    Xf: [T, N*C] float64.  Returns z [T, P], r [T], xhat [T, N*C].
    """
    r = np.sqrt(np.mean(Xf * Xf, axis=1) + eps)
    xhat = Xf / r[:, None]
    z = xhat @ W + bias[None, :]
    return z, r, xhat


def res_logits_active(X, W, bias, active, ncomp, eps):
    """O9: the k x k res logits from the k active rows alone.

    X: [T, N, C], W: [N*C, P].  Returns L [T, k, k], r_act [T], the normed
    active state xa_hat [T, k*C] and the weights it multiplies W_act
    [k*C, k*k] (the active streams' rows, in slot order, res columns).
    """
    T, N, C = X.shape
    k = len(active)
    res0 = N + k * ncomp
    xa = X[:, list(active), :].reshape(T, k * C)
    r_act = np.sqrt(np.mean(xa * xa, axis=1) + eps)
    xa_hat = xa / r_act[:, None]
    W_act = W.reshape(N, C, -1)[list(active)][:, :, res0:res0 + k * k].reshape(k * C, k * k)
    L = xa_hat @ W_act + bias[None, res0:res0 + k * k]
    return L.reshape(T, k, k), r_act, xa_hat, W_act


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def split_logits(z, N, k, ncomp):
    """Column layout of O1: pre | post (a-major) | res (a-major)."""
    T = z.shape[0]
    z_pre = z[:, :N]
    z_post = z[:, N:N + k * ncomp].reshape(T, k, ncomp)
    L = z[:, N + k * ncomp:N + k * ncomp + k * k].reshape(T, k, k)
    return z_pre, z_post, L


def sinkhorn(L, iters):
    """O3 / [R-mHC]: Sinkhorn normalisation of exp(L), per token.

    L: [T, k, k].  Returns H_res [T, k, k] and the list of iterates
    (the matrix after every row step and every column step), which the
    backward pass walks in reverse.
    """
    if iters < 1:
        raise ValueError("sinkhorn needs at least one iteration")
    M = np.exp(L - L.max(axis=2, keepdims=True))
    states = [M]
    for _ in range(iters):
        M = M / M.sum(axis=2, keepdims=True)      # every row sums to 1
        states.append(M)
        M = M / M.sum(axis=1, keepdims=True)      # every column sums to 1
        states.append(M)
    return M, states


def causal_depthwise_conv(out_bsc, w):
    """O4 / [R-TFA]: one causal depthwise convolution along the sequence.

    out_bsc: [B, S, C]; w: [C, K].  y[b, s, c] = sum_q w[c, q] *
    out[b, s - (K-1) + q, c], reading zero before position 0.
    """
    B, S, C = out_bsc.shape
    K = w.shape[1]
    y = np.zeros_like(out_bsc)
    for q in range(K):
        shift = K - 1 - q                 # how many positions back tap q looks
        if shift >= S:
            continue
        y[:, shift:, :] += w[None, None, :, q] * out_bsc[:, :S - shift, :]
    return y


def tfa_components(out, B, S, conv_ws):
    """[R-TFA]: U = [out, conv4(out), conv8(out), conv12(out)] -> [T, ncomp, C].

    conv_ws is () for the single-component (mHC-style) write-back.
    """
    T, C = out.shape
    out_bsc = out.reshape(B, S, C)
    comps = [out]
    for w in conv_ws:
        comps.append(causal_depthwise_conv(out_bsc, w).reshape(T, C))
    return np.stack(comps, axis=1)


def gram_schmidt(U, gs_eps):
    """O6 / [R-GS]: modified Gram-Schmidt over the components, per token.

    U: [T, m, C].  Returns (Ut [T, m, C], steps), steps = the list of
    (c, j, v_before, alpha, den) of every projection removal, in order,
    which the backward walks in reverse.
    """
    T, m, C = U.shape
    Ut = U.copy()
    steps = []
    for c in range(1, m):
        v = U[:, c, :].copy()
        for j in range(c):
            uj = Ut[:, j, :]
            den = np.sum(uj * uj, axis=1) + C * gs_eps
            alpha = np.sum(v * uj, axis=1) / den
            steps.append((c, j, v, alpha, den))
            v = v - alpha[:, None] * uj
        Ut[:, c, :] = v
    return Ut, steps


def layer_norm_flat(Xf, eps):
    """O7: LayerNorm of each token's flattened state, no affine parameters.

    Xf: [T, N*C].  Returns y [T, N*C], mean [T], sd [T]
    (sd = sqrt(population variance + eps)).
    """
    mu = Xf.mean(axis=1)
    d = Xf - mu[:, None]
    sd = np.sqrt(np.mean(d * d, axis=1) + eps)
    return d / sd[:, None], mu, sd


def route_select(rho, fixed, R):
    """O7: per-token active list -- the fixed streams, then the R streams
    that are not fixed with the largest router scores, largest first, equal
    scores to the lower stream id.  rho: [T, N].  Returns idx [T, k]."""
    T, N = rho.shape
    fixed = [int(i) for i in fixed]
    cand = np.array([i for i in range(N) if i not in fixed], dtype=np.int64)
    order = np.argsort(-rho[:, cand], axis=1, kind="stable")[:, :R]
    idx = np.empty((T, len(fixed) + R), dtype=np.int64)
    idx[:, :len(fixed)] = fixed
    idx[:, len(fixed):] = cand[order]
    return idx


def router(Xf, W_route, b_route, active, R, eps, route_idx=None):
    """O7: router scores, per-token active lists and write-back scales.

    Returns dict(idx [T,k], rho [T,N], s [T,k], y, mu, sd).  route_idx, if
    given, replaces the top-R choice (for checking another implementation's
    choice at near ties); the scores still come from rho.
    """
    T = Xf.shape[0]
    k = len(active)
    y, mu, sd = layer_norm_flat(Xf, eps)
    rho = y @ W_route + b_route[None, :]
    if route_idx is None:
        idx = route_select(rho, list(active)[:k - R], R)
    else:
        idx = np.asarray(route_idx, dtype=np.int64).reshape(T, k)
    s = np.ones((T, k))
    if R:
        s[:, k - R:] = sigmoid(np.take_along_axis(rho, idx[:, k - R:], axis=1))
    return dict(idx=idx, rho=rho, s=s, y=y, mu=mu, sd=sd)


def forward(X, out, W, bias, active, conv_ws, *, B, S, iters=20, eps=1e-6,
            gate_mode="sigmoid", gram_schmidt_on=False, gs_eps=1e-6,
            route=0, W_route=None, b_route=None, route_idx=None, active_tok=None,
            hres_active=False):
    """One xHC sublayer update, forward ([R-DRSW] write formula, O1-O5).

    X:      [B*S, N, C]  residual state before the update
    out:    [B*S, C]     sublayer output
    W:      [N*C, P]     projection weights, rows indexed i*C + c
    bias:   [P] or None
    active: k distinct stream ids; row/column a of H_res and row a of H_post
            bind to active[a] (with route = R > 0 only the first k - R are
            used: the fixed streams of O7)
    conv_ws: (w4, w8, w12) with shapes [C,4], [C,8], [C,12], or () for one
            write-back component
    route, W_route [N*C, N], b_route [N] or None, route_idx: the router of
            O7 (route = number of routed slots)
    active_tok: [T, k] per-token active lists (O8), or None
    hres_active: the res logits from the active rows (O9; fixed list only)

    Returns a dict with X_new, h_in and the intermediates (z, r, H_pre,
    H_post, H_res, U, idx [T, k] the per-token active list, s [T, k] the
    write-back scales, with a router rho, mu, sd, and with hres_active
    r_act).
    """
    X = np.asarray(X, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    conv_ws = tuple(np.asarray(w, dtype=np.float64) for w in conv_ws)
    T, N, C = X.shape
    k = len(active)
    ncomp = 1 + len(conv_ws)
    P = n_logits(N, k, ncomp)
    assert T == B * S and out.shape == (T, C) and W.shape == (N * C, P)
    fixed = list(active)[:k - route] if active_tok is None else []   # the host list entries that are read
    assert len(set(int(a) for a in fixed)) == len(fixed) and all(0 <= a < N for a in fixed)
    bias = np.zeros(P) if bias is None else np.asarray(bias, dtype=np.float64)

    # coefficients from the full flattened state (dense read of all streams)
    z, r, _ = rms_projection(X.reshape(T, N * C), W, bias, eps)
    extra = {}
    if hres_active:
        # O9: the res logits from the active rows alone
        assert not route and active_tok is None
        La, r_act, _, _ = res_logits_active(X, W, bias, active, ncomp, eps)
        z[:, N + k * ncomp:] = La.reshape(T, k * k)
        extra["r_act"] = r_act
    z_pre, z_post, L = split_logits(z, N, k, ncomp)
    if gate_mode == "sigmoid":
        H_pre, H_post = sigmoid(z_pre), sigmoid(z_post)
    elif gate_mode == "unit":
        H_pre, H_post = np.ones_like(z_pre), np.ones_like(z_post)
    else:
        raise ValueError(gate_mode)
    H_res, _ = sinkhorn(L, iters)

    # dense read: the sublayer input aggregates all N streams
    h_in = np.einsum("ti,tic->tc", H_pre, X)

    # temporal feature augmentation over the sublayer output
    U = tfa_components(out, B, S, conv_ws)
    if gram_schmidt_on:
        U, _ = gram_schmidt(U, gs_eps)

    # the per-token active list: fixed, or fixed + routed (O7)
    rt = _route(X.reshape(T, N * C), active, route, W_route, b_route, eps, route_idx, active_tok)
    idx, s = rt["idx"], rt["s"]

    # sparse write: only the k active streams are rewritten
    X_new = X.copy()
    tok = np.arange(T)[:, None]
    Xa = X[tok, idx, :]                                           # [T, k, C]
    X_new[tok, idx, :] = (np.einsum("tab,tbc->tac", H_res, Xa)
                          + s[:, :, None] * np.einsum("tam,tmc->tac", H_post, U))
    res = dict(X_new=X_new, h_in=h_in, z=z, r=r, H_pre=H_pre,
               H_post=H_post, H_res=H_res, U=U)
    res.update(rt)
    res.update(extra)
    return res


def _route(Xf, active, route, W_route, b_route, eps, route_idx, active_tok=None):
    """The per-token active list and scales: O5's fixed list (route = 0),
    O7's router, or O8's given lists."""
    T, NC = Xf.shape
    k = len(active)
    if active_tok is not None:
        assert not route
        idx = np.asarray(active_tok, dtype=np.int64).reshape(T, k)
        assert all(len(set(r)) == k for r in idx)
        return dict(idx=idx, s=np.ones((T, k)))
    if not route:
        return dict(idx=np.tile(np.asarray(active, dtype=np.int64), (T, 1)), s=np.ones((T, k)))
    assert 0 < route <= k
    W_route = np.asarray(W_route, dtype=np.float64)
    N = W_route.shape[1]
    assert W_route.shape == (NC, N) and route <= N - (k - route)
    b_route = np.zeros(N) if b_route is None else np.asarray(b_route, dtype=np.float64)
    return router(Xf, W_route, b_route, active, route, eps, route_idx)


# --------------------------------------------------------------------------
# backward pieces (derived by hand from the forward above)
# --------------------------------------------------------------------------

def sinkhorn_backward(L, iters, dH):
    """Gradient of O3 through the unrolled iterations.

    A row step R = M / rowsum(M) has dM = (dR - rowsum(dR * R)) / rowsum(M);
    a column step is the same along columns.  The row-max shift cancels in
    the first row step, so it carries no gradient; dL = dM0 * M0.
    """
    _, states = sinkhorn(L, iters)
    g = dH
    for it in range(iters, 0, -1):
        R = states[2 * it - 1]                      # after the row step
        Mc = states[2 * it]                         # after the column step
        colsum = R.sum(axis=1, keepdims=True)
        g = (g - (g * Mc).sum(axis=1, keepdims=True)) / colsum
        M = states[2 * it - 2]
        rowsum = M.sum(axis=2, keepdims=True)
        g = (g - (g * R).sum(axis=2, keepdims=True)) / rowsum
    return g * states[0]


def causal_depthwise_conv_backward(out_bsc, w, dy):
    """Adjoint of causal_depthwise_conv: returns (d_out, d_w)."""
    B, S, C = out_bsc.shape
    K = w.shape[1]
    d_out = np.zeros_like(out_bsc)
    d_w = np.zeros_like(w)
    for q in range(K):
        shift = K - 1 - q
        if shift >= S:
            continue
        # y[:, s] += w[q] * out[:, s - shift]   for s >= shift
        d_out[:, :S - shift, :] += w[None, None, :, q] * dy[:, shift:, :]
        d_w[:, q] += np.einsum("bsc,bsc->c", dy[:, shift:, :], out_bsc[:, :S - shift, :])
    return d_out, d_w


def gram_schmidt_backward(U, gs_eps, dUt):
    """Adjoint of gram_schmidt: dU from dUt, walking the removals backwards.

    One removal v' = v - alpha u~_j with alpha = <v, u~_j> / den_j and
    den_j = <u~_j, u~_j> + C*gs_eps gives, for the gradient dv' of v':
      dalpha = -<dv', u~_j>
      dv     = dv' + dalpha / den_j * u~_j
      du~_j += -alpha dv' + dalpha / den_j * (v - 2 alpha u~_j).
    u~_c = v after the last removal of component c, and the removals of
    later components only read u~_c, so u~_c's gradient is complete when
    its own removals are walked; it then flows to U_c.
    """
    Ut, steps = gram_schmidt(U, gs_eps)
    g = dUt.copy()                        # running gradient of every u~
    dU = np.zeros_like(U)
    c_cur, dv = None, None
    for c, j, v, alpha, den in reversed(steps):
        if c != c_cur:
            if c_cur is not None:
                dU[:, c_cur, :] = dv
            c_cur, dv = c, g[:, c, :].copy()
        uj = Ut[:, j, :]
        dalpha = -np.sum(dv * uj, axis=1)
        q = dalpha / den
        g[:, j, :] += -alpha[:, None] * dv + q[:, None] * (v - 2.0 * alpha[:, None] * uj)
        dv = dv + q[:, None] * uj
    if c_cur is not None:
        dU[:, c_cur, :] = dv
    dU[:, 0, :] = g[:, 0, :]
    return dU


def backward(X, out, W, bias, active, conv_ws, dX_new, dh_in, *, B, S,
             iters=20, eps=1e-6, gate_mode="sigmoid", gram_schmidt_on=False, gs_eps=1e-6,
             route=0, W_route=None, b_route=None, route_idx=None, active_tok=None,
             hres_active=False):
    """Gradients of the forward above for upstream gradients dX_new, dh_in.

    Returns dict(dX [T,N,C], dout [T,C], dW [N*C,P], db [P],
    dconv [list of [C,K]], dz [T,P]; with a router also dW_route [N*C,N],
    db_route [N], drho [T,N] and idx).
    """
    X = np.asarray(X, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    conv_ws = tuple(np.asarray(w, dtype=np.float64) for w in conv_ws)
    dX_new = np.asarray(dX_new, dtype=np.float64)
    dh_in = np.asarray(dh_in, dtype=np.float64)
    T, N, C = X.shape
    k = len(active)
    ncomp = 1 + len(conv_ws)
    P = n_logits(N, k, ncomp)
    act = list(active)
    bias = np.zeros(P) if bias is None else np.asarray(bias, dtype=np.float64)

    Xf = X.reshape(T, N * C)
    z, r, xhat = rms_projection(Xf, W, bias, eps)
    if hres_active:
        assert not route and active_tok is None
        La, r_act, xa_hat, W_act = res_logits_active(X, W, bias, act, ncomp, eps)
        z[:, N + k * ncomp:] = La.reshape(T, k * k)
    z_pre, z_post, L = split_logits(z, N, k, ncomp)
    if gate_mode == "sigmoid":
        H_pre, H_post = sigmoid(z_pre), sigmoid(z_post)
    else:
        H_pre, H_post = np.ones_like(z_pre), np.ones_like(z_post)
    H_res, _ = sinkhorn(L, iters)
    U_raw = tfa_components(out, B, S, conv_ws)
    U = gram_schmidt(U_raw, gs_eps)[0] if gram_schmidt_on else U_raw

    rt = _route(Xf, act, route, W_route, b_route, eps, route_idx, active_tok)
    idx, s = rt["idx"], rt["s"]
    tok = np.arange(T)[:, None]
    G = dX_new[tok, idx, :]                                       # [T, k, C]
    Xa = X[tok, idx, :]

    # pass-through rows keep their upstream gradient; rewritten rows do not
    dX = dX_new.copy()
    dX[tok, idx, :] = 0.0
    # through the mixing term and the write-back term (scaled by s)
    dH_res = np.einsum("tac,tbc->tab", G, Xa)
    dX[tok, idx, :] += np.einsum("tab,tac->tbc", H_res, G)
    dq = np.einsum("tac,tmc->tam", G, U)            # gradient of s_a H_post[a, m]
    dH_post = s[:, :, None] * dq
    dU = np.einsum("tam,tac->tmc", s[:, :, None] * H_post, G)
    # through the dense read
    dH_pre = np.einsum("tc,tic->ti", dh_in, X)
    dX += H_pre[:, :, None] * dh_in[:, None, :]

    # through the gates and Sinkhorn to the logits
    if gate_mode == "sigmoid":
        dz_pre = dH_pre * H_pre * (1.0 - H_pre)
        dz_post = dH_post * H_post * (1.0 - H_post)
    else:
        dz_pre = np.zeros_like(dH_pre)
        dz_post = np.zeros_like(dH_post)
    dL = sinkhorn_backward(L, iters, dH_res)
    dz = np.concatenate([dz_pre, dz_post.reshape(T, k * ncomp),
                         dL.reshape(T, k * k)], axis=1)

    # through the RMS-normed projection
    db = dz.sum(axis=0)
    dz_full = dz.copy()
    if hres_active:
        dz_full[:, N + k * ncomp:] = 0.0        # the res logits do not read the full state
    dW = xhat.T @ dz_full
    dxhat = dz_full @ W.T
    n = N * C
    dXf = (dxhat - xhat * (np.sum(dxhat * xhat, axis=1, keepdims=True) / n)) / r[:, None]
    dX += dXf.reshape(T, N, C)
    if hres_active:
        # O9: the res logits' RMS-normed projection of the active rows
        res0 = N + k * ncomp
        dLf = dz[:, res0:]
        dWa = xa_hat.T @ dLf                                   # [k*C, k*k]
        dW.reshape(N, C, P)[act, :, res0:] += dWa.reshape(k, C, k * k)
        dxa = dLf @ W_act.T
        dXa = (dxa - xa_hat * (np.sum(dxa * xa_hat, axis=1, keepdims=True) / (k * C))) / r_act[:, None]
        dX[:, act, :] += dXa.reshape(T, k, C)

    # through the router's scales, then its LayerNorm (O7)
    extra = {}
    if route:
        ds = np.sum(H_post * dq, axis=2)                         # [T, k]
        drho = np.zeros((T, N))
        sr = s[:, k - route:]
        drho[tok, idx[:, k - route:]] = ds[:, k - route:] * sr * (1.0 - sr)
        Wr = np.asarray(W_route, dtype=np.float64)
        y, sd = rt["y"], rt["sd"]
        dy = drho @ Wr.T
        dXr = (dy - dy.mean(axis=1, keepdims=True)
               - y * np.mean(dy * y, axis=1, keepdims=True)) / sd[:, None]
        dX += dXr.reshape(T, N, C)
        extra = dict(dW_route=y.T @ drho, db_route=drho.sum(axis=0), drho=drho, idx=idx)

    # through Gram-Schmidt, then temporal feature augmentation
    if gram_schmidt_on:
        dU = gram_schmidt_backward(U_raw, gs_eps, dU)
    dout = dU[:, 0, :].copy()
    out_bsc = out.reshape(B, S, C)
    dconv = []
    for m, w in enumerate(conv_ws):
        d_o, d_w = causal_depthwise_conv_backward(out_bsc, w, dU[:, m + 1, :].reshape(B, S, C))
        dout += d_o.reshape(T, C)
        dconv.append(d_w)
    res = dict(dX=dX, dout=dout, dW=dW, db=db, dconv=dconv, dz=dz)
    res.update(extra)
    return res

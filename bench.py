"""Benchmark of the xHC sublayer forward+backward on one MI355X.

One step = xhc_forward (in place, saving z and the old active rows) followed
by xhc_backward, over one batch of the fwd+bwd workload (B=2, S=4096,
C=4096, N=16 streams, k=4 active, TFA on, bf16 storage, fp32 arithmetic),
with every input resident in HBM before the timed region starts.

Prints one JSON line: tokens/s of the whole step, the roofline of the
dominant kernel (`roofline`, scope "kernel": algorithmic bytes per launch /
its average duration from HIP events on the launch stream), the whole step
against the same peak (`step_hbm`: on the method's bytes, on the bytes the
kernels touch, and on the measured counter bytes of the main kernels) and
the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "tokens/s and achieved HBM GB/s (% of peak), xHC N=16 k=4 sublayer fwd+bwd"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="fwdbwd4096")
    ap.add_argument("--cpu-tokens", type=int, default=8192,
                    help="tokens of the CPU oracle sample (whole sequences, then a causal prefix)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-timer", action="store_true", help="skip the per-kernel event pass")
    ap.add_argument("--no-chain", action="store_true",
                    help="stacked workloads: project every sublayer's state in its own pass instead of "
                         "carrying the projection from the previous sublayer's write pass")
    ap.add_argument("--split", action="store_true",
                    help="fwd+bwd: build the step from the split calls (xhc_forward_pre, xhc_forward_post, "
                         "xhc_backward_post, xhc_backward_pre) instead of xhc_forward and xhc_backward")
    ap.add_argument("--graph", action="store_true",
                    help="fwd+bwd: capture one step in a HIP graph (torch.cuda.CUDAGraph) and time its replays")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 2 GiB device copy (HBM counter calibration) and exit")
    ap.add_argument("--probe", action="store_true",
                    help="only run the hand-written bandwidth probes (libxhc_probe.so: streaming read, copy, "
                         "two reads + one write, and the per-token-row run patterns of the xHC kernels) and exit")
    return ap.parse_args()


def kernel_bytes(w, esz, save_rows=True):
    """Algorithmic HBM bytes per launch of each main kernel: every input and
    output it must touch, once (per token, in units of C elements):
      proj     reads the state                                  16C
      mix      reads state 16C + out C; writes h_in C, 4 rows 4C,
               saved old rows 4C                                26C
      bxdots   reads state 16C (12 rows + 4 saved) + dh_in C + G 4C  21C
      bdots    reads G 4C + out C; writes dout C                 6C
               (with Gram-Schmidt: the dots pass, reads G 4C + out C  5C)
      bgrad    reads state 16C + dX_new 16C + dh_in C; writes dX 16C  49C
      mixproj  reads state 16C + out C; writes h_in C, 4 rows 4C  22C
               (the write pass that also projects the state it writes
               for the next sublayer)
      gram     (Gram-Schmidt) reads out C
      bdots_gs (Gram-Schmidt) reads G 4C + out C; writes dout C  6C
    With the router:
      route_pass reads G 4C; writes the pass rows 4C               8C
      bgrad    reads state 16C + dX_new 12C + pass rows 4C + dh_in C;
               writes dX 16C                                    49C
    plus the projection weights (N*C x P, and N*C x N for the router) where
    a kernel reads them."""
    T, C, N, k, P = w.T, w.C, w.N, w.k, w.P
    unit = T * C * esz
    rt = getattr(w, "route", 0)
    wbytes = N * C * P * esz + (N * C * N * esz if rt else 0)
    gs = getattr(w, "gs", False)
    kb = {
        "proj": N * unit + wbytes,
        "mix": (N + 1 + 1 + k + (k if save_rows else 0)) * unit,
        "bxdots": (N + 1 + k) * unit,
        "bdots": (k + 1 + (0 if gs else 1)) * unit,
        "bgrad": (N + N + 1 + N) * unit + wbytes,
        "mixproj": (N + 1 + 1 + k) * unit + wbytes,
    }
    if gs:
        kb["gram"] = unit
        kb["bdots_gs"] = (k + 1 + 1) * unit
    if rt:
        kb["route_pass"] = 2 * k * unit
        del kb["mixproj"]
    return kb


# the source file that holds each kernel (the shared headers count for all)
KERNEL_SOURCE = {"proj": "xhc_fwd.hip", "mix": "xhc_fwd.hip", "bxdots": "xhc_bwd.hip", "bdots": "xhc_bwd.hip",
                 "bgrad": "xhc_bwd.hip", "mixproj": "xhc_chain.hip", "gram": "xhc_bwd.hip",
                 "bdots_gs": "xhc_bwd.hip", "route_pass": "xhc_route.hip"}


def source_digest(kernel=None):
    """sha256 (first 16 hex digits) of the sources a kernel is built from:
    the shared headers and the kernel's own file (every source when kernel
    is None)."""
    csrc = os.path.join(ROOT, "residual_stream_architecture_amd", "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "*")))
    if kernel is not None:
        files = [f for f in files if f.endswith(".h") or os.path.basename(f) == KERNEL_SOURCE[kernel]]
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"```json\n(.*?)\n```", txt, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_digest") != source_digest(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_probe(torch):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.int16, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    t = time.perf_counter()
    reps = 10
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t) / reps
    print(json.dumps({"copy_probe_bytes": 2 * n * 2, "ms": dt * 1e3, "GBps": 4 * n / dt / 1e9}), flush=True)


PROBE_RUNS = (128, 256, 512, 1024)


def bandwidth_probes(torch):
    """Bandwidth of plain access patterns on this GPU, timed with events on
    the launch stream (median of 10 launches after 3 warm-ups):
      stream_*   contiguous streaming, every workgroup its own slice
      rows_*     per-token rows of 128 KiB (the state of one token at
                 N = 16, C = 4096, bf16) over 8192 tokens; each workgroup owns
                 `run` bytes of every row of its token split -- 2r1w is the
                 backward assembly kernel's mix (state and dX_new read, dX
                 written), 1r the projection's and the backward dots' reads.
      frag_*     the same state as 16 rows of 8 KiB per token; each
                 workgroup owns 1 KiB of every row of a 64-token tile, each
                 wave 128 bytes, two 16-byte loads per lane and token: laid
                 out as MFMA A fragments (one instruction covers 16 rows x 64
                 bytes, half of each line) or as whole lines (8 rows x 128
                 bytes per instruction).
    Bytes are the bytes each probe must move (reads + writes)."""
    import ctypes
    from residual_stream_architecture_amd import build as b
    if not os.path.exists(b.PROBE_LIB):
        raise SystemExit(f"{b.PROBE_LIB} is missing: build first")
    L = ctypes.CDLL(b.PROBE_LIB)
    vp = ctypes.c_void_p
    L.xhc_probe_stream.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    L.xhc_probe_rows.argtypes = [vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, vp, vp]
    L.xhc_probe_frag.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    T, row = 8192, 16 * 4096 * 2
    nbytes = T * row                                   # 1 GiB per buffer
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(3)]
    for i, t in enumerate(bufs):
        t.fill_(i + 1)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    a, bb, d = (t.data_ptr() for t in bufs)

    def timed(fn, moved):
        for _ in range(3):
            rc = fn()
            if rc:
                raise RuntimeError(f"probe launch failed ({rc})")
        times = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            fn()
            e1.record(st)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        times.sort()
        med = times[len(times) // 2]
        return {"bytes": moved, "us": round(med * 1e6, 1), "GBps": round(moved / med / 1e9, 1),
                "frac_of_peak": round(moved / med / 1e9 / HBM_PEAK_GBPS, 4)}

    res = {}
    for nr, nw, name in ((1, 0, "1r"), (1, 1, "1r1w"), (2, 1, "2r1w")):
        for blocks in (1024, 4096):
            res[f"stream_{name}_wg{blocks}"] = timed(
                lambda: L.xhc_probe_stream(a, bb, d, nbytes, nr, nw, blocks, sink.data_ptr(), st.cuda_stream),
                (nr + nw) * nbytes)
    for nr, nw, name in ((1, 0, "1r"), (2, 1, "2r1w")):
        for run in PROBE_RUNS:
            splits = max(1, 2048 // (row // run))
            res[f"rows_{name}_run{run}"] = timed(
                lambda: L.xhc_probe_rows(a, bb, d, T, row, run, nr, nw, splits, sink.data_ptr(), st.cuda_stream),
                (nr + nw) * nbytes)
            res[f"rows_{name}_run{run}"]["grid"] = (row // run) * splits
    for mode, name in ((0, "frag_1r_mfma_layout"), (1, "frag_1r_whole_lines")):
        res[name] = timed(lambda: L.xhc_probe_frag(a, T, 16, row // 16, mode, sink.data_ptr(), st.cuda_stream),
                          nbytes)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "hbm bandwidth of plain access patterns", "peak_GBps": HBM_PEAK_GBPS,
                      "results": res}), flush=True)


def cpu_baseline(w, ntok):
    """The oracle, as it stands, on `ntok` tokens of the workload: whole
    sequences of it in turn (B=1 each, S=w.S), then a causally closed prefix
    of the next one when ntok is not a multiple of S."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import xhc_oracle as xo
    from residual_stream_architecture_amd import synth
    active = synth.active_streams(0, w.N, w.k)
    dt = 0.0
    left = ntok
    seq = 0
    while left > 0:
        S = min(left, w.S)
        sw = synth.Workload("cpu-sample", 1, S, w.C, w.N, w.k, w.ncomp, w.dtype, "fwdbwd")
        d = synth.make_inputs(sw, seed=seq, grads=True)
        rkw = {}
        if w.route:
            d.update(synth.make_router(sw, seq))
        h = {k: synth.as_float(d, k) for k in d}
        del d
        if w.route:
            rkw = dict(route=w.route, W_route=h["W_route"], b_route=h["b_route"])
        convs = (h["w4"], h["w8"], h["w12"])
        t = time.perf_counter()
        xo.forward(h["X"], h["out"], h["W"], h["bias"], active, convs, B=1, S=S, iters=w.iters, eps=w.eps,
                   gram_schmidt_on=w.gs, **rkw)
        xo.backward(h["X"], h["out"], h["W"], h["bias"], active, convs, h["dX_new"], h["dh_in"], B=1, S=S,
                    iters=w.iters, eps=w.eps, gram_schmidt_on=w.gs, **rkw)
        dt += time.perf_counter() - t
        del h
        left -= S
        seq += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(ntok / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"numpy fp64 oracle forward+backward over {ntok} tokens ({seq} sequence(s) of at most "
                      f"{w.S}) of the same workload (C={w.C}, N={w.N}, k={w.k}, TFA on"
                      f"{', Gram-Schmidt on' if w.gs else ''}{', router' if w.route else ''}): "
                      f"{dt:.1f} s of compute; "
                      f"BLAS threads={threads}, host cpus={os.cpu_count()}"}


def forward_bench(args, w, np, torch, synth, xhc):
    """Forward-only workloads (extra measurements; the default line is the
    fwd+bwd one).  One step = one in-place forward of every layer of the
    workload (48 for the stacked one, each with its own parameters and its
    rotating active set).  The state comes from the seeded generator; the
    per-layer parameters of the stack are drawn on the device from torch's
    generator seeded 1000 + layer (same shapes and distributions; the run
    time does not depend on the values).  A stack is chained by default:
    every sublayer but the last also projects the state it writes for the
    next one (xhc_forward_chain), so only the first sublayer reads its state
    twice."""
    T, N, C, P, k = w.T, w.N, w.C, w.P, w.k
    esz = 2 if w.dtype == "bf16" else 4
    sdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    chain = w.layers > 1 and not args.no_chain
    print(f"# workload {w} chain={chain}", file=sys.stderr, flush=True)
    d = synth.make_inputs(w, seed=0, state=True)
    X = torch.from_numpy(d.pop("X").view(np.int16)).cuda().view(torch.bfloat16) if esz == 2 else \
        torch.from_numpy(d.pop("X")).cuda()
    code = xhc.XHC_BF16 if esz == 2 else xhc.XHC_F32
    layers = []
    for l in range(w.layers):
        nc = synth.layer_ncomp(w, l)
        Pl = N + k * nc + k * k
        if w.layers == 1:
            p = {key: (torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16) if a.dtype == np.uint16
                       else torch.from_numpy(a).cuda()) for key, a in d.items()}
        else:
            g = torch.Generator(device="cuda")
            g.manual_seed(synth.stack_layer_seed(l))
            p = {"out": torch.randn(T, C, generator=g, device="cuda").to(sdt)}
            if nc == 4:
                p.update(w4=torch.randn(C, 4, generator=g, device="cuda") * 0.02,
                         w8=torch.randn(C, 8, generator=g, device="cuda") * 0.02,
                         w12=torch.randn(C, 12, generator=g, device="cuda") * 0.02)
            p.update(W=(torch.randn(N * C, Pl, generator=g, device="cuda") * 0.02).to(sdt),
                     bias=torch.zeros(Pl, device="cuda"))
        if w.route and w.layers > 1:
            # the router's weights of the sublayer (its fixed streams: the
            # first k - R of its rotating set)
            p.update(W_route=(torch.randn(N * C, N, generator=g, device="cuda") * 0.02).to(sdt),
                     b_route=torch.zeros(N, device="cuda"),
                     route_idx=torch.empty(T, k, dtype=torch.int32, device="cuda"))
        desc = xhc.make_desc(w.B, w.S, C, N, k, nc, code, w.iters, w.eps, gram_schmidt=w.gs, route=w.route)
        layers.append((p, synth.active_streams(l, N, k), desc, nc))
    del d
    h_in = torch.empty(T, C, dtype=sdt, device="cuda")
    ws_f = torch.empty(max(xhc.workspace_size(L[2], 0) for L in layers), dtype=torch.uint8, device="cuda")
    carries = ([torch.empty(max(xhc.carry_size(L[2]) for L in layers) // 4, device="cuda") for _ in range(2)]
               if chain else None)

    def step(timer=None):
        for l, (p, active, desc, nc) in enumerate(layers):
            conv = dict(w4=p["w4"], w8=p["w8"], w12=p["w12"]) if nc == 4 else {}
            extra = {}
            if chain:
                last = l + 1 == len(layers)
                extra = dict(carry_in=carries[l % 2] if l > 0 else None,
                             W_next=None if last else layers[l + 1][0]["W"],
                             carry_out=None if last else carries[(l + 1) % 2],
                             desc_next=None if last else layers[l + 1][2])
                if w.route and not last:
                    extra.update(W_route_next=layers[l + 1][0]["W_route"], active_next=layers[l + 1][1])
            if w.route:
                extra.update(W_route=p["W_route"], b_route=p["b_route"], route_idx=p["route_idx"])
            xhc.forward(X, p["out"], p["W"], active, X, h_in, B=w.B, S=w.S, bias=p["bias"], workspace=ws_f,
                        timer=timer, desc=desc, **conv, **extra)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    kernels = {}
    timer = xhc.Timer()
    for _ in range(max(1, min(args.steps, 5))):
        step(timer)
    torch.cuda.synchronize()
    kb = kernel_bytes(w, esz, save_rows=False)
    if w.route:
        # the stack's fused pass moves the same 22C per token with the router
        # (a token's routed rows are read twice, the second time from L2)
        kb["mixproj"] = (N + 1 + 1 + k) * T * C * esz + N * C * (P + N) * esz
    for name in xhc.kernel_names():
        ms, n = timer.read(name)
        if n:
            kernels[name] = {"avg_us": round(ms * 1e3 / n, 2), "launches": n}
            if name in ("proj", "mix", "mixproj"):
                kernels[name]["alg_GBps"] = round(kb[name] / (ms * 1e-3 / n) / 1e9, 1)
    # per token and step, in units of C: every sublayer reads its state, out
    # and writes h_in and k rows (22C at N = 16); without the chain every
    # sublayer also reads its state for the projection, with it only the first
    alg_c = (N + 1 + 1 + k) * w.layers
    touched_c = alg_c + N * (1 if chain else w.layers)
    result = {"metric": f"tokens/s, xHC sublayer forward ({w.name})", "value": round(T * args.steps / elapsed, 1),
              "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
              "config": {"workload": f"{w.name}: B={w.B} S={w.S} C={C} N={N} k={k} ncomp={w.ncomp} "
                                     f"layers={w.layers}"
                                     + (" (even sublayers attention-side: ncomp=1)" if w.alt else "")
                                     + (f" router: {k - w.route} fixed + {w.route} routed streams per token"
                                        if w.route else "")
                                     + ", in-place forward"
                                     + (", chained projection" if chain else "")},
              "layer_tokens_per_s": round(T * w.layers * args.steps / elapsed, 1),
              "step_hbm": {"alg_bytes_per_token_in_C": alg_c, "touched_bytes_per_token_in_C": touched_c,
                           "alg_GBps": round(alg_c * T * C * esz / (ms_per_step * 1e-3) / 1e9, 1)},
              "kernels": kernels}
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no multi-GPU path.",
              file=sys.stderr, flush=True)
        sys.exit(2)
    import numpy as np
    import torch
    from residual_stream_architecture_amd import synth
    from residual_stream_architecture_amd import xhc

    if args.copy_probe:
        copy_probe(torch)
        return
    if args.probe:
        bandwidth_probes(torch)
        return

    w = synth.WORKLOADS[args.workload]
    if w.phase != "fwdbwd":
        forward_bench(args, w, np, torch, synth, xhc)
        return
    T, N, C, P, k = w.T, w.N, w.C, w.P, w.k
    esz = 2 if w.dtype == "bf16" else 4
    print(f"# workload {w}", file=sys.stderr, flush=True)

    d = synth.make_inputs(w, seed=0, grads=True)
    rt = w.route
    if rt:
        d.update(synth.make_router(w, 0))

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    X = dev(d.pop("X"))
    dXn = dev(d.pop("dX_new"))
    dhin = dev(d.pop("dh_in"))
    out = dev(d["out"])
    W = dev(d["W"])
    bias = dev(d["bias"])
    convs = dict(w4=dev(d["w4"]), w8=dev(d["w8"]), w12=dev(d["w12"]))
    route_in = dict(W_route=dev(d["W_route"]), b_route=dev(d["b_route"])) if rt else {}
    del d
    sdt = X.dtype
    h_in = torch.empty(T, C, dtype=sdt, device="cuda")
    xact = torch.empty(T, k, C, dtype=sdt, device="cuda")
    dX = torch.empty_like(dXn)
    dout = torch.empty(T, C, dtype=sdt, device="cuda")
    dW = torch.empty(N * C, P, device="cuda")
    db = torch.empty(P, device="cuda")
    dws = dict(dw4=torch.empty(C, 4, device="cuda"), dw8=torch.empty(C, 8, device="cuda"),
               dw12=torch.empty(C, 12, device="cuda"))
    desc = xhc.make_desc(w.B, w.S, C, N, k, w.ncomp, xhc.XHC_BF16 if w.dtype == "bf16" else xhc.XHC_F32,
                         w.iters, w.eps, gram_schmidt=w.gs, route=rt)
    z_save = torch.empty(T, xhc.zsave_stride(desc), device="cuda")
    ws_f = torch.empty(xhc.workspace_size(desc, 0), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(xhc.workspace_size(desc, 1), dtype=torch.uint8, device="cuda")
    active = synth.active_streams(0, N, k)
    fwd_kw = dict(xact_save=xact)
    bwd_kw = dict(xact=xact)
    if rt:
        ridx = torch.empty(T, k, dtype=torch.int32, device="cuda")
        fwd_kw.update(route_idx=ridx, **route_in)
        bwd_kw.update(W_route=route_in["W_route"], route_idx=ridx,
                      dW_route=torch.empty(N * C, N, device="cuda"), db_route=torch.empty(N, device="cuda"))

    def step(timer=None):
        xhc.forward(X, out, W, active, X, h_in, B=w.B, S=w.S, bias=bias, z_save=z_save,
                    workspace=ws_f, timer=timer, desc=desc, **convs, **fwd_kw)
        xhc.backward(X, out, W, active, dXn, dhin, dX, dout, dW, B=w.B, S=w.S, bias=bias,
                     z_save=z_save, db=db, workspace=ws_b, timer=timer, desc=desc, **convs, **dws, **bwd_kw)

    if args.split:
        # the same step from the split calls: the sublayer's output and dh_in
        # stand ready (synthetic), so the calls run back to back
        if w.gs:
            raise SystemExit("--split: not with Gram-Schmidt (the split backward refuses it)")
        bwd_state = torch.empty(xhc.bwd_state_size(desc) // 4, dtype=torch.float32, device="cuda")
        pre_kw = dict(route_idx=ridx, **route_in) if rt else {}
        lists_kw = dict(route_idx=ridx) if rt else {}
        bpre_kw = {key: bwd_kw[key] for key in ("W_route", "route_idx", "dW_route", "db_route")} if rt else {}

        def step(timer=None):
            xhc.forward_pre(X, W, active, h_in, z_save, desc=desc, bias=bias, workspace=ws_f, timer=timer,
                            **pre_kw)
            xhc.forward_post(X, out, active, z_save, desc=desc, xact_save=xact, workspace=ws_f, timer=timer,
                             **convs, **lists_kw)
            xhc.backward_post(out, active, z_save, dXn, dout, bwd_state, desc=desc, workspace=ws_b, timer=timer,
                              **convs, **dws, **lists_kw)
            xhc.backward_pre(X, W, active, z_save, dXn, dhin, bwd_state, dX, dW, desc=desc, xact=xact, bias=bias,
                             db=db, workspace=ws_b, timer=timer, **bpre_kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if args.graph:
        # the library launches only kernels on the current stream, so one
        # step captures whole; replays redo the same work on the same buffers
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T * args.steps / elapsed
    print(f"# timed {args.steps} steps{' (graph replays)' if args.graph else ''}: {ms_per_step:.3f} ms/step",
          file=sys.stderr, flush=True)

    # per-kernel durations from HIP events recorded on the launch stream
    kernels = {}
    roofline = None
    if not args.no_timer:
        timer = xhc.Timer()
        for _ in range(args.steps):
            step(timer)
        torch.cuda.synchronize()
        kb = kernel_bytes(w, esz)
        if args.split:
            kb.pop("mixproj", None)      # the pre and post passes move different bytes under one name
            if rt:
                kb.pop("mix", None)      # the routed post pass moves each token's rows only, not 26C
        for name in xhc.kernel_names():
            ms, n = timer.read(name)
            if n:
                kernels[name] = {"avg_us": round(ms * 1e3 / n, 2), "launches": n}
        for name, byts in kb.items():
            if name in kernels:
                avg_s = kernels[name]["avg_us"] * 1e-6
                kernels[name]["alg_bytes"] = byts
                kernels[name]["alg_GBps"] = round(byts / avg_s / 1e9, 1)
        dom = max(kb, key=lambda n: kernels.get(n, {}).get("avg_us", 0.0))
        achieved = kernels[dom]["alg_GBps"]
        roofline = {"bound": "hbm", "scope": "kernel", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": measured_traffic(dom, w.name)}

    # whole-step accounting in units of C per token (bf16)
    alg_step_c = (N + 1 + 1 + k) + (N + N + 1 + 1 + N + 1)        # 22C forward + 51C backward
    impl_step_c = 16 + 26 + 21 + 6 + 49                             # what the kernels above touch
    if w.gs:
        impl_step_c += 1 + 5                                        # gram pass, the dots pass of B1
    if rt:
        impl_step_c += 8                                            # the pass rows (written, read)
    step_bytes = alg_step_c * T * C * esz
    step_s = ms_per_step * 1e-3
    step_hbm = {"alg_bytes_per_token_in_C": alg_step_c, "touched_bytes_per_token_in_C": impl_step_c,
                "alg_GBps": round(step_bytes / step_s / 1e9, 1),
                "alg_frac_of_peak": round(step_bytes / step_s / 1e9 / HBM_PEAK_GBPS, 4),
                "touched_frac_of_peak": round(impl_step_c * T * C * esz / step_s / 1e9 / HBM_PEAK_GBPS, 4)}
    # the step on measured counter bytes: the main kernels' calibrated
    # FETCH+WRITE bytes (committed rocprofv3 summaries on the current
    # sources) per step, over the whole step's time; the small kernels
    # (coefficients, reductions, weight packing) have no summary and count 0
    if kernels:
        meas = {}
        for name in kernel_bytes(w, esz):
            t = measured_traffic(name, w.name)
            if t is not None and name in kernels:
                meas[name] = t * kernels[name]["launches"] / args.steps
        if meas:
            mb = sum(meas.values())
            step_hbm.update(measured_bytes_per_step=int(mb), measured_kernels=sorted(meas),
                            measured_frac_of_peak=round(mb / step_s / 1e9 / HBM_PEAK_GBPS, 4))
    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"xHC sublayer fwd+bwd ({w.name}): B={w.B} S={w.S} C={C} N={N} k={k} "
                               f"TFA K=4/8/12{', Gram-Schmidt' if w.gs else ''}, 20 Sinkhorn iters, "
                               + (f"router: {k - rt} fixed + {rt} routed streams per token, " if rt else "")
                               + ("split calls (forward pre, post; backward post, pre)" if args.split
                                  else "in-place forward + backward"),
                   "global_batch": w.B, "seq_len": w.S},
        "step_hbm": step_hbm,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

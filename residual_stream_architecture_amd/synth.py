"""Seeded synthetic inputs for the xHC sublayer (shared by tests and bench).

This module holds no arithmetic of the method: it only draws random numbers,
rounds them to the storage type and names the workloads.  Both the oracle
checks and the GPU runs take their inputs from here.

Draw order for one call of `make_inputs` (numpy default_rng(seed),
standard_normal in float32):
    X [T,N,C] * 1, out [T,C] * 1, w4 [C,4] * 0.02, w8 [C,8] * 0.02,
    w12 [C,12] * 0.02 (only when ncomp == 4), W [N*C,P] * 0.02,
    then, if grads=True, dX_new [T,N,C] * 1 and dh_in [T,C] * 1.
In bf16 workloads X, out, W, dX_new and dh_in are rounded to bf16
(round-to-nearest-even); the conv weights stay fp32; the bias is zero.
A router's weights come from `make_router` (its own generator, seed + 7000):
W_route [N*C,N] * 0.02, bf16-rounded in bf16 workloads; b_route is zero.
"""

from dataclasses import dataclass
import numpy as np

_CHUNK = 1 << 24          # values drawn per call, to bound host memory


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    C: int
    N: int
    k: int
    ncomp: int
    dtype: str            # "f32" or "bf16"
    phase: str            # "fwd", "fwdbwd" or "stack"
    layers: int = 1
    iters: int = 20
    eps: float = 1e-6
    gs: bool = False      # Gram-Schmidt over the write-back components
    alt: bool = False     # stack: even sublayers attention-side (one component, no TFA)
    route: int = 0        # routed slots (the first k - route active streams are fixed)

    @property
    def T(self):
        return self.B * self.S

    @property
    def P(self):
        return self.N + self.k * self.ncomp + self.k * self.k


WORKLOADS = {
    # tiny fp32 sublayer forward, streams 0-3 active
    "tiny": Workload("tiny", 1, 64, 64, 16, 4, 4, "f32", "fwd"),
    # bf16 sublayer forward, active set rotating with the layer id
    "fwd2048": Workload("fwd2048", 4, 2048, 2048, 16, 4, 4, "bf16", "fwd"),
    # mHC-style dense update: N = k = 4, one write-back component
    "mhc4": Workload("mhc4", 4, 4096, 4096, 4, 4, 1, "bf16", "fwd"),
    # bf16 sublayer forward + backward (the headline workload)
    "fwdbwd4096": Workload("fwdbwd4096", 2, 4096, 4096, 16, 4, 4, "bf16", "fwdbwd"),
    # the same with Gram-Schmidt over the four write-back components
    "fwdbwd4096_gs": Workload("fwdbwd4096_gs", 2, 4096, 4096, 16, 4, 4, "bf16", "fwdbwd", gs=True),
    # the same with the router: streams 0 and 1 fixed, two chosen per token
    "fwdbwd4096_route": Workload("fwdbwd4096_route", 2, 4096, 4096, 16, 4, 4, "bf16", "fwdbwd", route=2),
    # 48 stacked sublayer updates, state carried in HBM
    "stack48": Workload("stack48", 1, 8192, 7168, 16, 4, 4, "bf16", "stack", layers=48),
    # the same stack alternating attention-side sublayers (out only) with
    # MLP-side ones (TFA), as the pages place TFA after the MLP/MoE only
    "stack48_alt": Workload("stack48_alt", 1, 8192, 7168, 16, 4, 4, "bf16", "stack", layers=48, alt=True),
    # the same stack with the router in every sublayer: the first two streams
    # of the rotating set fixed, two chosen per token
    "stack48_route": Workload("stack48_route", 1, 8192, 7168, 16, 4, 4, "bf16", "stack", layers=48, route=2),
}


def layer_ncomp(w, layer):
    """Write-back components of sublayer `layer` of a stack."""
    return 1 if (w.alt and layer % 2 == 0) else w.ncomp


def active_streams(layer, N, k):
    """Rotating active set of layer `layer`: ((k*layer + j) mod N), j < k."""
    return [int((k * layer + j) % N) for j in range(k)]


def bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round-to-nearest-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_to_f32(bits):
    """uint16 bf16 bit patterns -> the exact float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw(rng, shape, scale, as_bf16):
    """Draw standard normals in chunks; returns float32 or uint16 bf16 bits."""
    n = int(np.prod(shape))
    dst = np.empty(n, dtype=np.uint16 if as_bf16 else np.float32)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        v = rng.standard_normal(m, dtype=np.float32)
        if scale != 1.0:
            v *= np.float32(scale)
        dst[s:s + m] = bf16_bits(v) if as_bf16 else v
    return dst.reshape(shape)


def make_inputs(w: Workload, seed=0, grads=False, state=True):
    """Draw one sublayer's inputs.  bf16 tensors come back as uint16 bits.

    state=False skips X (used for the per-layer draws of the stacked
    workload, whose state is carried from layer to layer).
    """
    rng = np.random.default_rng(seed)
    lowp = w.dtype == "bf16"
    T, N, C = w.T, w.N, w.C
    d = {}
    if state:
        d["X"] = _draw(rng, (T, N, C), 1.0, lowp)
    d["out"] = _draw(rng, (T, C), 1.0, lowp)
    if w.ncomp == 4:
        d["w4"] = _draw(rng, (C, 4), 0.02, False)
        d["w8"] = _draw(rng, (C, 8), 0.02, False)
        d["w12"] = _draw(rng, (C, 12), 0.02, False)
    d["W"] = _draw(rng, (N * C, w.P), 0.02, lowp)
    d["bias"] = np.zeros(w.P, dtype=np.float32)
    if grads:
        d["dX_new"] = _draw(rng, (T, N, C), 1.0, lowp)
        d["dh_in"] = _draw(rng, (T, C), 1.0, lowp)
    return d


def make_router(w: Workload, seed=0):
    """The router's weights: W_route [N*C, N] and a zero b_route."""
    rng = np.random.default_rng(seed + 7000)
    return dict(W_route=_draw(rng, (w.N * w.C, w.N), 0.02, w.dtype == "bf16"),
                b_route=np.zeros(w.N, dtype=np.float32))


def as_float(d, key):
    """Exact float32 view of an input (decodes bf16 bits)."""
    a = d[key]
    return bf16_to_f32(a) if a.dtype == np.uint16 else a


def stack_layer_seed(layer):
    """Per-layer seed of the stacked workload's out, conv and W draws."""
    return 1000 + layer

"""ctypes binding of libxhc (include/xhc.h), same names as the C ABI.

Argument marshalling only: torch tensors provide device pointers and the
current HIP stream; every step of the update runs in the library's kernels.
Importing this module fails loudly when libxhc.so has not been built.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# XHC_LIBRARY names another build of the same library (a sanitised host build
# for the ABI tests, say); by default the in-tree one.
LIB_PATH = os.environ.get("XHC_LIBRARY") or os.path.join(_PKG, "libxhc.so")

XHC_F32, XHC_BF16 = 0, 1
XHC_GATE_SIGMOID, XHC_GATE_UNIT = 0, 1
XHC_PHASE_FWD, XHC_PHASE_BWD, XHC_PHASE_PRE, XHC_PHASE_POST = 0, 1, 2, 3
XHC_PHASE_BWD_POST, XHC_PHASE_BWD_PRE = 4, 5
XHC_STATUS_ID_RANGE, XHC_STATUS_ID_REPEAT = 1, 2
ERRORS = {0: "XHC_OK", -1: "XHC_ERR_NULL", -2: "XHC_ERR_SHAPE", -3: "XHC_ERR_INDEX",
          -4: "XHC_ERR_ALIAS", -5: "XHC_ERR_ALIGN", -6: "XHC_ERR_UNSUPPORTED",
          -7: "XHC_ERR_WORKSPACE", -8: "XHC_ERR_HIP", -9: "XHC_ERR_SCRATCH"}
(XHC_OK, XHC_ERR_NULL, XHC_ERR_SHAPE, XHC_ERR_INDEX, XHC_ERR_ALIAS, XHC_ERR_ALIGN, XHC_ERR_UNSUPPORTED,
 XHC_ERR_WORKSPACE, XHC_ERR_HIP, XHC_ERR_SCRATCH) = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
NOALLOC_SCRATCH_BYTES = 64 << 20      # XHC_NOALLOC_SCRATCH_BYTES

_vp = ctypes.c_void_p
_fp = ctypes.POINTER(ctypes.c_float)


class xhc_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("S", ctypes.c_int32), ("C", ctypes.c_int32),
                ("N", ctypes.c_int32), ("k", ctypes.c_int32), ("ncomp", ctypes.c_int32),
                ("sinkhorn_iters", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
                ("gram_schmidt", ctypes.c_int32), ("gs_eps", ctypes.c_float),
                ("route", ctypes.c_int32), ("per_token_active", ctypes.c_int32),
                ("hres_active", ctypes.c_int32)]


class xhc_fwd_args(ctypes.Structure):
    _fields_ = [("X", _vp), ("out", _vp), ("w4", _vp), ("w8", _vp), ("w12", _vp),
                ("W", _vp), ("bias", _vp), ("active", ctypes.POINTER(ctypes.c_int32)),
                ("X_new", _vp), ("h_in", _vp), ("z_save", _vp), ("xact_save", _vp),
                ("timer", _vp), ("W_route", _vp), ("b_route", _vp), ("route_idx", _vp), ("status", _vp)]


class xhc_bwd_args(ctypes.Structure):
    _fields_ = [("X", _vp), ("xact", _vp), ("out", _vp), ("w4", _vp), ("w8", _vp), ("w12", _vp),
                ("W", _vp), ("bias", _vp), ("active", ctypes.POINTER(ctypes.c_int32)),
                ("z_save", _vp), ("dX_new", _vp), ("dh_in", _vp), ("dX", _vp), ("dout", _vp),
                ("dW", _vp), ("db", _vp), ("dw4", _vp), ("dw8", _vp), ("dw12", _vp),
                ("accumulate", ctypes.c_int32), ("timer", _vp),
                ("W_route", _vp), ("route_idx", _vp), ("dW_route", _vp), ("db_route", _vp),
                ("b_route", _vp), ("status", _vp)]


class xhc_chain_args(ctypes.Structure):
    _fields_ = [("carry_in", _vp), ("W_next", _vp), ("carry_out", _vp),
                ("desc_next", ctypes.POINTER(xhc_desc)), ("W_route_next", _vp),
                ("active_next", ctypes.POINTER(ctypes.c_int32))]


class xhc_pre_args(ctypes.Structure):
    _fields_ = [("X", _vp), ("W", _vp), ("bias", _vp), ("active", ctypes.POINTER(ctypes.c_int32)),
                ("h_in", _vp), ("z_save", _vp), ("carry_in", _vp), ("W_next", _vp), ("carry_out", _vp),
                ("desc_next", ctypes.POINTER(xhc_desc)), ("timer", _vp),
                ("W_route", _vp), ("b_route", _vp), ("route_idx", _vp), ("status", _vp)]


class xhc_post_args(ctypes.Structure):
    _fields_ = [("X", _vp), ("out", _vp), ("w4", _vp), ("w8", _vp), ("w12", _vp),
                ("active", ctypes.POINTER(ctypes.c_int32)), ("z_save", _vp), ("xact_save", _vp),
                ("W_next", _vp), ("carry_out", _vp), ("desc_next", ctypes.POINTER(xhc_desc)), ("timer", _vp),
                ("route_idx", _vp)]


class xhc_bwd_post_args(ctypes.Structure):
    _fields_ = [("out", _vp), ("w4", _vp), ("w8", _vp), ("w12", _vp), ("active", ctypes.POINTER(ctypes.c_int32)),
                ("z_save", _vp), ("dX_new", _vp), ("dout", _vp), ("dw4", _vp), ("dw8", _vp), ("dw12", _vp),
                ("bwd_state", _vp), ("accumulate", ctypes.c_int32), ("timer", _vp),
                ("route_idx", _vp), ("status", _vp)]


class xhc_bwd_pre_args(ctypes.Structure):
    _fields_ = [("X", _vp), ("xact", _vp), ("W", _vp), ("bias", _vp), ("active", ctypes.POINTER(ctypes.c_int32)),
                ("z_save", _vp), ("dX_new", _vp), ("dh_in", _vp), ("bwd_state", _vp), ("dX", _vp), ("dW", _vp),
                ("db", _vp), ("accumulate", ctypes.c_int32), ("timer", _vp),
                ("W_route", _vp), ("route_idx", _vp), ("dW_route", _vp), ("db_route", _vp)]


class XhcError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({lib.xhc_strerror(code).decode()})")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m residual_stream_architecture_amd.build`")
    # torch's HIP runtime must be in the process before the library: torch
    # ships its own libamdhip64 and asks for it under another name, so when
    # the library comes first and binds the system runtime, torch loads a
    # second one, and the library's launches then run in a runtime that does
    # not own torch's streams and memory.  Loaded after torch, the library's
    # libamdhip64.so.7 resolves to the one already there.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    L.xhc_workspace_size.argtypes = [ctypes.POINTER(xhc_desc), ctypes.c_int]
    L.xhc_workspace_size.restype = ctypes.c_size_t
    L.xhc_validate.argtypes = [ctypes.POINTER(xhc_desc), _vp, ctypes.c_int]
    L.xhc_validate.restype = ctypes.c_int
    L.xhc_forward.argtypes = [ctypes.POINTER(xhc_desc), ctypes.POINTER(xhc_fwd_args), _vp, ctypes.c_size_t, _vp]
    L.xhc_forward.restype = ctypes.c_int
    L.xhc_forward_noalloc.argtypes = [ctypes.POINTER(xhc_desc), ctypes.POINTER(xhc_fwd_args), _vp]
    L.xhc_forward_noalloc.restype = ctypes.c_int
    L.xhc_carry_size.argtypes = [ctypes.POINTER(xhc_desc)]
    L.xhc_carry_size.restype = ctypes.c_size_t
    L.xhc_forward_chain.argtypes = [ctypes.POINTER(xhc_desc), ctypes.POINTER(xhc_fwd_args),
                                    ctypes.POINTER(xhc_chain_args), _vp, ctypes.c_size_t, _vp]
    L.xhc_forward_chain.restype = ctypes.c_int
    L.xhc_forward_pre.argtypes = [ctypes.POINTER(xhc_desc), ctypes.POINTER(xhc_pre_args), _vp, ctypes.c_size_t,
                                  _vp]
    L.xhc_forward_pre.restype = ctypes.c_int
    L.xhc_forward_post.argtypes = [ctypes.POINTER(xhc_desc), ctypes.POINTER(xhc_post_args), _vp, ctypes.c_size_t,
                                   _vp]
    L.xhc_forward_post.restype = ctypes.c_int
    L.xhc_backward.argtypes = [ctypes.POINTER(xhc_desc), ctypes.POINTER(xhc_bwd_args), _vp, ctypes.c_size_t, _vp]
    L.xhc_backward.restype = ctypes.c_int
    L.xhc_bwd_state_size.argtypes = [ctypes.POINTER(xhc_desc)]
    L.xhc_bwd_state_size.restype = ctypes.c_size_t
    L.xhc_backward_post.argtypes = [ctypes.POINTER(xhc_desc), ctypes.POINTER(xhc_bwd_post_args), _vp,
                                    ctypes.c_size_t, _vp]
    L.xhc_backward_post.restype = ctypes.c_int
    L.xhc_backward_pre.argtypes = [ctypes.POINTER(xhc_desc), ctypes.POINTER(xhc_bwd_pre_args), _vp,
                                   ctypes.c_size_t, _vp]
    L.xhc_backward_pre.restype = ctypes.c_int
    L.xhc_strerror.argtypes = [ctypes.c_int]
    L.xhc_strerror.restype = ctypes.c_char_p
    L.xhc_timer_create.argtypes = []
    L.xhc_timer_create.restype = _vp
    L.xhc_timer_destroy.argtypes = [_vp]
    L.xhc_timer_destroy.restype = None
    L.xhc_timer_reset.argtypes = [_vp]
    L.xhc_timer_reset.restype = None
    L.xhc_timer_read.argtypes = [_vp, ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_int64)]
    L.xhc_timer_read.restype = ctypes.c_int
    L.xhc_kernel_count.argtypes = []
    L.xhc_kernel_count.restype = ctypes.c_int
    L.xhc_zsave_stride.argtypes = [ctypes.POINTER(xhc_desc)]
    L.xhc_zsave_stride.restype = ctypes.c_int32
    L.xhc_kernel_name.argtypes = [ctypes.c_int]
    L.xhc_kernel_name.restype = ctypes.c_char_p
    return L


lib = _load()


def make_desc(B, S, C, N, k, ncomp, dtype, iters=20, eps=1e-6, gate_mode=XHC_GATE_SIGMOID,
              gram_schmidt=False, gs_eps=1e-6, route=0, per_token_active=False, hres_active=False):
    return xhc_desc(B, S, C, N, k, ncomp, iters, eps, dtype, gate_mode, int(gram_schmidt), gs_eps, int(route),
                    int(per_token_active), int(hres_active))


def zsave_stride(desc):
    """Floats per token of z_save (logits, r and, with a router, its record)."""
    return lib.xhc_zsave_stride(ctypes.byref(desc))


def workspace_size(desc, phase):
    return lib.xhc_workspace_size(ctypes.byref(desc), phase)


def carry_size(desc):
    return lib.xhc_carry_size(ctypes.byref(desc))


def bwd_state_size(desc):
    return lib.xhc_bwd_state_size(ctypes.byref(desc))


def strerror(code):
    return lib.xhc_strerror(code).decode()


def kernel_names():
    return [lib.xhc_kernel_name(i).decode() for i in range(lib.xhc_kernel_count())]


class Timer:
    """Per-kernel HIP-event timer (xhc_timer)."""

    def __init__(self):
        self._lib = lib                  # kept: module globals may be gone when a timer dies at exit
        self.handle = lib.xhc_timer_create()

    def reset(self):
        lib.xhc_timer_reset(self.handle)

    def read(self, kernel):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        rc = lib.xhc_timer_read(self.handle, kernel.encode(), ctypes.byref(ms), ctypes.byref(n))
        if rc:
            raise XhcError(rc, "xhc_timer_read")
        return ms.value, n.value

    def __del__(self):
        if getattr(self, "handle", None) and getattr(self, "_lib", None) is not None:
            self._lib.xhc_timer_destroy(self.handle)
            self.handle = None


# ---------------------------------------------------------------------------
# torch-facing wrappers (pointer and stream plumbing)
# ---------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return XHC_BF16
    if t.dtype == torch.float32:
        return XHC_F32
    raise TypeError(f"unsupported state dtype {t.dtype}")


def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _workspace(desc, phase, device, workspace, stream):
    """The caller's workspace, or a fresh one.  A fresh one is allocated on
    torch's current stream and freed when the call returns, while the
    kernels may still run on `stream`: it is recorded on that stream, so the
    caching allocator hands the block out again only after the stream's
    work up to now has finished."""
    import torch
    need = workspace_size(desc, phase)
    if need == 0:
        raise XhcError(-2, "xhc_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
        if stream is not None:
            workspace.record_stream(stream)
    return workspace, need


def _active_array(active):
    arr = (ctypes.c_int32 * len(active))(*[int(a) for a in active])
    return arr


def forward(X, out, W, active, X_new, h_in, *, B, S, w4=None, w8=None, w12=None, bias=None,
            z_save=None, xact_save=None, iters=20, eps=1e-6, gate_mode=XHC_GATE_SIGMOID,
            workspace=None, stream=None, timer=None, desc=None, carry_in=None, W_next=None,
            carry_out=None, gram_schmidt=False, gs_eps=1e-6, desc_next=None, route=0, W_route=None,
            b_route=None, route_idx=None, status=None, W_route_next=None, active_next=None):
    """xhc_forward on torch device tensors.  X [B*S,N,C], out [B*S,C], W [N*C,P].

    With carry_in, W_next or carry_out given, calls xhc_forward_chain: carry_in
    is the previous call's carry_out (X is then not projected and W may be
    None); W_next [N*C,P] with carry_out (xhc_carry_size bytes) forms the next
    sublayer's projection partials from X_new; desc_next (an xhc_desc) describes
    that sublayer when it differs from this one (k, ncomp, ...).  gram_schmidt=True
    orthogonalises the write-back components (modified Gram-Schmidt, epsilon gs_eps).
    route=R > 0 chooses the last R active slots per token with the router
    (W_route [N*C,N], b_route [N]); route_idx [B*S,k] int32 receives the
    per-token active lists, and active then needs only its first k-R entries.
    With desc.per_token_active = 1 (make_desc(..., per_token_active=True))
    route_idx instead holds the caller's per-token lists, and active is not read;
    status (int32 [2] on the device, zeroed by the caller) then receives the
    XHC_STATUS_* flags and the count of tokens whose list is bad.
    In a chain whose next sublayer has a router, W_route_next [N*C,N] and
    active_next (its host active list) give that router's columns."""
    T, N, C = X.shape
    ncomp = 4 if w4 is not None else 1
    if desc is None:
        desc = make_desc(B, S, C, N, len(active), ncomp, _dtype_code(X), iters, eps, gate_mode,
                         gram_schmidt, gs_eps, route)
    act = _active_array(active)
    args = xhc_fwd_args(_ptr(X), _ptr(out), _ptr(w4), _ptr(w8), _ptr(w12), _ptr(W), _ptr(bias),
                        ctypes.cast(act, ctypes.POINTER(ctypes.c_int32)), _ptr(X_new), _ptr(h_in),
                        _ptr(z_save), _ptr(xact_save), None if timer is None else timer.handle,
                        _ptr(W_route), _ptr(b_route), _ptr(route_idx), _ptr(status))
    ws, need = _workspace(desc, XHC_PHASE_FWD, X.device, workspace, stream)
    if carry_in is None and W_next is None and carry_out is None and desc_next is None:
        rc = lib.xhc_forward(ctypes.byref(desc), ctypes.byref(args), ws.data_ptr(), ws.numel(),
                             _stream_handle(stream))
        if rc:
            raise XhcError(rc, "xhc_forward")
        return
    act_next = _active_array(active_next) if active_next is not None else None
    chain = xhc_chain_args(_ptr(carry_in), _ptr(W_next), _ptr(carry_out),
                           None if desc_next is None else ctypes.pointer(desc_next), _ptr(W_route_next),
                           None if act_next is None else ctypes.cast(act_next, ctypes.POINTER(ctypes.c_int32)))
    rc = lib.xhc_forward_chain(ctypes.byref(desc), ctypes.byref(args), ctypes.byref(chain), ws.data_ptr(),
                               ws.numel(), _stream_handle(stream))
    if rc:
        raise XhcError(rc, "xhc_forward_chain")


def _desc_ptr(d):
    return None if d is None else ctypes.pointer(d)


def forward_pre(X, W, active, h_in, z_save, *, desc, bias=None, carry_in=None, W_next=None, carry_out=None,
                desc_next=None, workspace=None, stream=None, timer=None, W_route=None, b_route=None,
                route_idx=None, status=None):
    """xhc_forward_pre: coefficients and the dense read h_in of the state X
    (read only), z_save for the post call; with W_next/carry_out the next
    sublayer's projection partials over this sublayer's untouched rows.
    With a router (desc.route > 0) W_route/b_route are read and route_idx
    [B*S,k] int32 receives the per-token lists; with desc.per_token_active
    route_idx holds the caller's lists (status: optional int32[2] check)."""
    act = _active_array(active)
    args = xhc_pre_args(_ptr(X), _ptr(W), _ptr(bias), ctypes.cast(act, ctypes.POINTER(ctypes.c_int32)),
                        _ptr(h_in), _ptr(z_save), _ptr(carry_in), _ptr(W_next), _ptr(carry_out),
                        _desc_ptr(desc_next), None if timer is None else timer.handle,
                        _ptr(W_route), _ptr(b_route), _ptr(route_idx), _ptr(status))
    ws, need = _workspace(desc, XHC_PHASE_FWD, X.device, workspace, stream)
    rc = lib.xhc_forward_pre(ctypes.byref(desc), ctypes.byref(args), ws.data_ptr(), ws.numel(),
                             _stream_handle(stream))
    if rc:
        raise XhcError(rc, "xhc_forward_pre")


def forward_post(X, out, active, z_save, *, desc, w4=None, w8=None, w12=None, xact_save=None, W_next=None,
                 carry_out=None, desc_next=None, workspace=None, stream=None, timer=None, route_idx=None):
    """xhc_forward_post: the sparse write of the pre call's sublayer, in place
    in X, from its output `out` and the pre call's z_save; with W_next the
    new rows' projection partials are added to the pre call's carry_out.
    With per-token lists (router or given) route_idx is the pre call's."""
    act = _active_array(active)
    args = xhc_post_args(_ptr(X), _ptr(out), _ptr(w4), _ptr(w8), _ptr(w12),
                         ctypes.cast(act, ctypes.POINTER(ctypes.c_int32)), _ptr(z_save), _ptr(xact_save),
                         _ptr(W_next), _ptr(carry_out), _desc_ptr(desc_next), None if timer is None else timer.handle,
                         _ptr(route_idx))
    ws, need = _workspace(desc, XHC_PHASE_FWD, X.device, workspace, stream)
    rc = lib.xhc_forward_post(ctypes.byref(desc), ctypes.byref(args), ws.data_ptr(), ws.numel(),
                              _stream_handle(stream))
    if rc:
        raise XhcError(rc, "xhc_forward_post")


def forward_noalloc(X, out, W, active, X_new, h_in, *, B, S, w4=None, w8=None, w12=None, bias=None,
                    z_save=None, xact_save=None, iters=20, eps=1e-6, gate_mode=XHC_GATE_SIGMOID, stream=None,
                    desc=None, gram_schmidt=False, gs_eps=1e-6, route=0, W_route=None, b_route=None,
                    route_idx=None, status=None):
    """xhc_forward_noalloc: xhc_forward with the library's static scratch
    array in place of a workspace (no device memory is allocated)."""
    T, N, C = X.shape
    ncomp = 4 if w4 is not None else 1
    if desc is None:
        desc = make_desc(B, S, C, N, len(active), ncomp, _dtype_code(X), iters, eps, gate_mode,
                         gram_schmidt, gs_eps, route)
    act = _active_array(active)
    args = xhc_fwd_args(_ptr(X), _ptr(out), _ptr(w4), _ptr(w8), _ptr(w12), _ptr(W), _ptr(bias),
                        ctypes.cast(act, ctypes.POINTER(ctypes.c_int32)), _ptr(X_new), _ptr(h_in),
                        _ptr(z_save), _ptr(xact_save), None, _ptr(W_route), _ptr(b_route), _ptr(route_idx),
                        _ptr(status))
    rc = lib.xhc_forward_noalloc(ctypes.byref(desc), ctypes.byref(args), _stream_handle(stream))
    if rc:
        raise XhcError(rc, "xhc_forward_noalloc")


def backward(X, out, W, active, dX_new, dh_in, dX, dout, dW, *, B, S, xact=None, w4=None, w8=None,
             w12=None, bias=None, z_save=None, db=None, dw4=None, dw8=None, dw12=None, accumulate=False,
             iters=20, eps=1e-6, gate_mode=XHC_GATE_SIGMOID, workspace=None, stream=None, timer=None,
             desc=None, gram_schmidt=False, gs_eps=1e-6, route=0, W_route=None, route_idx=None,
             dW_route=None, db_route=None, b_route=None, status=None):
    """xhc_backward on torch device tensors (with a router: the forward's
    z_save and route_idx, and dW_route [N*C,N] / db_route [N] fp32 outputs;
    with per-token lists given by the caller: the same route_idx).

    With a router and z_save=None the backward recomputes the router's
    scores, and b_route must then be the forward's b_route: the library
    refuses a missing one (XHC_ERR_NULL) rather than reading it as zero --
    pass a zero tensor if the forward ran without one."""
    T, N, C = X.shape
    ncomp = 4 if w4 is not None else 1
    if desc is None:
        desc = make_desc(B, S, C, N, len(active), ncomp, _dtype_code(X), iters, eps, gate_mode,
                         gram_schmidt, gs_eps, route)
    act = _active_array(active)
    args = xhc_bwd_args(_ptr(X), _ptr(xact), _ptr(out), _ptr(w4), _ptr(w8), _ptr(w12), _ptr(W), _ptr(bias),
                        ctypes.cast(act, ctypes.POINTER(ctypes.c_int32)), _ptr(z_save), _ptr(dX_new),
                        _ptr(dh_in), _ptr(dX), _ptr(dout), _ptr(dW), _ptr(db), _ptr(dw4), _ptr(dw8),
                        _ptr(dw12), int(bool(accumulate)), None if timer is None else timer.handle,
                        _ptr(W_route), _ptr(route_idx), _ptr(dW_route), _ptr(db_route), _ptr(b_route),
                        _ptr(status))
    ws, need = _workspace(desc, XHC_PHASE_BWD, X.device, workspace, stream)
    rc = lib.xhc_backward(ctypes.byref(desc), ctypes.byref(args), ws.data_ptr(), ws.numel(),
                          _stream_handle(stream))
    if rc:
        raise XhcError(rc, "xhc_backward")


def backward_post(out, active, z_save, dX_new, dout, bwd_state, *, desc, w4=None, w8=None, w12=None, dw4=None,
                  dw8=None, dw12=None, accumulate=False, workspace=None, stream=None, timer=None, route_idx=None,
                  status=None):
    """xhc_backward_post: dout, the conv-weight gradients and the dot
    partials (into bwd_state, a device buffer of bwd_state_size(desc) bytes)
    from dX_new and the forward's z_save (and, with per-token lists, its
    route_idx; status: optional int32[2] check of the lists)."""
    act = _active_array(active)
    args = xhc_bwd_post_args(_ptr(out), _ptr(w4), _ptr(w8), _ptr(w12),
                             ctypes.cast(act, ctypes.POINTER(ctypes.c_int32)), _ptr(z_save), _ptr(dX_new),
                             _ptr(dout), _ptr(dw4), _ptr(dw8), _ptr(dw12), _ptr(bwd_state),
                             int(bool(accumulate)), None if timer is None else timer.handle,
                             _ptr(route_idx), _ptr(status))
    ws, need = _workspace(desc, XHC_PHASE_BWD, out.device, workspace, stream)
    rc = lib.xhc_backward_post(ctypes.byref(desc), ctypes.byref(args), ws.data_ptr(), ws.numel(),
                               _stream_handle(stream))
    if rc:
        raise XhcError(rc, "xhc_backward_post")


def backward_pre(X, W, active, z_save, dX_new, dh_in, bwd_state, dX, dW, *, desc, xact=None, bias=None, db=None,
                 accumulate=False, workspace=None, stream=None, timer=None, W_route=None, route_idx=None,
                 dW_route=None, db_route=None):
    """xhc_backward_pre: dX, dW and db from dX_new, dh_in and the bwd_state
    that xhc_backward_post left; with a router also dW_route [N*C,N] and
    db_route [N] (fp32), from W_route and the forward's route_idx."""
    act = _active_array(active)
    args = xhc_bwd_pre_args(_ptr(X), _ptr(xact), _ptr(W), _ptr(bias),
                            ctypes.cast(act, ctypes.POINTER(ctypes.c_int32)), _ptr(z_save), _ptr(dX_new),
                            _ptr(dh_in), _ptr(bwd_state), _ptr(dX), _ptr(dW), _ptr(db),
                            int(bool(accumulate)), None if timer is None else timer.handle,
                            _ptr(W_route), _ptr(route_idx), _ptr(dW_route), _ptr(db_route))
    ws, need = _workspace(desc, XHC_PHASE_BWD, X.device, workspace, stream)
    rc = lib.xhc_backward_pre(ctypes.byref(desc), ctypes.byref(args), ws.data_ptr(), ws.numel(),
                              _stream_handle(stream))
    if rc:
        raise XhcError(rc, "xhc_backward_pre")


def validate(desc, args, phase):
    """xhc_validate on an xhc_fwd_args / xhc_bwd_args structure (host only)."""
    return lib.xhc_validate(ctypes.byref(desc), ctypes.cast(ctypes.byref(args), _vp), phase)

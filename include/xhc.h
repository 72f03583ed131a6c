/*
 * xhc.h -- C ABI of libxhc: one xHC (Expanded Hyper-Connections) sublayer
 * update of an N-stream residual state, forward and backward, on an AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed (sources: the "xHC: Expanded Hyper-Connections" research
 * retrospective on qingkeai.online, sections "把 N 调大以后，事情开始不太对了"
 * (multi-stream state and the H_pre / H_post / H_res roles, Sinkhorn),
 * "最便宜的新信息，可能就在相邻 token 里" (Temporal Feature Augmentation)
 * and "模型可以拥有 16 条 streams，但每层只更新 4 条" (dense read, sparse
 * write); the explainer "xHC：把残差流扩到 N=16 的可扩展超连接", section
 * "核心方法"):
 *
 *   for every token t (T = B*S tokens, each with N streams of C channels):
 *     xbar  = X[t] flattened, xbar[i*C + c] = X[t, i, c]
 *     r     = sqrt(mean(xbar^2) + rms_eps)
 *     z     = (xbar / r) @ W + bias                      z in R^P
 *             P = N + k*ncomp + k*k, columns [pre N | post k*ncomp | res k*k]
 *             (post and res are a-major: post[a, m] = z[N + a*ncomp + m],
 *              L[a, b] = z[N + k*ncomp + a*k + b])
 *     H_pre = sigmoid(z_pre), H_post = sigmoid(z_post)  (1 in unit-gate mode)
 *     H_res = Sinkhorn(L): M = exp(L - rowmax L), then sinkhorn_iters times
 *             divide rows by their sums, then columns by their sums
 *     h_in[t]        = sum_i H_pre[i] X[t, i]                   (dense read)
 *     U_0 = out[t];  U_m[t, c] = sum_q w_m[c, q] out[t - K_m + 1 + q, c]
 *             for K_1..3 = 4, 8, 12 (causal, zero before the sequence start,
 *             w_m[c, K_m - 1] multiplies the current token)     (TFA)
 *     X_new[t, i_a]  = sum_b H_res[a, b] X[t, i_b] + sum_m H_post[a, m] U_m[t]
 *     X_new[t, i]    = X[t, i] for i not active        (sparse write, bitwise)
 *   with i_a = active[a], a < k.  With desc->gram_schmidt = 1 the write uses
 *   the orthogonalised components U~ (see xhc_desc) in place of U.  With
 *   desc->route = R > 0 the last R of the k active streams are chosen per
 *   token by a router and their write-back term is scaled (see xhc_desc).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless a field says HOST.  The caller owns
 *     all memory; the library never allocates, frees or synchronises, with
 *     two exceptions, both opt-in: a call that carries a timer (args->timer)
 *     creates the HIP events it records, and xhc_timer_read waits for them
 *     (see the timer calls at the end); xhc_forward_noalloc looks up its
 *     static array once per device.  Work is enqueued asynchronously on
 *     `stream` (NULL = the null stream).
 *   - Layouts are dense, row-major, C contiguous: X, X_new, dX_new, dX are
 *     [T, N, C]; out, h_in, dh_in, dout are [T, C]; W and dW are [N*C, P];
 *     w4/w8/w12 and their gradients are [C, 4], [C, 8], [C, 12].
 *   - dtype XHC_BF16: X, out, W, h_in, X_new, xact_save, dX_new, dh_in, dX,
 *     dout are bfloat16; arithmetic is fp32 (MFMA with fp32 accumulation);
 *     outputs are rounded to nearest even.  dtype XHC_F32: those are fp32.
 *     Conv weights, bias, z_save and every parameter gradient are fp32.
 *   - Every device pointer must be 16-byte aligned.
 *   - Return value: XHC_OK (0) or a negative XHC_ERR_* code.  A validation
 *     failure launches nothing.  XHC_ERR_HIP reports a launch failure.
 *   - Calls are reentrant; the library keeps no mutable global state.  Calls
 *     on different streams must not share output or workspace buffers.
 */
#ifndef XHC_H
#define XHC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* xhc_stream_t;   /* a hipStream_t */

enum { XHC_F32 = 0, XHC_BF16 = 1 };
enum { XHC_GATE_SIGMOID = 0, XHC_GATE_UNIT = 1 };
enum { XHC_PHASE_FWD = 0, XHC_PHASE_BWD = 1, XHC_PHASE_PRE = 2, XHC_PHASE_POST = 3,
       XHC_PHASE_BWD_POST = 4, XHC_PHASE_BWD_PRE = 5 };

enum {
  XHC_OK = 0,
  XHC_ERR_NULL = -1,         /* a required pointer is NULL                  */
  XHC_ERR_SHAPE = -2,        /* sizes out of the supported range            */
  XHC_ERR_INDEX = -3,        /* active index out of range or repeated       */
  XHC_ERR_ALIAS = -4,        /* forbidden overlap between buffers           */
  XHC_ERR_ALIGN = -5,        /* a pointer is not 16-byte aligned            */
  XHC_ERR_UNSUPPORTED = -6,  /* a mode the library does not implement       */
  XHC_ERR_WORKSPACE = -7,    /* workspace NULL or smaller than required     */
  XHC_ERR_HIP = -8,          /* a HIP call or kernel launch failed          */
  XHC_ERR_SCRATCH = -9       /* xhc_forward_noalloc: the problem needs more
                                scratch than XHC_NOALLOC_SCRATCH_BYTES      */
};

/* Size of the static device scratch array of xhc_forward_noalloc (64 MiB;
 * each GPU the library runs on holds one until the process ends). */
#define XHC_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Problem description.  Supported: B, S >= 1; 1 <= k <= 4; k <= N <= 16;
 * ncomp in {1, 4} (4 = TFA on: out plus three causal convolutions; 1 = out
 * only, the mHC-style write-back); C >= 8 with C % 8 == 0;
 * 1 <= sinkhorn_iters <= 64; rms_eps >= 0; B*S*N*C < 2^31.
 *
 * The last bound keeps every element index of the state within 32 bits (the
 * kernels address it through 32-bit buffer offsets); larger states are
 * XHC_ERR_SHAPE.  Sequences do not interact, so a larger batch runs as
 * several calls over groups of whole sequences, each with its pointers
 * offset to the group's first token (B = the group's size); in the backward,
 * accumulate = 1 on every call after the first sums dW, db and the conv
 * gradients over the groups (up to the order of fp32 sums).
 *
 * Gram-Schmidt (gram_schmidt = 1; source: the retrospective's section
 * "Conv 带来了新信息，也带来了新的麻烦", which removes from each conv
 * component its projections on the components before it and keeps the
 * output as it is): per token, over the C channels, U~_0 = U_0 and for
 * c = 1, 2, 3, starting from v = U_c, for j = 0 .. c-1 in turn
 *   v -= <v, U~_j> / (<U~_j, U~_j> + C * gs_eps) * U~_j,   U~_c = v;
 * the write then uses U~ in place of U.  No normalisation.  gs_eps > 0 keeps
 * a zero component (zero conv weights) at 0.  With ncomp == 1 it is the
 * identity.  A description with gram_schmidt = 0 (a zero-filled tail) is the
 * form without it, which the pages use when the backbone trains with Muon.
 * Accuracy: the library runs the procedure on each token's 4x4 Gram matrix
 * of the raw components (fp32 sums over C), the same procedure in exact
 * arithmetic.  Its error grows with the conditioning of that matrix: with
 * nearly collinear components (cosines of 0.99 and more) and fp32 storage,
 * X_new, h_in, dX and dout stay within 1e-4 + 1e-4 |ref| of an fp64
 * reference, but the gradient of the post logits carries relative errors up
 * to about 1e-3 on small entries, and dW, db and the conv-weight gradients
 * (sums over tokens) are then within 1e-3 of each column's largest
 * magnitude (about 1e-4 measured at cosine 0.999) rather than element by
 * element.
 *
 * Router (route = R > 0; source: the retrospective's section "模型可以拥有
 * 16 条 streams，但每层只更新 4 条", the paragraphs on fixed and routed
 * streams and on the sigmoid router): active[0 .. k-R) are fixed streams,
 * written at every token; slots k-R .. k-1 are chosen per token.  Scores
 *   y   = (xbar - mean(xbar)) / sqrt(var(xbar) + rms_eps)  (LayerNorm of the
 *         flattened state, population variance, no affine parameters: a gain
 *         and a shift fold into W_route and b_route)
 *   rho = y @ W_route + b_route                             rho in R^N
 * slot k-R+j takes the stream with the (j+1)-th largest rho among the
 * N-(k-R) streams that are not fixed (equal scores: lower stream id first;
 * the choice is made on fp32 scores), and its write-back term is scaled by
 * s = sigmoid(rho):  X_new[t, i_a] = sum_b H_res[a,b] X[t, i_b]
 * + s_a sum_m H_post[a,m] U_m.  The choice is discrete: the gradient reaches
 * the chosen streams' scores through s only.  Supported with 1 <= R <= k
 * (R = k: no fixed stream, all N streams are candidates); chained as
 * xhc_chain_args states.
 *
 * H_res from the active rows (hres_active = 1; source: the retrospective's
 * section "模型可以拥有 16 条 streams，但每层只更新 4 条", which credits the
 * sparse write with generating H_res at k^3 C instead of N^3 C cost): the
 * k*k res logits are the RMS-normed projection of the k active rows alone,
 *   xa = [X[t, i_0], .., X[t, i_{k-1}]],  r_act = sqrt(mean(xa^2) + rms_eps)
 *   L[a, b] = sum_{a'} X[t, i_{a'}] / r_act . W[i_{a'}*C .. , res column
 *             a*k + b] + bias
 * (the active streams' rows of W, normalised by the active state's own
 * RMS); the pre and post logits stay those of the full state.  W's res
 * columns on the other streams' rows are not read, and xhc_backward writes
 * zeros there in dW (or leaves them with accumulate = 1).  z_save then
 * holds P + 2 floats per token: logits, r, r_act.  With k = N it is the
 * default form. */
typedef struct {
  int32_t B, S, C, N, k, ncomp;
  int32_t sinkhorn_iters;   /* Sinkhorn row+column steps (20 by default)    */
  float rms_eps;            /* epsilon inside the RMS (1e-6 by default)     */
  int32_t dtype;            /* XHC_F32 or XHC_BF16                          */
  int32_t gate_mode;        /* XHC_GATE_SIGMOID, or XHC_GATE_UNIT (test mode:
                               H_pre = H_post = 1, no gate gradient)        */
  int32_t gram_schmidt;     /* 0: off; 1: modified Gram-Schmidt over U      */
  float gs_eps;             /* > 0 and finite when gram_schmidt = 1 (1e-6)  */
  int32_t route;            /* 0: the active list of every token is `active`;
                               R > 0: R routed slots (the retrospective's
                               setting is k = 4, R = 2)                     */
  int32_t per_token_active; /* 1: the caller gives every token its own list
                               in route_idx [T,k] (an input to both calls;
                               no router, write-back unscaled; the lists
                               must hold distinct streams, ids outside
                               [0, N) are read as 0, and the calls report
                               such lists through args->status); requires
                               route = 0; chained as xhc_chain_args
                               states.  0: off                              */
  int32_t hres_active;      /* 1: H_res generated from the k active rows (see
                               below); requires route = 0 and
                               per_token_active = 0, and is not chained.
                               0: off (every logit from the full state)     */
} xhc_desc;

/* Optional per-kernel timer (HIP events around every kernel a call
 * launches); NULL in normal use. */
typedef struct xhc_timer xhc_timer;

typedef struct {
  const void* X;       /* [T,N,C] state before the update                     */
  const void* out;     /* [T,C] sublayer output                               */
  const float* w4;     /* [C,4]  } TFA conv weights; all three NULL iff       */
  const float* w8;     /* [C,8]  } ncomp == 1                                 */
  const float* w12;    /* [C,12] }                                            */
  const void* W;       /* [N*C,P] projection weights, row i*C + c             */
  const float* bias;   /* [P] or NULL (zero)                                  */
  const int32_t* active; /* HOST [k] distinct stream ids; order binds row a.
                          With route = R > 0 only the first k-R are read;
                          with desc->per_token_active none (may be NULL)     */
  void* X_new;         /* [T,N,C]; == X: in place, only the k active rows are
                          written; otherwise must not overlap X and all N rows
                          are written (inactive rows copied bitwise)          */
  void* h_in;          /* [T,C] dense-read sublayer input; no overlap with X,
                          X_new, out                                          */
  float* z_save;       /* [T, xhc_zsave_stride(desc)] per token: logits z, r
                          (and with a router its record), or NULL; the
                          backward needs it                                   */
  void* xact_save;     /* [T,k,C] the k active rows of X before the update
                          (slot order: with a router, each token's list), or
                          NULL; the backward needs it after an in-place call  */
  xhc_timer* timer;    /* NULL, or a timer from xhc_timer_create             */
  /* router (read only when desc->route > 0; route_idx also with
     desc->per_token_active) */
  const void* W_route; /* [N*C,N] router weights, storage type, row i*C + c   */
  const float* b_route;  /* [N] or NULL (zero)                                */
  int32_t* route_idx;  /* [T,k] per-token active list (output), or NULL; the
                          backward needs it.  With desc->per_token_active
                          the caller's lists (input, required)               */
  int32_t* status;     /* NULL, or device int32[2] (16-byte aligned) that the
                          call checks given per-token lists into; see
                          XHC_STATUS_*.  Left untouched without
                          desc->per_token_active                              */
} xhc_fwd_args;

typedef struct {
  const void* X;       /* [T,N,C] state: the forward's input X, or (when xact
                          is not NULL) its in-place output X_new              */
  const void* xact;    /* [T,k,C] xact_save of an in-place forward, or NULL   */
  const void* out;     /* [T,C]                                               */
  const float *w4, *w8, *w12;  /* as in the forward                           */
  const void* W;       /* [N*C,P]                                             */
  const float* bias;   /* [P] or NULL                                         */
  const int32_t* active;  /* HOST [k], the forward's active list              */
  const float* z_save; /* [T, xhc_zsave_stride(desc)] from the forward, or
                          NULL (recomputed; then not with xact when the lists
                          are per token: router or given lists)              */
  const void* dX_new;  /* [T,N,C] gradient w.r.t. X_new                       */
  const void* dh_in;   /* [T,C] gradient w.r.t. h_in                          */
  void* dX;            /* [T,N,C] gradient w.r.t. X; may be == dX_new, must
                          not partially overlap it                            */
  void* dout;          /* [T,C] gradient w.r.t. out                           */
  float* dW;           /* [N*C,P] fp32                                        */
  float* db;           /* [P] fp32, or NULL                                   */
  float *dw4, *dw8, *dw12;  /* fp32 conv-weight gradients; NULL iff ncomp == 1 */
  int32_t accumulate;  /* 0: overwrite dW/db/dw* (and dW_route/db_route);
                          1: add to them                                      */
  xhc_timer* timer;
  /* router (read only when desc->route > 0; route_idx also with
     desc->per_token_active) */
  const void* W_route; /* [N*C,N]                                             */
  const int32_t* route_idx;  /* [T,k] the forward's per-token active lists    */
  float* dW_route;     /* [N*C,N] fp32                                        */
  float* db_route;     /* [N] fp32, or NULL                                   */
  const float* b_route;  /* [N] or NULL (zero): read only to recompute the
                          router's scores when z_save is NULL                 */
  int32_t* status;     /* NULL, or device int32[2] as in xhc_fwd_args: the
                          lists in route_idx are checked (router or given
                          lists); left untouched with one list for all      */
} xhc_bwd_args;

/* Status word of per-token active lists.  A call given args->status and
 * per-token lists checks every token's list on the device before its other
 * kernels: for each token with an id outside [0, N) or an id that appears
 * twice, it ORs XHC_STATUS_ID_RANGE and/or XHC_STATUS_ID_REPEAT into
 * status[0] and adds 1 to status[1] (the number of such tokens).  The call
 * never clears the word: zero it before the call (a fill kernel under graph
 * capture) and read it once the stream has finished the call.  Results
 * that depend on a flagged token (its own rows; in the backward also the
 * sums over tokens -- dW, db, the conv-weight gradients -- and dout within
 * the convolution window before it) are unspecified, but no access leaves
 * the caller's buffers: an out-of-range id reads as stream 0. */
enum { XHC_STATUS_ID_RANGE = 1, XHC_STATUS_ID_REPEAT = 2 };

/* Bytes of device workspace the call needs (phase XHC_PHASE_FWD for the
 * forward calls, XHC_PHASE_BWD for the backward ones); 0 for an invalid
 * description.  Pure host code. */
size_t xhc_workspace_size(const xhc_desc* desc, int phase);

/* Floats per token of z_save: P + 1 (logits, r) without a router; with
 * route = R > 0, P + 3 + 3R: logits, r, the LayerNorm mean and sd, then per
 * routed slot its score rho, rho - b_route and the column sum of W_route of
 * the chosen stream; with hres_active, P + 2: logits, r, r_act.  0 for an
 * invalid description.  Pure host code. */
int32_t xhc_zsave_stride(const xhc_desc* desc);

/* Checks desc and args (an xhc_fwd_args*, xhc_bwd_args*, xhc_pre_args*,
 * xhc_post_args*, xhc_bwd_post_args* or xhc_bwd_pre_args* for
 * XHC_PHASE_FWD, _BWD, _PRE, _POST, _BWD_POST, _BWD_PRE):
 * NULLs, shapes, indices, aliasing, alignment.  Pure host code, no HIP
 * call, usable without a GPU.  Returns XHC_OK or the first error found. */
int xhc_validate(const xhc_desc* desc, const void* args, int phase);

/* Forward update.  workspace: device buffer of at least
 * xhc_workspace_size(desc, XHC_PHASE_FWD) bytes, 256-byte aligned, not
 * shared with a concurrent call. */
int xhc_forward(const xhc_desc* desc, const xhc_fwd_args* args,
                void* workspace, size_t workspace_bytes, xhc_stream_t stream);

/* xhc_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The scratch that xhc_forward keeps in
 * the caller's workspace lives in a static device array of the library
 * instead (XHC_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends);
 * the call allocates and frees nothing.  Arguments and results are those of
 * xhc_forward (same kernels); args->timer must be NULL (a timer creates HIP
 * events: XHC_ERR_UNSUPPORTED).  A problem whose xhc_workspace_size(desc,
 * XHC_PHASE_FWD) exceeds XHC_NOALLOC_SCRATCH_BYTES is refused with
 * XHC_ERR_SCRATCH before anything is launched.  Every call on one GPU uses
 * that GPU's one array, which keeps the last call's contents: calls that
 * overlap in time on one GPU (other streams, other threads) race on it and
 * must be serialised by the caller.  The first call on a device looks up
 * that device's copy of the array (hipGetSymbolAddress, with the device
 * current); a failure there is XHC_ERR_HIP. */
int xhc_forward_noalloc(const xhc_desc* desc, const xhc_fwd_args* args, xhc_stream_t stream);

/* Backward of xhc_forward: gradients of X, out, W, bias and the conv
 * weights from those of X_new and h_in, through the unrolled Sinkhorn.
 * Reductions over tokens are deterministic (fixed order, no atomics). */
int xhc_backward(const xhc_desc* desc, const xhc_bwd_args* args,
                 void* workspace, size_t workspace_bytes, xhc_stream_t stream);

/* Chained forward of a stack of sublayers (source: the closing section of
 * the retrospective, which names an exactly equivalent dense-read correction
 * beyond the sparse write without giving its mechanism; this is a reading of
 * it).  The next sublayer may differ in k, ncomp, gates, Sinkhorn steps,
 * epsilons and Gram-Schmidt -- a stack alternates attention-side sublayers
 * with one write-back component and MLP-side ones with TFA (section
 * "最便宜的新信息，可能就在相邻 token 里" keeps TFA on the MLP side only) --
 * but shares B, S, C, N and the storage type.  Sublayer l's write pass reads
 * every row of its state and writes the k active rows, so the next
 * sublayer's state differs only in those rows; the pass also forms the next
 * sublayer's projection partials (x'.W' and sum x'^2 over each block of
 * channels, x' = X_new as stored), and the next call starts from them
 * instead of reading its state a second time.  Results equal those of
 * xhc_forward called layer by layer, up to the order of fp32 sums.
 *
 * Per-token lists (a router, desc->route > 0, or given lists) chain at N = 16
 * and k = 4, in place, with route = 2 (two fixed, two routed slots), route =
 * 4 or given lists (XHC_ERR_UNSUPPORTED otherwise): the pass reads each
 * token's own active rows and projects the new state row by row, the
 * routed rows' new values in place of the values it read.  A next sublayer
 * with a router gets its router's logits and sum(x') in the carry too; the
 * call then needs that sublayer's W_route_next and (with fixed slots) its
 * active_next. */
typedef struct {
  const void* carry_in;   /* NULL: project X here as xhc_forward does; else the
                             carry_out of the previous call, whose X_new is
                             this call's X (args->W is then not read)      */
  const void* W_next;     /* [N*C,P] projection weights of the next sublayer,
                             or NULL (no carry out: the last sublayer)      */
  void* carry_out;        /* xhc_carry_size(next description) bytes, or NULL
                             iff W_next is NULL; may be == carry_in (it is
                             consumed before it is written), otherwise no
                             overlap with any other buffer of the call      */
  const xhc_desc* desc_next; /* HOST; the next sublayer's description, or
                             NULL: the same as this call's.  W_next is then
                             [N*C, P of desc_next].  XHC_ERR_SHAPE when B, S,
                             C, N or dtype differ from this call's          */
  const void* W_route_next;  /* [N*C,N] the next sublayer's router weights, iff
                             it has a router (and W_next is given)           */
  const int32_t* active_next; /* HOST [k] the next sublayer's active list (its
                             fixed slots are read), with a router there      */
} xhc_chain_args;

/* Bytes of one carry buffer (fp32 partials per token and channel block);
 * 0 for an invalid description.  Pure host code. */
size_t xhc_carry_size(const xhc_desc* desc);

/* xhc_forward with the chaining of xhc_chain_args.  chain == NULL behaves
 * as xhc_forward.  Same workspace as xhc_forward (whatever desc_next is); the
 * carry buffers are the caller's.  Errors as xhc_forward, plus XHC_ERR_NULL
 * for W_next without carry_out, XHC_ERR_ALIAS for a carry overlapping another
 * buffer and XHC_ERR_SHAPE for a desc_next that does not describe the same
 * state (B, S, C, N, dtype) or is invalid. */
int xhc_forward_chain(const xhc_desc* desc, const xhc_fwd_args* args,
                      const xhc_chain_args* chain, void* workspace,
                      size_t workspace_bytes, xhc_stream_t stream);

/* Split forward (source: the retrospective's section "把 N 调大以后，事情开始不
 * 太对了": H_pre reads the sublayer's input, the sublayer F runs, H_post
 * writes its output back -- in a model, out = F(h_in) exists only after the
 * dense read).  xhc_forward_pre forms the coefficients and h_in;
 * xhc_forward_post, given out, rewrites the k active rows in place.  The
 * two calls in turn compute what xhc_forward computes in place (up to the
 * order of fp32 sums), and the backward is xhc_backward (or its split form
 * below) with the pre call's z_save.  Chained: the pre call of a sublayer
 * whose next sublayer's weights W_next are given also forms that
 * sublayer's projection partials over the rows this sublayer leaves
 * untouched (they are read anyway), and the post call adds the rewritten
 * rows' partials to the same carry; the next pre call starts from it
 * (carry_in) instead of reading its state for the projection -- the
 * dense-read correction of the retrospective's closing section, one state
 * read per sublayer.  hres_active not with a carry (XHC_ERR_UNSUPPORTED).
 *
 * With per-token lists (a router, desc->route > 0, or the caller's,
 * desc->per_token_active) there is no carry (XHC_ERR_UNSUPPORTED with
 * W_next or carry_in).  The pre call then runs the router, saves its record
 * in z_save and its choice in route_idx; its dense read does not depend on
 * the lists.  The post call takes route_idx and rewrites each token's own
 * rows: it reads only those rows and `out` (the routed slots' write-back
 * scaled by the saved scores, as xhc_forward does). */
typedef struct {
  const void* X;          /* [T,N,C] the state (read only)                     */
  const void* W;          /* [N*C,P]; not read with carry_in                    */
  const float* bias;      /* [P] or NULL (zero)                                 */
  const int32_t* active;  /* HOST [k] distinct stream ids, as xhc_forward's     */
  void* h_in;             /* [T,C] dense-read sublayer input                    */
  float* z_save;          /* [T, xhc_zsave_stride(desc)] required: logits and r;
                             xhc_forward_post and the backward read it          */
  const void* carry_in;   /* NULL: project X here; else the carry that the
                             previous sublayer's xhc_forward_post completed     */
  const void* W_next;     /* NULL, or the next sublayer's W [N*C, P_next]       */
  void* carry_out;        /* xhc_carry_size(next description) bytes iff W_next:
                             receives the untouched rows' partials; may equal
                             carry_in (consumed first)                          */
  const xhc_desc* desc_next; /* HOST, the next sublayer's description, or NULL
                             (the same); same B, S, C, N, dtype                 */
  xhc_timer* timer;
  /* per-token lists (read only with desc->route > 0 or per_token_active) */
  const void* W_route;    /* [N*C,N] router weights, with a router              */
  const float* b_route;   /* [N] or NULL (zero)                                 */
  int32_t* route_idx;     /* [T,k]: the router's lists (output, required: the
                             post call and the backward read them), or the
                             caller's given lists (input)                       */
  int32_t* status;        /* NULL, or device int32[2]: given lists are checked
                             into it (XHC_STATUS_*)                             */
} xhc_pre_args;

typedef struct {
  void* X;                /* [T,N,C] the state the pre call read; its k active
                             rows are rewritten in place                        */
  const void* out;        /* [T,C] the sublayer output F(h_in)                  */
  const float *w4, *w8, *w12;  /* TFA conv weights, NULL iff ncomp == 1         */
  const int32_t* active;  /* HOST [k], the pre call's                           */
  const float* z_save;    /* the pre call's z_save                              */
  void* xact_save;        /* [T,k,C] the old active rows (for the backward), or NULL */
  const void* W_next;     /* NULL, or the pre call's W_next                     */
  void* carry_out;        /* the pre call's carry_out (the new rows' partials
                             are added to it) iff W_next                        */
  const xhc_desc* desc_next; /* as in the pre call                              */
  xhc_timer* timer;
  const int32_t* route_idx; /* [T,k] the pre call's lists; required with a
                             router or given lists, otherwise not read          */
} xhc_post_args;

/* Workspace: xhc_workspace_size(desc, XHC_PHASE_FWD) bytes for either call
 * (its contents need not survive between them).  Errors as xhc_forward. */
int xhc_forward_pre(const xhc_desc* desc, const xhc_pre_args* args, void* workspace, size_t workspace_bytes,
                    xhc_stream_t stream);
int xhc_forward_post(const xhc_desc* desc, const xhc_post_args* args, void* workspace, size_t workspace_bytes,
                     xhc_stream_t stream);

/* Split backward, the reverse of the split forward (source: the same
 * section; in backpropagation the gradient reaches the write-back first and
 * the dense read last, with the sublayer's own backward between them).
 * xhc_backward_post runs first: from dX_new and the pre call's z_save it
 * forms dout (the gradient the sublayer's backward starts from), the conv-
 * weight gradients, and the dots of the gradient of each rewritten row with
 * each write-back component, which it leaves in the caller's bwd_state.
 * The sublayer's backward then turns dout into dh_in, and xhc_backward_pre
 * forms dX, dW and db from dX_new, dh_in and bwd_state.  The two calls in
 * turn run the kernels of xhc_backward in its order and give the same
 * results bit for bit (same z_save).  With a router or given lists both
 * calls take the forward's route_idx, and the second also the router's
 * weights and gradients.  With Gram-Schmidt the first call also runs the
 * part of the coefficient backward that the gradient through the
 * orthogonalisation needs (it reads the component dots and the saved
 * logits only), and the second call runs the whole coefficient backward.
 * With accumulate = 1 each call adds to the gradients it writes. */
typedef struct {
  const void* out;        /* [T,C] the sublayer output                          */
  const float *w4, *w8, *w12;  /* TFA conv weights, NULL iff ncomp == 1         */
  const int32_t* active;  /* HOST [k], the forward's active list                */
  const float* z_save;    /* [T, xhc_zsave_stride(desc)] the forward's, required */
  const void* dX_new;     /* [T,N,C] gradient w.r.t. X_new                      */
  void* dout;             /* [T,C] gradient w.r.t. out                          */
  float *dw4, *dw8, *dw12;  /* fp32 conv-weight gradients, NULL iff ncomp == 1  */
  void* bwd_state;        /* xhc_bwd_state_size(desc) bytes, 16-byte aligned:
                             written here, read by xhc_backward_pre            */
  int32_t accumulate;     /* 0: overwrite dw*; 1: add to them                   */
  xhc_timer* timer;
  const int32_t* route_idx; /* [T,k] the forward's per-token lists; required
                             with a router or given lists, otherwise not read   */
  int32_t* status;        /* NULL, or device int32[2]: the lists in route_idx
                             are checked into it (XHC_STATUS_*)                 */
} xhc_bwd_post_args;

typedef struct {
  const void* X;          /* [T,N,C] as in xhc_bwd_args                         */
  const void* xact;       /* [T,k,C] or NULL, as in xhc_bwd_args                */
  const void* W;          /* [N*C,P]                                            */
  const float* bias;      /* [P] or NULL                                        */
  const int32_t* active;  /* HOST [k], the forward's active list                */
  const float* z_save;    /* the forward's z_save, required                     */
  const void* dX_new;     /* [T,N,C] as given to xhc_backward_post              */
  const void* dh_in;      /* [T,C] gradient w.r.t. h_in                         */
  const void* bwd_state;  /* written by xhc_backward_post on the same problem   */
  void* dX;               /* [T,N,C]; may be == dX_new, must not partially
                             overlap it                                         */
  float* dW;              /* [N*C,P] fp32                                       */
  float* db;              /* [P] fp32, or NULL                                  */
  int32_t accumulate;     /* 0: overwrite dW/db (and dW_route/db_route); 1: add */
  xhc_timer* timer;
  /* per-token lists (read only with desc->route > 0 or per_token_active) */
  const void* W_route;    /* [N*C,N], with a router                             */
  const int32_t* route_idx; /* [T,k] the forward's per-token lists, required   */
  float* dW_route;        /* [N*C,N] fp32, with a router                        */
  float* db_route;        /* [N] fp32, or NULL                                  */
} xhc_bwd_pre_args;

/* Bytes of bwd_state (fp32 dot partials per token and channel block); 0 for
 * an invalid description.  Pure host code. */
size_t xhc_bwd_state_size(const xhc_desc* desc);

/* Workspace: xhc_workspace_size(desc, XHC_PHASE_BWD) bytes for either call
 * (its contents need not survive between them; bwd_state must).  Errors as
 * xhc_backward. */
int xhc_backward_post(const xhc_desc* desc, const xhc_bwd_post_args* args, void* workspace,
                      size_t workspace_bytes, xhc_stream_t stream);
int xhc_backward_pre(const xhc_desc* desc, const xhc_bwd_pre_args* args, void* workspace,
                     size_t workspace_bytes, xhc_stream_t stream);

/* Message of an XHC_* code (static string). */
const char* xhc_strerror(int code);

/* Timer: records HIP events around each kernel launched by calls that carry
 * it, on the call's stream.  It is the one part of the library that creates
 * HIP objects: a call that carries a timer creates (hipEventCreate) each
 * event the first time the timer needs it and keeps it for reuse after
 * xhc_timer_reset; xhc_timer_destroy destroys them.  A failed creation only
 * drops that measurement.  xhc_timer_read blocks the calling thread until
 * the recorded events of `kernel` have completed (hipEventSynchronize), then
 * returns the summed milliseconds and launch count of the kernel named
 * `kernel` (one of the names xhc_kernel_name returns), or a negative code.
 * A timer is not for code under graph capture (event records would be
 * captured) nor for xhc_forward_noalloc (XHC_ERR_UNSUPPORTED); it is not
 * safe to share between threads. */
xhc_timer* xhc_timer_create(void);
void xhc_timer_destroy(xhc_timer* timer);
void xhc_timer_reset(xhc_timer* timer);
int xhc_timer_read(xhc_timer* timer, const char* kernel, double* total_ms,
                   int64_t* launches);
int xhc_kernel_count(void);
const char* xhc_kernel_name(int i);

#ifdef __cplusplus
}
#endif
#endif /* XHC_H */

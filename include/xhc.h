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
 *     all memory; the library never allocates, frees or synchronises.  Work
 *     is enqueued asynchronously on `stream` (NULL = the null stream).
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
enum { XHC_PHASE_FWD = 0, XHC_PHASE_BWD = 1 };

enum {
  XHC_OK = 0,
  XHC_ERR_NULL = -1,         /* a required pointer is NULL                  */
  XHC_ERR_SHAPE = -2,        /* sizes out of the supported range            */
  XHC_ERR_INDEX = -3,        /* active index out of range or repeated       */
  XHC_ERR_ALIAS = -4,        /* forbidden overlap between buffers           */
  XHC_ERR_ALIGN = -5,        /* a pointer is not 16-byte aligned            */
  XHC_ERR_UNSUPPORTED = -6,  /* a mode the library does not implement       */
  XHC_ERR_WORKSPACE = -7,    /* workspace NULL or smaller than required     */
  XHC_ERR_HIP = -8           /* a HIP call or kernel launch failed          */
};

/* Problem description.  Supported: B, S >= 1; 1 <= k <= 4; k <= N <= 16;
 * ncomp in {1, 4} (4 = TFA on: out plus three causal convolutions; 1 = out
 * only, the mHC-style write-back); C >= 8 with C % 8 == 0;
 * 1 <= sinkhorn_iters <= 64; rms_eps >= 0; B*S*N*C < 2^31.
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
 * the chosen streams' scores through s only.  Supported with at most 15
 * candidate streams (N - (k-R) <= 15, so at N = 16 at least one fixed
 * stream) and 1 <= R <= k; not with the chained forward. */
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
                               [0, N) are read as 0); requires route = 0 and
                               is not chained.  0: off                      */
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
} xhc_bwd_args;

/* Bytes of device workspace the call needs (phase XHC_PHASE_FWD or
 * XHC_PHASE_BWD); 0 for an invalid description.  Pure host code. */
size_t xhc_workspace_size(const xhc_desc* desc, int phase);

/* Floats per token of z_save: P + 1 (logits, r) without a router; with
 * route = R > 0, P + 3 + 3R: logits, r, the LayerNorm mean and sd, then per
 * routed slot its score rho, rho - b_route and the column sum of W_route of
 * the chosen stream.  0 for an invalid description.  Pure host code. */
int32_t xhc_zsave_stride(const xhc_desc* desc);

/* Checks desc and args (an xhc_fwd_args* or xhc_bwd_args* per phase):
 * NULLs, shapes, indices, aliasing, alignment.  Pure host code, no HIP
 * call, usable without a GPU.  Returns XHC_OK or the first error found. */
int xhc_validate(const xhc_desc* desc, const void* args, int phase);

/* Forward update.  workspace: device buffer of at least
 * xhc_workspace_size(desc, XHC_PHASE_FWD) bytes, 256-byte aligned, not
 * shared with a concurrent call. */
int xhc_forward(const xhc_desc* desc, const xhc_fwd_args* args,
                void* workspace, size_t workspace_bytes, xhc_stream_t stream);

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
 * xhc_forward called layer by layer, up to the order of fp32 sums. */
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

/* Message of an XHC_* code (static string). */
const char* xhc_strerror(int code);

/* Timer: records HIP events around each kernel launched by calls that carry
 * it.  xhc_timer_read synchronises on the recorded events and returns the
 * summed milliseconds and launch count of the kernel named `kernel` (one of
 * the names xhc_kernel_name returns), or a negative code. */
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

// Internal launch interface between the C-ABI entry points and the kernels.
#pragma once
#include <hip/hip_runtime.h>

#include "xhc_plan.h"

struct xhc_timer;   // defined in xhc_api.cpp

namespace xhc {

// Kernel ids reported by the timer (names in xhc_api.cpp).
enum KernelId {
  KID_PACK_WT = 0, KID_PROJ, KID_COEF, KID_MIX,
  KID_PACK_WP, KID_BDOTS, KID_BCOEF, KID_BGRAD, KID_BREDUCE, KID_BXDOTS,
  KID_MIXPROJ, KID_GRAM, KID_BDOTS_GS, KID_RCOLSUM, KID_RPASS, KID_RDWR, KID_CHECK, KID_BPREP,
  KID_COUNT
};
// Alias kept for the backward's coefficient recompute from z_save.
constexpr KernelId KID_BCOEF_FWD = KID_COEF;

// Records a start event before and a stop event after the launches in its
// scope when a timer is attached (no-op otherwise).
void timer_mark(xhc_timer* tm, int kid, hipStream_t st, bool start);
struct TimedLaunch {
  xhc_timer* tm; int kid; hipStream_t st;
  TimedLaunch(xhc_timer* t, int k, hipStream_t s) : tm(t), kid(k), st(s) { if (tm) timer_mark(tm, kid, st, true); }
  ~TimedLaunch() { if (tm) timer_mark(tm, kid, st, false); }
};

// Where each stream's rows of the pre-update state live: element pointer of
// stream i's row for token 0 and the element stride between tokens.  Either
// the state itself (base X + i*C, stride N*C) or, for the active streams
// after an in-place forward, the saved rows (base xact + a*C, stride k*C).
struct StreamRows {
  const void* base[16];
  int64_t stride[16];
};

inline StreamRows stream_rows(const Plan& p, const void* X, const void* xact, const int32_t* active) {
  StreamRows s;
  const char* xb = static_cast<const char*>(X);
  for (int i = 0; i < 16; ++i) {
    s.base[i] = xb + (size_t)(i < p.N ? i : 0) * p.C * p.esz;
    s.stride[i] = p.NC;
  }
  if (xact) {
    const char* ab = static_cast<const char*>(xact);
    for (int a = 0; a < p.k; ++a) {
      s.base[active[a]] = ab + (size_t)a * p.C * p.esz;
      s.stride[active[a]] = (int64_t)p.k * p.C;
    }
  }
  return s;
}

// The active-row form's description for the kernels (mask 0 when it is off).
inline HresActive hres_active(const Plan& p, const int32_t* active) {
  HresActive h{0u, 0, 0, 0.f};
  if (!p.hact) return h;
  for (int a = 0; a < p.k; ++a) h.mask |= 1u << active[a];
  h.res0 = p.N + p.k * p.nc;
  h.res1 = h.res0 + p.k * p.k;
  h.inv_kc = 1.0f / ((float)p.k * (float)p.C);
  return h;
}

// Order in which the fused write + next-projection pass visits the state
// rows: the k active rows (in the order of `active`), then the other rows
// ascending; entries past N repeat the first.  Slot s in bits 4s .. 4s+3.
struct RowOrder { uint64_t bits; };
__host__ __device__ inline int row_of(const RowOrder& o, int slot) { return (int)((o.bits >> (4 * slot)) & 15u); }

int launch_forward(const Plan& p, const xhc_fwd_args* a, void* ws, hipStream_t st);
// Forward with an optional projection carried in from the previous sublayer
// (carry_in) and an optional projection of X_new for the next sublayer
// (W_next -> carry_out).
// pn: the next sublayer's plan (its P, tile count and carry layout).
int launch_forward_chain(const Plan& p, const Plan& pn, const xhc_fwd_args* a, const xhc_chain_args* c, void* ws,
                         hipStream_t st);
// The buffers of the fused write pass (xhc_chain.hip).
struct MixArgs {
  const void* X;
  const void* out;
  const float *w4, *w8, *w12;
  void* X_new;
  void* h_in;
  void* xact_save;
  const int32_t* active;
};
// Passes of k_mixproj: the whole write pass, its dense read only, its sparse write only.
enum { MIX_FULL = 0, MIX_PRE = 1, MIX_POST = 2 };
// Per-token lists in the fused pass: the rows that are not fixed (ascending)
// and the caller's lists (NULL: the router's, from the coefficient records).
struct MixRoute {
  RowOrder cand;
  int ncand;
  const int32_t* ids;
};
void launch_mixproj(const Plan& p, const Plan& pn, int mode, const MixArgs& m, const float* coef, const void* Wf,
                    float* carry, hipStream_t st, const int32_t* ids = nullptr);
// Split forward (xhc_forward_pre / xhc_forward_post).
int launch_forward_pre(const Plan& p, const Plan& pn, const xhc_pre_args* a, void* ws, hipStream_t st);
int launch_forward_post(const Plan& p, const Plan& pn, const xhc_post_args* a, void* ws, hipStream_t st);
int launch_coef_bwd(const Plan& p, const void* X, const void* xact, const int32_t* active, const void* W,
                    const float* bias, const float* z_save, void* ws, float* coef, float* z_out,
                    hipStream_t st, xhc_timer* tm, const void* W_route, const float* b_route,
                    const int32_t* force);
int launch_backward(const Plan& p, const xhc_bwd_args* a, void* ws, hipStream_t st);
int launch_coef_saved(const Plan& p, const float* z_save, float* coef, hipStream_t st, xhc_timer* tm);
// Split backward (xhc_backward_post, then xhc_backward_pre).
int launch_backward_post(const Plan& p, const xhc_bwd_post_args* a, void* ws, hipStream_t st);
int launch_backward_pre(const Plan& p, const xhc_bwd_pre_args* a, void* ws, hipStream_t st);
// Gram-Schmidt's Gram records of the components (forward): gram[cb][t][16]
// partials over channel blocks of B1_WAVES * B1_WAVE_CH.
void launch_gram(const Plan& p, const void* out, const float* w4, const float* w8, const float* w12, float* gram,
                 hipStream_t st);
// Router (xhc_route.hip): partial column sums of W_route, rcs[RCS_BLK][16].
void launch_route_colsum(const Plan& p, const void* W_route, float* rcs, hipStream_t st);
// Router, backward: pass[t][b] = sum_a H_res[a, b] G_a, and dW_route from
// B2's partials.
void launch_check_lists(const Plan& p, const int32_t* ids, int32_t* status, hipStream_t st);
void launch_route_pass(const Plan& p, const void* dXn, const int32_t* ridx, const float* hres, void* pass,
                       hipStream_t st);
void launch_route_dwr(const Plan& p, const float* dwp, const float* rred, float* dWr, int accumulate,
                      hipStream_t st);
// Router, split forward: the routed slots' post coefficients of records
// rebuilt from z_save, times sigmoid of their saved scores.
void launch_route_scale_post(const Plan& p, const float* z_save, float* coef, hipStream_t st);

}  // namespace xhc

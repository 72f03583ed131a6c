// C-ABI entry points of libxhc: validation, workspace planning, dispatch,
// per-kernel timer.  Validation and planning are plain host code.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "xhc_launch.h"
#include "xhc_plan.h"

namespace xhc {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int make_plan(const xhc_desc* d, Plan* p) {
  if (!d || !p) return XHC_ERR_NULL;
  if (d->B < 1 || d->S < 1 || d->C < 8 || (d->C % 8) != 0) return XHC_ERR_SHAPE;
  if (d->k < 1 || d->k > 4 || d->N < d->k || d->N > 16) return XHC_ERR_SHAPE;
  if (d->ncomp != 1 && d->ncomp != 4) return XHC_ERR_SHAPE;
  if (d->sinkhorn_iters < 1 || d->sinkhorn_iters > 64) return XHC_ERR_SHAPE;
  if (!(d->rms_eps >= 0.f) || !std::isfinite(d->rms_eps)) return XHC_ERR_SHAPE;
  if (d->dtype != XHC_F32 && d->dtype != XHC_BF16) return XHC_ERR_UNSUPPORTED;
  if (d->gate_mode != XHC_GATE_SIGMOID && d->gate_mode != XHC_GATE_UNIT) return XHC_ERR_UNSUPPORTED;
  if (d->gram_schmidt != 0 && d->gram_schmidt != 1) return XHC_ERR_UNSUPPORTED;
  if (d->gram_schmidt && !(d->gs_eps > 0.f && std::isfinite(d->gs_eps))) return XHC_ERR_SHAPE;
  const int64_t T = (int64_t)d->B * d->S;
  if (T * d->N * (int64_t)d->C >= ((int64_t)1 << 31)) return XHC_ERR_SHAPE;
  if (d->route < 0 || d->route > d->k) return XHC_ERR_SHAPE;
  if (d->per_token_active != 0 && d->per_token_active != 1) return XHC_ERR_UNSUPPORTED;
  if (d->per_token_active && d->route) return XHC_ERR_UNSUPPORTED;
  if (d->hres_active != 0 && d->hres_active != 1) return XHC_ERR_UNSUPPORTED;
  if (d->hres_active && (d->route || d->per_token_active)) return XHC_ERR_UNSUPPORTED;

  Plan& q = *p;
  q.B = d->B; q.S = d->S; q.C = d->C; q.N = d->N; q.k = d->k; q.nc = d->ncomp;
  q.P = q.N + q.k * q.nc + q.k * q.k;
  q.NT = (int)cdiv(q.P, 16);
  q.T = (int)T;
  q.iters = d->sinkhorn_iters; q.dtype = d->dtype; q.gate = d->gate_mode; q.eps = d->rms_eps;
  q.NC = (int64_t)q.N * q.C;
  q.esz = q.dtype == XHC_BF16 ? 2 : 4;
  q.gs = d->gram_schmidt == 1 && q.nc == 4;
  q.gs_ceps = q.gs ? (float)q.C * d->gs_eps : 0.f;
  q.R = d->route;
  q.pt = q.R > 0 || d->per_token_active == 1;
  q.nfix = q.k - q.R;
  q.ncand = q.R ? q.N - q.nfix : 0;
  if (q.R) q.NT = 4;                       // tile 3: the router's candidate columns
  q.hact = d->hres_active == 1;
  q.zsv = q.R ? q.P + 3 + 3 * q.R : q.hact ? q.P + 2 : q.P + 1;
  q.dzs = q.pt ? DZ_R : 48;
  q.dwr = q.pt ? 64 : 48;
  q.rec_bytes = q.pt ? REC_R_BYTES : REC_BYTES;

  // forward
  q.SK = q.N;
  q.ZST = q.NT * 16 + 4;
  q.proj_tiles = (int)cdiv(T, PROJ_TOK);
  q.mix_cblocks = (int)cdiv(q.C, MIX_THREADS * MIX_CH);
  {
    const int64_t waves_per_row = cdiv(q.C, MIX_CH * 64) * q.B;
    const int64_t segs = std::max<int64_t>(1, MIX_TARGET_WAVES / std::max<int64_t>(1, waves_per_row));
    q.mix_lseg = (int)std::max<int64_t>(16, cdiv(q.S, segs));
    q.mix_segs = (int)cdiv(q.S, q.mix_lseg);
  }

  // backward: B1 segments sized for ~2048 waves
  q.b1_cblocks = (int)cdiv(q.C, B1_WAVES * B1_WAVE_CH);
  {
    const int64_t waves_per_row = (int64_t)q.b1_cblocks * B1_WAVES;
    const int64_t want_rows = std::max<int64_t>(1, cdiv(2048, waves_per_row));
    const int64_t segs = std::max<int64_t>(1, cdiv(want_rows, q.B));
    int64_t lseg = cdiv(cdiv(q.S, segs), 12) * 12;
    lseg = std::max<int64_t>(lseg, 12);
    q.b1_lseg = (int)lseg;
    q.b1_segs = (int)cdiv(q.S, lseg);
  }
  q.bx_cblocks = (int)cdiv(q.C, BX_CB);
  q.bx_tiles = (int)cdiv(T, BX_TOK);
  // with per-token lists the active rows change per token: all rows in groups of 4
  q.b2_rowgroups = q.pt ? (int)cdiv(q.N, 4) : 1 + (int)cdiv(q.N - q.k, 4);
  q.b2_cblocks = (int)cdiv(q.C, B2_CB);
  q.Tpad = cdiv(T, B2_TT) * B2_TT;
  {
    const int64_t base = (int64_t)q.b2_rowgroups * q.b2_cblocks;
    const int64_t steps = cdiv(T, B2_TT * B2_SUB);            // iterations of B2_SUB tiles
    int64_t ts = std::min<int64_t>(std::max<int64_t>(1, (B2_TARGET_WG + base / 2) / base), steps);
    const int64_t steps_per = cdiv(steps, ts);
    q.b2_tok_per_split = (int)(steps_per * B2_TT * B2_SUB);
    q.b2_ts = (int)cdiv(T, q.b2_tok_per_split);
  }

  // chained forward: channel blocks of whole chunks, at most 16 of them
  {
    const int cw = q.dtype == XHC_BF16 ? 64 : 32;
    q.mp_nch = (int)cdiv(q.C, cw);
    const int ncb = std::min(16, q.mp_nch);
    q.mp_cpw = (int)cdiv(q.mp_nch, ncb);
    q.mp_ncb = (int)cdiv(q.mp_nch, q.mp_cpw);
    q.mp_nbatch = (int)cdiv(T, 128);
    q.carry_bytes = (size_t)q.mp_ncb * T * q.ZST * 4;
  }

  // workspace layouts
  size_t o = 0;
  // sized for the largest tile count: a chained call packs the next
  // sublayer's W there, whose P may differ
  q.off_wt = o;     o = align256(o + (size_t)q.N * cdiv(q.C, 32) * 32 * NT_MAX * 16 * q.esz);
  q.off_zpart = o;  o = align256(o + (size_t)q.SK * T * q.ZST * 4);
  q.off_coef = o;   o = align256(o + (size_t)T * COEF_STRIDE * 4);
  q.off_gram = o;   o = align256(o + (q.gs ? (size_t)q.b1_cblocks * T * 16 * 4 : 0));
  q.off_rcs = o;    o = align256(o + (q.R ? (size_t)(RCS_BLK + 1) * 16 * 4 : 0));
  q.fwd_bytes = o;
  // backward reuses the forward regions (projection recompute) and adds:
  q.off_zbuf = o;   o = align256(o + (size_t)T * q.zsv * 4);
  q.off_wp = o;     o = align256(o + (size_t)q.NC * 64 * q.esz);
  q.off_dpart = o;  o = align256(o + (size_t)q.b1_cblocks * T * DOT_STRIDE * 4);
  q.off_dpa = o;    o = align256(o + (size_t)q.bx_cblocks * T * BX_OUT * 4);
  q.off_dwpart = o; o = align256(o + (q.nc == 4 ? (size_t)q.B * q.b1_segs * q.C * 24 * 4 : 0));
  q.off_dz = o;     o = align256(o + (size_t)T * q.dzs * 4);
  q.off_rec = o;    o = align256(o + (size_t)(q.Tpad / B2_TT) * q.rec_bytes);
  q.off_dwpart2 = o; o = align256(o + (size_t)q.b2_ts * q.NC * q.dwr * 4);
  q.off_gss = o;    o = align256(o + (q.gs ? (size_t)T * 16 * 4 : 0));
  q.off_hres = o;   o = align256(o + (q.pt ? (size_t)T * 16 * 4 : 0));
  q.off_pass = o;   o = align256(o + (q.pt ? (size_t)T * q.k * q.C * q.esz : 0));
  q.off_rred = o;   o = align256(o + (q.pt ? (size_t)16 * 4 : 0));
  q.bwd_bytes = o;
  q.state_bytes = (size_t)q.b1_cblocks * T * DOT_STRIDE * 4;
  return XHC_OK;
}

// ---------------------------------------------------------------------------
// validation helpers
// ---------------------------------------------------------------------------
struct Span { const char* lo; size_t n; };
static Span span(const void* p, size_t n) { return Span{static_cast<const char*>(p), n}; }
static bool overlap(Span a, Span b) {
  if (!a.lo || !b.lo || !a.n || !b.n) return false;
  return a.lo < b.lo + b.n && b.lo < a.lo + a.n;
}
static bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

// The host active list: all k entries, with a router the k - R fixed ones,
// with the caller's per-token lists none.
static int check_active(const Plan& p, const int32_t* act) {
  const int n = p.pt && !p.R ? 0 : p.nfix;
  if (n && !act) return XHC_ERR_NULL;
  for (int a = 0; a < n; ++a) {
    if (act[a] < 0 || act[a] >= p.N) return XHC_ERR_INDEX;
    for (int b = 0; b < a; ++b)
      if (act[a] == act[b]) return XHC_ERR_INDEX;
  }
  return XHC_OK;
}

// Outputs may not overlap each other nor any input, except the listed
// permitted identity (same base, same size).
static bool any_overlap(const std::vector<Span>& outs, const std::vector<Span>& ins, Span same_a, Span same_b) {
  for (size_t i = 0; i < outs.size(); ++i) {
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlap(outs[i], outs[j])) return true;
    for (const Span& in : ins) {
      if (outs[i].lo == same_a.lo && in.lo == same_b.lo && same_a.lo == same_b.lo && same_a.n == same_b.n &&
          outs[i].lo != nullptr)
        continue;
      if (overlap(outs[i], in)) return true;
    }
  }
  return false;
}

static int validate_fwd(const Plan& p, const xhc_fwd_args* a, bool need_W = true) {
  if (!a) return XHC_ERR_NULL;
  if (!a->X || !a->out || (need_W && !a->W) || !a->X_new || !a->h_in) return XHC_ERR_NULL;
  const bool has_conv = a->w4 || a->w8 || a->w12;
  if (p.nc == 4 && (!a->w4 || !a->w8 || !a->w12)) return XHC_ERR_NULL;
  if (p.nc == 1 && has_conv) return XHC_ERR_UNSUPPORTED;
  if (p.R && !a->W_route) return XHC_ERR_NULL;
  if (p.pt && !p.R && !a->route_idx) return XHC_ERR_NULL;
  int rc = check_active(p, a->active);
  if (rc) return rc;
  const void* ptrs[] = {a->X, a->out, a->w4, a->w8, a->w12, a->W, a->bias, a->X_new, a->h_in, a->z_save, a->xact_save,
                        p.R ? a->W_route : nullptr, p.R ? a->b_route : nullptr, p.pt ? a->route_idx : nullptr,
                        p.pt && !p.R ? a->status : nullptr};
  for (const void* q : ptrs)
    if (misaligned(q)) return XHC_ERR_ALIGN;
  const size_t T = p.T, e = p.esz;
  const Span X = span(a->X, T * p.NC * e), Xn = span(a->X_new, T * p.NC * e);
  const Span out = span(a->out, T * p.C * e), hin = span(a->h_in, T * p.C * e);
  const Span W = span(a->W, (size_t)p.NC * p.P * e), bias = span(a->bias, a->bias ? (size_t)p.P * 4 : 0);
  const Span w4 = span(a->w4, a->w4 ? (size_t)p.C * 16 : 0), w8 = span(a->w8, a->w8 ? (size_t)p.C * 32 : 0),
             w12 = span(a->w12, a->w12 ? (size_t)p.C * 48 : 0);
  const Span zs = span(a->z_save, a->z_save ? T * p.zsv * 4 : 0);
  const Span xs = span(a->xact_save, a->xact_save ? T * p.k * p.C * e : 0);
  const Span Wr = span(p.R ? a->W_route : nullptr, (size_t)p.NC * p.N * e);
  const Span br = span(p.R ? a->b_route : nullptr, (size_t)p.N * 4);
  const Span ri = span(p.pt ? a->route_idx : nullptr, T * p.k * 4);
  const Span stw = span(p.pt && !p.R ? a->status : nullptr, 8);
  if (a->X_new != a->X && overlap(X, Xn)) return XHC_ERR_ALIAS;
  const bool ri_out = p.R > 0;                  // the router writes the lists; given lists are read
  std::vector<Span> outs = {Xn, hin, zs, xs, stw};
  std::vector<Span> ins = {X, out, W, bias, w4, w8, w12, Wr, br};
  (ri_out ? outs : ins).push_back(ri);
  if (any_overlap(outs, ins, Xn, X)) return XHC_ERR_ALIAS;
  return XHC_OK;
}

// Chained forward: the carry buffers and the next sublayer's weights.
// pn: the next sublayer's plan (== p without desc_next)
static int validate_chain(const Plan& p, const Plan& pn, const xhc_fwd_args* a, const xhc_chain_args* c) {
  if (!c) return XHC_OK;
  if (p.pt) {
    // per-token lists: the full pass at N = 16, k = 4, in place, with two or
    // four slots chosen per token
    const int rts = p.R ? p.R : p.k;
    if (p.N != 16 || p.k != 4 || a->X_new != a->X || (rts != 2 && rts != 4)) return XHC_ERR_UNSUPPORTED;
  }
  // the carried partials sum every stream of a channel block
  if (p.hact || pn.hact) return XHC_ERR_UNSUPPORTED;
  if ((c->W_next == nullptr) != (c->carry_out == nullptr)) return XHC_ERR_NULL;
  if (misaligned(c->carry_in) || misaligned(c->carry_out) || misaligned(c->W_next)) return XHC_ERR_ALIGN;
  if (c->W_next && pn.R) {
    // the next sublayer's router columns and candidate order
    if (!c->W_route_next) return XHC_ERR_NULL;
    if (misaligned(c->W_route_next)) return XHC_ERR_ALIGN;
    const int rc = check_active(pn, c->active_next);
    if (rc) return rc;
  }
  if (pn.B != p.B || pn.S != p.S || pn.C != p.C || pn.N != p.N || pn.dtype != p.dtype) return XHC_ERR_SHAPE;
  const size_t T = p.T, e = p.esz;
  const Span cin = span(c->carry_in, c->carry_in ? p.carry_bytes : 0);
  const Span cout = span(c->carry_out, c->carry_out ? pn.carry_bytes : 0);
  const Span Wn = span(c->W_next, c->W_next ? (size_t)pn.NC * pn.P * e : 0);
  const Span Wrn = span(c->W_next && pn.R ? c->W_route_next : nullptr, (size_t)pn.NC * pn.N * e);
  const Span X = span(a->X, T * p.NC * e), Xn = span(a->X_new, T * p.NC * e);
  const Span out = span(a->out, T * p.C * e), hin = span(a->h_in, T * p.C * e);
  const Span W = span(a->W, a->W ? (size_t)p.NC * p.P * e : 0);
  const Span bias = span(a->bias, a->bias ? (size_t)p.P * 4 : 0);
  const Span w4 = span(a->w4, a->w4 ? (size_t)p.C * 16 : 0), w8 = span(a->w8, a->w8 ? (size_t)p.C * 32 : 0),
             w12 = span(a->w12, a->w12 ? (size_t)p.C * 48 : 0);
  const Span zs = span(a->z_save, a->z_save ? T * p.zsv * 4 : 0);
  const Span xs = span(a->xact_save, a->xact_save ? T * p.k * p.C * e : 0);
  const Span ri = span(p.pt ? a->route_idx : nullptr, T * p.k * 4);
  const Span outs[] = {Xn, hin, zs, xs, p.R ? ri : Span{nullptr, 0}};
  const Span ins[] = {X, out, W, bias, w4, w8, w12, p.R ? Span{nullptr, 0} : ri};
  // carry_out: an output (carry_in identical to it is permitted)
  if (c->carry_out) {
    for (const Span& o : outs)
      if (overlap(cout, o)) return XHC_ERR_ALIAS;
    for (const Span& i : ins)
      if (overlap(cout, i)) return XHC_ERR_ALIAS;
    if (overlap(cout, Wn) || overlap(cout, Wrn)) return XHC_ERR_ALIAS;
    if (c->carry_in && c->carry_in != c->carry_out && overlap(cout, cin)) return XHC_ERR_ALIAS;
  }
  // carry_in and W_next: inputs, no overlap with the call's outputs
  for (const Span& o : outs) {
    if (overlap(cin, o)) return XHC_ERR_ALIAS;
    if (overlap(Wn, o) || overlap(Wrn, o)) return XHC_ERR_ALIAS;
  }
  return XHC_OK;
}

// Split forward (xhc_forward_pre / xhc_forward_post): pn is the next
// sublayer's plan (== p without desc_next).
static int check_split_modes(const Plan& p, const Plan& pn, bool carried) {
  // per-token lists: the carried partials would need each token's own rows
  if (carried && (p.pt || pn.pt)) return XHC_ERR_UNSUPPORTED;
  // the carried partials sum every stream of a channel block
  if (carried && (p.hact || pn.hact)) return XHC_ERR_UNSUPPORTED;
  if (pn.B != p.B || pn.S != p.S || pn.C != p.C || pn.N != p.N || pn.dtype != p.dtype) return XHC_ERR_SHAPE;
  return XHC_OK;
}

static int validate_pre(const Plan& p, const Plan& pn, const xhc_pre_args* a) {
  if (!a) return XHC_ERR_NULL;
  int rc = check_split_modes(p, pn, a->carry_in || a->W_next);
  if (rc) return rc;
  if (!a->X || !a->h_in || !a->z_save || (!a->carry_in && !a->W)) return XHC_ERR_NULL;
  if ((a->W_next == nullptr) != (a->carry_out == nullptr)) return XHC_ERR_NULL;
  if (p.R && !a->W_route) return XHC_ERR_NULL;
  if (p.pt && !a->route_idx) return XHC_ERR_NULL;
  rc = check_active(p, a->active);
  if (rc) return rc;
  const void* ptrs[] = {a->X, a->W, a->bias, a->h_in, a->z_save, a->carry_in, a->W_next, a->carry_out,
                        p.R ? a->W_route : nullptr, p.R ? a->b_route : nullptr, p.pt ? a->route_idx : nullptr,
                        p.pt && !p.R ? a->status : nullptr};
  for (const void* q : ptrs)
    if (misaligned(q)) return XHC_ERR_ALIGN;
  const size_t T = p.T, e = p.esz;
  const Span X = span(a->X, T * p.NC * e), hin = span(a->h_in, T * p.C * e);
  const Span W = span(a->W, a->W && !a->carry_in ? (size_t)p.NC * p.P * e : 0);
  const Span bias = span(a->bias, a->bias ? (size_t)p.P * 4 : 0);
  const Span zs = span(a->z_save, T * p.zsv * 4);
  const Span cin = span(a->carry_in, a->carry_in ? p.carry_bytes : 0);
  const Span Wn = span(a->W_next, a->W_next ? (size_t)pn.NC * pn.P * e : 0);
  const Span cout = span(a->carry_out, a->carry_out ? pn.carry_bytes : 0);
  // carry_out may be carry_in itself: the coefficients consume it first
  const Span cout_chk = (a->carry_out && a->carry_out == a->carry_in) ? Span{nullptr, 0} : cout;
  const Span Wr = span(p.R ? a->W_route : nullptr, (size_t)p.NC * p.N * e);
  const Span br = span(p.R ? a->b_route : nullptr, (size_t)p.N * 4);
  const Span ri = span(p.pt ? a->route_idx : nullptr, T * p.k * 4);
  const Span stw = span(p.pt && !p.R ? a->status : nullptr, 8);
  std::vector<Span> outs = {hin, zs, cout_chk, stw};
  std::vector<Span> ins = {X, W, bias, cin, Wn, Wr, br};
  (p.R ? outs : ins).push_back(ri);            // the router writes the lists; given lists are read
  if (any_overlap(outs, ins, Span{nullptr, 0}, Span{nullptr, 0})) return XHC_ERR_ALIAS;
  if (a->carry_out && a->carry_out == a->carry_in) {
    for (const Span& o : {hin, zs})
      if (overlap(cout, o)) return XHC_ERR_ALIAS;
    for (const Span& i : {X, W, bias, Wn})
      if (overlap(cout, i)) return XHC_ERR_ALIAS;
  }
  return XHC_OK;
}

static int validate_post(const Plan& p, const Plan& pn, const xhc_post_args* a) {
  if (!a) return XHC_ERR_NULL;
  int rc = check_split_modes(p, pn, a->W_next != nullptr);
  if (rc) return rc;
  if (!a->X || !a->out || !a->z_save) return XHC_ERR_NULL;
  if (p.nc == 4 && (!a->w4 || !a->w8 || !a->w12)) return XHC_ERR_NULL;
  if (p.nc == 1 && (a->w4 || a->w8 || a->w12)) return XHC_ERR_UNSUPPORTED;
  if ((a->W_next == nullptr) != (a->carry_out == nullptr)) return XHC_ERR_NULL;
  if (p.pt && !a->route_idx) return XHC_ERR_NULL;
  rc = check_active(p, a->active);
  if (rc) return rc;
  const void* ptrs[] = {a->X, a->out, a->w4, a->w8, a->w12, a->z_save, a->xact_save, a->W_next, a->carry_out,
                        p.pt ? a->route_idx : nullptr};
  for (const void* q : ptrs)
    if (misaligned(q)) return XHC_ERR_ALIGN;
  const size_t T = p.T, e = p.esz;
  const Span X = span(a->X, T * p.NC * e), out = span(a->out, T * p.C * e);
  const Span w4 = span(a->w4, a->w4 ? (size_t)p.C * 16 : 0), w8 = span(a->w8, a->w8 ? (size_t)p.C * 32 : 0),
             w12 = span(a->w12, a->w12 ? (size_t)p.C * 48 : 0);
  const Span zs = span(a->z_save, T * p.zsv * 4);
  const Span xs = span(a->xact_save, a->xact_save ? T * p.k * p.C * e : 0);
  const Span Wn = span(a->W_next, a->W_next ? (size_t)pn.NC * pn.P * e : 0);
  const Span cout = span(a->carry_out, a->carry_out ? pn.carry_bytes : 0);
  const Span ri = span(p.pt ? a->route_idx : nullptr, T * p.k * 4);
  std::vector<Span> outs = {X, xs, cout};
  std::vector<Span> ins = {out, w4, w8, w12, zs, Wn, ri};
  if (any_overlap(outs, ins, Span{nullptr, 0}, Span{nullptr, 0})) return XHC_ERR_ALIAS;
  return XHC_OK;
}

static int validate_bwd(const Plan& p, const xhc_bwd_args* a) {
  if (!a) return XHC_ERR_NULL;
  if (!a->X || !a->out || !a->W || !a->dX_new || !a->dh_in || !a->dX || !a->dout || !a->dW) return XHC_ERR_NULL;
  if (p.nc == 4 && (!a->w4 || !a->w8 || !a->w12 || !a->dw4 || !a->dw8 || !a->dw12)) return XHC_ERR_NULL;
  if (p.nc == 1 && (a->w4 || a->w8 || a->w12 || a->dw4 || a->dw8 || a->dw12)) return XHC_ERR_UNSUPPORTED;
  if (a->accumulate != 0 && a->accumulate != 1) return XHC_ERR_UNSUPPORTED;
  if (p.R) {
    // the router's choice and scores come from the forward's records
    if (!a->route_idx || !a->W_route || !a->dW_route) return XHC_ERR_NULL;
    // recomputing the scores needs the forward's b_route: a NULL here would
    // silently stand for zero while the forward may have used another value
    if (!a->z_save && !a->b_route) return XHC_ERR_NULL;
  }
  if (p.pt && !a->route_idx) return XHC_ERR_NULL;
  // recomputing the logits maps saved rows by the host list: not per token
  if (p.pt && a->xact && !a->z_save) return XHC_ERR_UNSUPPORTED;
  int rc = check_active(p, a->active);
  if (rc) return rc;
  const void* ptrs[] = {a->X, a->xact, a->out, a->w4, a->w8, a->w12, a->W, a->bias, a->z_save, a->dX_new,
                        a->dh_in, a->dX, a->dout, a->dW, a->db, a->dw4, a->dw8, a->dw12,
                        p.R ? a->W_route : nullptr, p.pt ? a->route_idx : nullptr,
                        p.R ? a->dW_route : nullptr, p.R ? a->db_route : nullptr,
                        p.R ? a->b_route : nullptr, p.pt ? a->status : nullptr};
  for (const void* q : ptrs)
    if (misaligned(q)) return XHC_ERR_ALIGN;
  const size_t T = p.T, e = p.esz;
  const Span X = span(a->X, T * p.NC * e), xact = span(a->xact, a->xact ? T * p.k * p.C * e : 0);
  const Span out = span(a->out, T * p.C * e), W = span(a->W, (size_t)p.NC * p.P * e);
  const Span bias = span(a->bias, a->bias ? (size_t)p.P * 4 : 0);
  const Span w4 = span(a->w4, a->w4 ? (size_t)p.C * 16 : 0), w8 = span(a->w8, a->w8 ? (size_t)p.C * 32 : 0),
             w12 = span(a->w12, a->w12 ? (size_t)p.C * 48 : 0);
  const Span zs = span(a->z_save, a->z_save ? T * p.zsv * 4 : 0);
  const Span Wr = span(p.R ? a->W_route : nullptr, (size_t)p.NC * p.N * e);
  const Span ri = span(p.pt ? a->route_idx : nullptr, T * p.k * 4);
  const Span dWr = span(p.R ? a->dW_route : nullptr, (size_t)p.NC * p.N * 4);
  const Span dbr = span(p.R ? a->db_route : nullptr, (size_t)p.N * 4);
  const Span dXn = span(a->dX_new, T * p.NC * e), dhin = span(a->dh_in, T * p.C * e);
  const Span dX = span(a->dX, T * p.NC * e), dout = span(a->dout, T * p.C * e);
  const Span dW = span(a->dW, (size_t)p.NC * p.P * 4), db = span(a->db, a->db ? (size_t)p.P * 4 : 0);
  const Span dw4 = span(a->dw4, a->dw4 ? (size_t)p.C * 16 : 0), dw8 = span(a->dw8, a->dw8 ? (size_t)p.C * 32 : 0),
             dw12 = span(a->dw12, a->dw12 ? (size_t)p.C * 48 : 0);
  if (a->dX != a->dX_new && overlap(dX, dXn)) return XHC_ERR_ALIAS;
  const Span stw = span(p.pt ? a->status : nullptr, 8);
  std::vector<Span> outs = {dX, dout, dW, db, dw4, dw8, dw12, dWr, dbr, stw};
  const Span br = span(p.R ? a->b_route : nullptr, (size_t)p.N * 4);
  std::vector<Span> ins = {X, xact, out, W, bias, w4, w8, w12, zs, dXn, dhin, Wr, ri, br};
  if (any_overlap(outs, ins, dX, dXn)) return XHC_ERR_ALIAS;
  return XHC_OK;
}

// Split backward (xhc_backward_post / xhc_backward_pre).
static int check_split_bwd_modes(const Plan& p, int accumulate) {
  (void)p;
  if (accumulate != 0 && accumulate != 1) return XHC_ERR_UNSUPPORTED;
  return XHC_OK;
}

static int validate_bwd_post(const Plan& p, const xhc_bwd_post_args* a) {
  if (!a) return XHC_ERR_NULL;
  int rc = check_split_bwd_modes(p, a->accumulate);
  if (rc) return rc;
  if (!a->out || !a->z_save || !a->dX_new || !a->dout || !a->bwd_state) return XHC_ERR_NULL;
  if (p.nc == 4 && (!a->w4 || !a->w8 || !a->w12 || !a->dw4 || !a->dw8 || !a->dw12)) return XHC_ERR_NULL;
  if (p.nc == 1 && (a->w4 || a->w8 || a->w12 || a->dw4 || a->dw8 || a->dw12)) return XHC_ERR_UNSUPPORTED;
  if (p.pt && !a->route_idx) return XHC_ERR_NULL;
  rc = check_active(p, a->active);
  if (rc) return rc;
  const void* ptrs[] = {a->out, a->w4, a->w8, a->w12, a->z_save, a->dX_new, a->dout, a->dw4, a->dw8, a->dw12,
                        a->bwd_state, p.pt ? a->route_idx : nullptr, p.pt ? a->status : nullptr};
  for (const void* q : ptrs)
    if (misaligned(q)) return XHC_ERR_ALIGN;
  const size_t T = p.T, e = p.esz;
  const Span out = span(a->out, T * p.C * e);
  const Span w4 = span(a->w4, a->w4 ? (size_t)p.C * 16 : 0), w8 = span(a->w8, a->w8 ? (size_t)p.C * 32 : 0),
             w12 = span(a->w12, a->w12 ? (size_t)p.C * 48 : 0);
  const Span zs = span(a->z_save, T * p.zsv * 4);
  const Span dXn = span(a->dX_new, T * p.NC * e), dout = span(a->dout, T * p.C * e);
  const Span dw4 = span(a->dw4, a->dw4 ? (size_t)p.C * 16 : 0), dw8 = span(a->dw8, a->dw8 ? (size_t)p.C * 32 : 0),
             dw12 = span(a->dw12, a->dw12 ? (size_t)p.C * 48 : 0);
  const Span st = span(a->bwd_state, p.state_bytes);
  const Span ri = span(p.pt ? a->route_idx : nullptr, T * p.k * 4);
  const Span stw = span(p.pt ? a->status : nullptr, 8);
  std::vector<Span> outs = {dout, dw4, dw8, dw12, st, stw};
  std::vector<Span> ins = {out, w4, w8, w12, zs, dXn, ri};
  if (any_overlap(outs, ins, Span{nullptr, 0}, Span{nullptr, 0})) return XHC_ERR_ALIAS;
  return XHC_OK;
}

static int validate_bwd_pre(const Plan& p, const xhc_bwd_pre_args* a) {
  if (!a) return XHC_ERR_NULL;
  int rc = check_split_bwd_modes(p, a->accumulate);
  if (rc) return rc;
  if (!a->X || !a->W || !a->z_save || !a->dX_new || !a->dh_in || !a->bwd_state || !a->dX || !a->dW)
    return XHC_ERR_NULL;
  if (p.R && (!a->W_route || !a->dW_route)) return XHC_ERR_NULL;
  if (p.pt && !a->route_idx) return XHC_ERR_NULL;
  rc = check_active(p, a->active);
  if (rc) return rc;
  const void* ptrs[] = {a->X, a->xact, a->W, a->bias, a->z_save, a->dX_new, a->dh_in, a->bwd_state, a->dX, a->dW,
                        a->db, p.R ? a->W_route : nullptr, p.pt ? a->route_idx : nullptr,
                        p.R ? a->dW_route : nullptr, p.R ? a->db_route : nullptr};
  for (const void* q : ptrs)
    if (misaligned(q)) return XHC_ERR_ALIGN;
  const size_t T = p.T, e = p.esz;
  const Span X = span(a->X, T * p.NC * e), xact = span(a->xact, a->xact ? T * p.k * p.C * e : 0);
  const Span W = span(a->W, (size_t)p.NC * p.P * e), bias = span(a->bias, a->bias ? (size_t)p.P * 4 : 0);
  const Span zs = span(a->z_save, T * p.zsv * 4), st = span(a->bwd_state, p.state_bytes);
  const Span dXn = span(a->dX_new, T * p.NC * e), dhin = span(a->dh_in, T * p.C * e);
  const Span dX = span(a->dX, T * p.NC * e);
  const Span dW = span(a->dW, (size_t)p.NC * p.P * 4), db = span(a->db, a->db ? (size_t)p.P * 4 : 0);
  if (a->dX != a->dX_new && overlap(dX, dXn)) return XHC_ERR_ALIAS;
  const Span Wr = span(p.R ? a->W_route : nullptr, (size_t)p.NC * p.N * e);
  const Span ri = span(p.pt ? a->route_idx : nullptr, T * p.k * 4);
  const Span dWr = span(p.R ? a->dW_route : nullptr, (size_t)p.NC * p.N * 4);
  const Span dbr = span(p.R ? a->db_route : nullptr, (size_t)p.N * 4);
  std::vector<Span> outs = {dX, dW, db, dWr, dbr};
  std::vector<Span> ins = {X, xact, W, bias, zs, dXn, dhin, st, Wr, ri};
  if (any_overlap(outs, ins, dX, dXn)) return XHC_ERR_ALIAS;
  return XHC_OK;
}

int prepare_forward(const xhc_desc* d, const xhc_fwd_args* a, Plan* p) {
  int rc = make_plan(d, p);
  if (rc) return rc;
  return validate_fwd(*p, a);
}

}  // namespace xhc

// ---------------------------------------------------------------------------
// timer
// ---------------------------------------------------------------------------
struct xhc_timer {
  struct Rec { int kid; hipEvent_t start, stop; };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  hipEvent_t get() {
    if (used == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};

static const char* const kKernelNames[xhc::KID_COUNT] = {
    "pack_wt", "proj", "coef", "mix", "pack_wp", "bdots", "bcoef", "bgrad", "breduce", "bxdots", "mixproj", "gram",
    "bdots_gs", "route_colsum", "route_pass", "route_dwr", "check_lists", "bwd_prep"};

namespace xhc {
void timer_mark(xhc_timer* tm, int kid, hipStream_t st, bool start) {
  hipEvent_t e = tm->get();
  if (!e) return;
  hipEventRecord(e, st);
  if (start) {
    tm->recs.push_back({kid, e, nullptr});
  } else {
    for (size_t i = tm->recs.size(); i-- > 0;)
      if (tm->recs[i].kid == kid && tm->recs[i].stop == nullptr) { tm->recs[i].stop = e; break; }
  }
}
}  // namespace xhc

extern "C" {

size_t xhc_workspace_size(const xhc_desc* desc, int phase) {
  xhc::Plan p;
  if (xhc::make_plan(desc, &p) != XHC_OK) return 0;
  if (phase == XHC_PHASE_FWD) return p.fwd_bytes;
  if (phase == XHC_PHASE_BWD) return p.bwd_bytes;
  return 0;
}

size_t xhc_bwd_state_size(const xhc_desc* desc) {
  xhc::Plan p;
  if (xhc::make_plan(desc, &p) != XHC_OK) return 0;
  return p.state_bytes;
}

// The next sublayer's plan of a split call (== p without desc_next).
static int next_plan(const xhc::Plan& p, const xhc_desc* desc_next, xhc::Plan* pn) {
  *pn = p;
  if (!desc_next) return XHC_OK;
  const int rc = xhc::make_plan(desc_next, pn);
  return rc ? XHC_ERR_SHAPE : XHC_OK;
}

int xhc_validate(const xhc_desc* desc, const void* args, int phase) {
  xhc::Plan p;
  int rc = xhc::make_plan(desc, &p);
  if (rc) return rc;
  if (phase == XHC_PHASE_FWD) return xhc::validate_fwd(p, static_cast<const xhc_fwd_args*>(args));
  if (phase == XHC_PHASE_BWD) return xhc::validate_bwd(p, static_cast<const xhc_bwd_args*>(args));
  if (phase == XHC_PHASE_BWD_POST) return xhc::validate_bwd_post(p, static_cast<const xhc_bwd_post_args*>(args));
  if (phase == XHC_PHASE_BWD_PRE) return xhc::validate_bwd_pre(p, static_cast<const xhc_bwd_pre_args*>(args));
  if (phase == XHC_PHASE_PRE || phase == XHC_PHASE_POST) {
    if (!args) return XHC_ERR_NULL;
    const xhc_desc* dn = phase == XHC_PHASE_PRE ? static_cast<const xhc_pre_args*>(args)->desc_next
                                                : static_cast<const xhc_post_args*>(args)->desc_next;
    xhc::Plan pn;
    rc = next_plan(p, dn, &pn);
    if (rc) return rc;
    return phase == XHC_PHASE_PRE ? xhc::validate_pre(p, pn, static_cast<const xhc_pre_args*>(args))
                                  : xhc::validate_post(p, pn, static_cast<const xhc_post_args*>(args));
  }
  return XHC_ERR_UNSUPPORTED;
}

// The launchers report a failed launch through hipGetLastError(), which
// returns the last error of ANY HIP call made on the calling thread.  Other
// code on that thread (a framework probing pointer attributes, say) may
// leave an error pending that it chose to ignore; clear it before this
// call's launches so that only their errors are reported as XHC_ERR_HIP.
static void clear_pending_hip_error() { (void)hipGetLastError(); }

static int check_ws(const xhc::Plan& p, void* ws, size_t bytes, size_t need) {
  (void)p;
  if (!ws) return XHC_ERR_WORKSPACE;
  if (bytes < need) return XHC_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return XHC_ERR_ALIGN;
  return XHC_OK;
}

int xhc_forward(const xhc_desc* desc, const xhc_fwd_args* args, void* workspace, size_t workspace_bytes,
                xhc_stream_t stream) {
  xhc::Plan p;
  int rc = xhc::make_plan(desc, &p);
  if (rc) return rc;
  rc = xhc::validate_fwd(p, args);
  if (rc) return rc;
  rc = check_ws(p, workspace, workspace_bytes, p.fwd_bytes);
  if (rc) return rc;
  clear_pending_hip_error();
  return xhc::launch_forward(p, args, workspace, reinterpret_cast<hipStream_t>(stream));
}

int32_t xhc_zsave_stride(const xhc_desc* desc) {
  xhc::Plan p;
  if (xhc::make_plan(desc, &p) != XHC_OK) return 0;
  return p.zsv;
}

size_t xhc_carry_size(const xhc_desc* desc) {
  xhc::Plan p;
  if (xhc::make_plan(desc, &p) != XHC_OK) return 0;
  return p.carry_bytes;
}

int xhc_forward_chain(const xhc_desc* desc, const xhc_fwd_args* args, const xhc_chain_args* chain, void* workspace,
                      size_t workspace_bytes, xhc_stream_t stream) {
  xhc::Plan p;
  int rc = xhc::make_plan(desc, &p);
  if (rc) return rc;
  rc = xhc::validate_fwd(p, args, !(chain && chain->carry_in));
  if (rc) return rc;
  xhc::Plan pn = p;
  if (chain && chain->desc_next) {
    rc = xhc::make_plan(chain->desc_next, &pn);
    if (rc) return rc;
  }
  rc = xhc::validate_chain(p, pn, args, chain);
  if (rc) return rc;
  rc = check_ws(p, workspace, workspace_bytes, p.fwd_bytes);
  if (rc) return rc;
  clear_pending_hip_error();
  return xhc::launch_forward_chain(p, pn, args, chain, workspace, reinterpret_cast<hipStream_t>(stream));
}

int xhc_forward_pre(const xhc_desc* desc, const xhc_pre_args* args, void* workspace, size_t workspace_bytes,
                    xhc_stream_t stream) {
  xhc::Plan p, pn;
  int rc = xhc::make_plan(desc, &p);
  if (rc) return rc;
  if (!args) return XHC_ERR_NULL;
  rc = next_plan(p, args->desc_next, &pn);
  if (rc) return rc;
  rc = xhc::validate_pre(p, pn, args);
  if (rc) return rc;
  rc = check_ws(p, workspace, workspace_bytes, p.fwd_bytes);
  if (rc) return rc;
  clear_pending_hip_error();
  return xhc::launch_forward_pre(p, pn, args, workspace, reinterpret_cast<hipStream_t>(stream));
}

int xhc_forward_post(const xhc_desc* desc, const xhc_post_args* args, void* workspace, size_t workspace_bytes,
                     xhc_stream_t stream) {
  xhc::Plan p, pn;
  int rc = xhc::make_plan(desc, &p);
  if (rc) return rc;
  if (!args) return XHC_ERR_NULL;
  rc = next_plan(p, args->desc_next, &pn);
  if (rc) return rc;
  rc = xhc::validate_post(p, pn, args);
  if (rc) return rc;
  rc = check_ws(p, workspace, workspace_bytes, p.fwd_bytes);
  if (rc) return rc;
  clear_pending_hip_error();
  return xhc::launch_forward_post(p, pn, args, workspace, reinterpret_cast<hipStream_t>(stream));
}

int xhc_backward(const xhc_desc* desc, const xhc_bwd_args* args, void* workspace, size_t workspace_bytes,
                 xhc_stream_t stream) {
  xhc::Plan p;
  int rc = xhc::make_plan(desc, &p);
  if (rc) return rc;
  rc = xhc::validate_bwd(p, args);
  if (rc) return rc;
  rc = check_ws(p, workspace, workspace_bytes, p.bwd_bytes);
  if (rc) return rc;
  clear_pending_hip_error();
  return xhc::launch_backward(p, args, workspace, reinterpret_cast<hipStream_t>(stream));
}

int xhc_backward_post(const xhc_desc* desc, const xhc_bwd_post_args* args, void* workspace, size_t workspace_bytes,
                      xhc_stream_t stream) {
  xhc::Plan p;
  int rc = xhc::make_plan(desc, &p);
  if (rc) return rc;
  rc = xhc::validate_bwd_post(p, args);
  if (rc) return rc;
  rc = check_ws(p, workspace, workspace_bytes, p.bwd_bytes);
  if (rc) return rc;
  clear_pending_hip_error();
  return xhc::launch_backward_post(p, args, workspace, reinterpret_cast<hipStream_t>(stream));
}

int xhc_backward_pre(const xhc_desc* desc, const xhc_bwd_pre_args* args, void* workspace, size_t workspace_bytes,
                     xhc_stream_t stream) {
  xhc::Plan p;
  int rc = xhc::make_plan(desc, &p);
  if (rc) return rc;
  rc = xhc::validate_bwd_pre(p, args);
  if (rc) return rc;
  rc = check_ws(p, workspace, workspace_bytes, p.bwd_bytes);
  if (rc) return rc;
  clear_pending_hip_error();
  return xhc::launch_backward_pre(p, args, workspace, reinterpret_cast<hipStream_t>(stream));
}

const char* xhc_strerror(int code) {
  switch (code) {
    case XHC_OK: return "ok";
    case XHC_ERR_NULL: return "a required pointer is NULL";
    case XHC_ERR_SHAPE: return "sizes out of the supported range";
    case XHC_ERR_INDEX: return "active stream index out of range or repeated";
    case XHC_ERR_ALIAS: return "forbidden overlap between buffers";
    case XHC_ERR_ALIGN: return "pointer not aligned (16 bytes; workspace 256 bytes)";
    case XHC_ERR_UNSUPPORTED: return "mode not supported";
    case XHC_ERR_WORKSPACE: return "workspace missing or too small";
    case XHC_ERR_HIP: return "HIP call or kernel launch failed";
    case XHC_ERR_SCRATCH: return "problem needs more scratch than the library's static buffer holds";
    default: return "unknown xhc error";
  }
}

xhc_timer* xhc_timer_create(void) { return new xhc_timer(); }

void xhc_timer_destroy(xhc_timer* t) {
  if (!t) return;
  for (hipEvent_t e : t->pool) hipEventDestroy(e);
  delete t;
}

void xhc_timer_reset(xhc_timer* t) {
  if (!t) return;
  t->recs.clear();
  t->used = 0;
}

int xhc_timer_read(xhc_timer* t, const char* kernel, double* total_ms, int64_t* launches) {
  if (!t || !kernel || !total_ms || !launches) return XHC_ERR_NULL;
  int kid = -1;
  for (int i = 0; i < xhc::KID_COUNT; ++i)
    if (std::strcmp(kernel, kKernelNames[i]) == 0) kid = i;
  if (kid < 0) return XHC_ERR_UNSUPPORTED;
  double ms = 0.0;
  int64_t n = 0;
  for (const auto& r : t->recs) {
    if (r.kid != kid || !r.stop) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return XHC_ERR_HIP;
    float f = 0.f;
    if (hipEventElapsedTime(&f, r.start, r.stop) != hipSuccess) return XHC_ERR_HIP;
    ms += f;
    ++n;
  }
  *total_ms = ms;
  *launches = n;
  return XHC_OK;
}

int xhc_kernel_count(void) { return xhc::KID_COUNT; }

const char* xhc_kernel_name(int i) { return (i >= 0 && i < xhc::KID_COUNT) ? kKernelNames[i] : nullptr; }

}  // extern "C"

// Forward kernels of the xHC sublayer update (gfx950).
//
// Sources: "xHC: Expanded Hyper-Connections" research retrospective
// (qingkeai.online), sections "把 N 调大以后，事情开始不太对了" (state, roles
// of H_pre/H_post/H_res, Sinkhorn), "最便宜的新信息，可能就在相邻 token 里"
// (TFA: causal depthwise convolutions, K = 4, 8, 12) and "模型可以拥有 16 条
// streams，但每层只更新 4 条" (dense read, sparse write, write formula).
//
// Pipeline of one forward call (all on the caller's stream):
//   k_pack_wt  W [N*C, P] -> Wt [16*NT, N*C]: K-contiguous B operand
//   k_proj     per (stream, 64-token tile): partial x.W (MFMA) and sum x^2
//   k_coef     per token: reduce partials, r, z, gates, Sinkhorn (registers)
//   k_mix      per (sequence segment, channel block): dense read h_in, TFA
//              over a 12-row causal window, sparse write of the k rows
#include "xhc_device.h"
#include "xhc_launch.h"

namespace xhc {

// ---------------------------------------------------------------------------
// W [NC, P] (row j = i*C + c) -> Wt [NTP, NC], rows p >= P zero.
// ---------------------------------------------------------------------------
template <typename R>
__global__ void k_pack_wt(const R* __restrict__ W, R* __restrict__ Wt, int64_t NC, int P, int NTP) {
  int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= NC) return;
  for (int p = 0; p < NTP; ++p) Wt[(size_t)p * NC + j] = p < P ? W[(size_t)j * P + p] : R(0);
}

// ---------------------------------------------------------------------------
// Projection partials.  Workgroup = (stream `split`, tile of 64 tokens);
// wave w owns tokens tile*64 + 16w .. +16 as MFMA rows; columns are the NT
// 16-wide logit tiles.  The K loop runs over the stream's C channels in
// steps of 32 (lane group g = lane/16 holds K elements 8g..8g+8 of a step).
// Stream rows come from `src` (the state, or after an in-place forward the
// saved active rows for the active streams).
// Output zpart[split][t][0..16NT) = sum_c X[t,split,c] W[split*C+c, p],
//        zpart[split][t][16NT]    = sum_c X[t,split,c]^2.
// ---------------------------------------------------------------------------
template <typename E, int NT>
__global__ __launch_bounds__(256) void k_proj(StreamRows src, const void* __restrict__ Wt,
                                              float* __restrict__ zpart, int T, int C, int64_t NC,
                                              int ZST, int ntiles) {
  constexpr int U = 4;
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int split = lb / ntiles;
  const int tile = lb - split * ntiles;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int t = tile * PROJ_TOK + wave * 16 + r;
  const bool tv = t < T;
  const void* X = src.base[split];
  const size_t xrow = (size_t)(tv ? t : 0) * src.stride[split];
  const size_t wcol = (size_t)split * C;

  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;

  const int nks = (C + 31) >> 5;
  for (int ks = 0; ks < nks; ks += U) {
    V8<E> a[U], b[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = (ks + u) * 32 + 8 * g;
      const bool kv = (ks + u) < nks && kb < C;
      a[u] = (kv && tv) ? V8<E>::load(X, xrow + kb) : V8<E>::zero();
#pragma unroll
      for (int n = 0; n < NT; ++n)
        b[u][n] = kv ? V8<E>::load(Wt, (size_t)(16 * n + r) * NC + wcol + kb) : V8<E>::zero();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int j = 0; j < 8; ++j) { const float v = a[u].f(j); ss = fmaf(v, v, ss); }
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = mma32(a[u], b[u][n], acc[n]);
    }
  }
  ss += shfl_xor(ss, 16);
  ss += shfl_xor(ss, 32);

  float* zp = zpart + (size_t)split * T * ZST;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int tt = tile * PROJ_TOK + wave * 16 + 4 * g + e;     // D row 4g+e
    if (tt < T) {
#pragma unroll
      for (int n = 0; n < NT; ++n) zp[(size_t)tt * ZST + 16 * n + r] = acc[n][e];
    }
  }
  if (g == 0 && tv) zp[(size_t)t * ZST + 16 * NT] = ss;
}

// ---------------------------------------------------------------------------
// Coefficients.  16 lanes per token; lane e owns logit columns e, e+16, e+32
// and entry (a, b) = (e/4, e%4) of the k x k Sinkhorn matrix, whose row sums
// are quad reductions (xor 1, 2) and column sums xor 4, 8 reductions.
// Either reduces projection partials (zpart != NULL) or reloads z and r from
// z_in (a forward's z_save).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_coef(const float* __restrict__ zpart, int SK, int ZST, int NTP,
                                              const float* __restrict__ z_in, const float* __restrict__ bias,
                                              float* __restrict__ coef, float* __restrict__ z_out, int T,
                                              int N, int k, int nc, int P, float inv_nc_total, float eps,
                                              int iters, int unit_gates) {
  __shared__ float zs[16][COEF_STRIDE];
  const int e = threadIdx.x & 15, tok = threadIdx.x >> 4;
  const int t = blockIdx.x * 16 + tok;
  const bool tv = t < T;
  float r = 0.f;
  if (zpart) {
    float ss = (tv && e < SK) ? zpart[((size_t)e * T + t) * ZST + NTP] : 0.f;
    ss += shfl_xor(ss, 1);
    ss += shfl_xor(ss, 2);
    ss += shfl_xor(ss, 4);
    ss += shfl_xor(ss, 8);
    r = sqrtf(ss * inv_nc_total + eps);
#pragma unroll
    for (int n = 0; n < 3; ++n) {
      const int p = e + 16 * n;
      float z = 0.f;
      if (tv && p < P) {
        for (int s = 0; s < SK; ++s) z += zpart[((size_t)s * T + t) * ZST + p];
        z = z / r + (bias ? bias[p] : 0.f);
      }
      zs[tok][p] = z;
    }
  } else {
    r = tv ? z_in[(size_t)t * (P + 1) + P] : 1.f;
#pragma unroll
    for (int n = 0; n < 3; ++n) {
      const int p = e + 16 * n;
      zs[tok][p] = (tv && p < P) ? z_in[(size_t)t * (P + 1) + p] : 0.f;
    }
  }
  __syncthreads();
  if (!tv) return;
  float* co = coef + (size_t)t * COEF_STRIDE;

  // gates
  co[CO_PRE + e] = e < N ? (unit_gates ? 1.f : sigmoid(zs[tok][e])) : 0.f;
  {
    const int a = e >> 2, m = e & 3;
    co[CO_POST + e] = (a < k && m < nc) ? (unit_gates ? 1.f : sigmoid(zs[tok][N + a * nc + m])) : 0.f;
  }
  // Sinkhorn on the k x k res logits
  {
    const int a = e >> 2, b = e & 3;
    const bool valid = a < k && b < k;
    const float L = valid ? zs[tok][N + k * nc + a * k + b] : -INFINITY;
    float mx = fmaxf(L, shfl_xor(L, 1));
    mx = fmaxf(mx, shfl_xor(mx, 2));
    float M = valid ? expf(L - mx) : 0.f;
    for (int it = 0; it < iters; ++it) {
      float rs = M + shfl_xor(M, 1);
      rs += shfl_xor(rs, 2);
      M = valid ? M / rs : 0.f;
      float cs = M + shfl_xor(M, 4);
      cs += shfl_xor(cs, 8);
      M = valid ? M / cs : 0.f;
    }
    co[CO_RES + e] = M;
  }
  co[48 + e] = e == 0 ? r : 0.f;
  if (z_out) {
#pragma unroll
    for (int n = 0; n < 3; ++n) {
      const int p = e + 16 * n;
      if (p < P) z_out[(size_t)t * (P + 1) + p] = zs[tok][p];
    }
    if (e == 0) z_out[(size_t)t * (P + 1) + P] = r;
  }
}

// ---------------------------------------------------------------------------
// Dense read + TFA + sparse write.  Thread = MIX_CH consecutive channels of
// one sequence segment of MIX_LSEG tokens, swept in order.  The last 12 rows
// of `out` live in a register ring indexed by position mod 12 (segments start
// at multiples of 12, so the index is a compile-time constant in the
// 12-fold unrolled loop).  All reads of a token's rows happen before its
// writes, so X_new == X (in place) is safe.
// ---------------------------------------------------------------------------
struct Active { int id[4]; };

template <typename E, int NCOMP>
__global__ __launch_bounds__(MIX_THREADS) void k_mix(
    const void* __restrict__ X, const void* __restrict__ out, const float* __restrict__ w4,
    const float* __restrict__ w8, const float* __restrict__ w12, const float* __restrict__ coef,
    void* Xnew, void* __restrict__ hin, void* __restrict__ xact, int S, int C, int N, int k,
    Active act, int in_place, int segs_per_seq) {
  using V = Vec<E, MIX_CH>;
  const int c = (blockIdx.x * MIX_THREADS + threadIdx.x) * MIX_CH;
  const bool cv = c < C;
  const int seg = blockIdx.y;
  const int bseq = seg / segs_per_seq;
  const int s0 = (seg - bseq * segs_per_seq) * MIX_LSEG;
  const int s1 = min(s0 + MIX_LSEG, S);
  const size_t tok0 = (size_t)bseq * S;

  float wa[MIX_CH][4], wb[MIX_CH][8], wc[MIX_CH][12];
  if (NCOMP == 4) {
#pragma unroll
    for (int ch = 0; ch < MIX_CH; ++ch) {
      const int cc = cv ? c + ch : 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) wa[ch][q] = w4[(size_t)cc * 4 + q];
#pragma unroll
      for (int q = 0; q < 8; ++q) wb[ch][q] = w8[(size_t)cc * 8 + q];
#pragma unroll
      for (int q = 0; q < 12; ++q) wc[ch][q] = w12[(size_t)cc * 12 + q];
    }
  }

  float ring[12][MIX_CH];
#pragma unroll
  for (int j = 0; j < 12; ++j) {
    const int s = s0 - 12 + j;
    if (NCOMP == 4 && j > 0 && s >= 0 && cv) {
      V v = V::load(out, (tok0 + s) * C + c);
      v.to_float(ring[j]);
    } else {
#pragma unroll
      for (int ch = 0; ch < MIX_CH; ++ch) ring[j][ch] = 0.f;
    }
  }

  for (int g0 = s0; g0 < s1; g0 += 12) {
#pragma unroll
    for (int j = 0; j < 12; ++j) {
      const int s = g0 + j;
      if (s < s1) {
        const size_t t = tok0 + s;
        const float* co = coef + t * COEF_STRIDE;
        if (cv) {
          V ov = V::load(out, t * C + c);
          ov.to_float(ring[j]);
          float hacc[MIX_CH], o[4][MIX_CH], xa_keep[4][MIX_CH];
          V xa_raw[4];
#pragma unroll
          for (int ch = 0; ch < MIX_CH; ++ch) {
            hacc[ch] = 0.f;
#pragma unroll
            for (int a = 0; a < 4; ++a) o[a][ch] = 0.f;
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if (i < N) {
              V xv = V::load(X, (t * N + i) * C + c);
              float xf[MIX_CH];
              xv.to_float(xf);
              const float hp = co[CO_PRE + i];
#pragma unroll
              for (int ch = 0; ch < MIX_CH; ++ch) hacc[ch] = fmaf(hp, xf[ch], hacc[ch]);
#pragma unroll
              for (int b = 0; b < 4; ++b) {
                if (b < k && i == act.id[b]) {
                  xa_raw[b] = xv;
#pragma unroll
                  for (int ch = 0; ch < MIX_CH; ++ch) xa_keep[b][ch] = xf[ch];
                }
              }
              if (!in_place) {
                bool is_act = false;
#pragma unroll
                for (int b = 0; b < 4; ++b) is_act |= (b < k && i == act.id[b]);
                if (!is_act) xv.store(Xnew, (t * N + i) * C + c);
              }
            }
          }
          V::from_float(hacc).store(hin, t * C + c);

          // write-back components U_0..U_{NCOMP-1}
          float u[4][MIX_CH];
#pragma unroll
          for (int ch = 0; ch < MIX_CH; ++ch) {
            u[0][ch] = ring[j][ch];
            if (NCOMP == 4) {
              float s4 = 0.f, s8 = 0.f, s12 = 0.f;
#pragma unroll
              for (int q = 0; q < 4; ++q) s4 = fmaf(wa[ch][q], ring[(j + 12 - 3 + q) % 12][ch], s4);
#pragma unroll
              for (int q = 0; q < 8; ++q) s8 = fmaf(wb[ch][q], ring[(j + 12 - 7 + q) % 12][ch], s8);
#pragma unroll
              for (int q = 0; q < 12; ++q) s12 = fmaf(wc[ch][q], ring[(j + 12 - 11 + q) % 12][ch], s12);
              u[1][ch] = s4; u[2][ch] = s8; u[3][ch] = s12;
            }
          }
          // sparse write of the k active rows
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            if (a < k) {
              float res[MIX_CH];
#pragma unroll
              for (int ch = 0; ch < MIX_CH; ++ch) {
                float v = 0.f;
#pragma unroll
                for (int b = 0; b < 4; ++b)
                  if (b < k) v = fmaf(co[CO_RES + a * 4 + b], xa_keep[b][ch], v);
#pragma unroll
                for (int m = 0; m < NCOMP; ++m) v = fmaf(co[CO_POST + a * 4 + m], u[m][ch], v);
                res[ch] = v;
              }
              if (xact) xa_raw[a].store(xact, (t * k + a) * C + c);
              V::from_float(res).store(Xnew, (t * N + act.id[a]) * C + c);
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename R>
static void launch_pack_wt(const Plan& p, const void* W, void* Wt, hipStream_t st, xhc_timer* tm) {
  TimedLaunch tl(tm, KID_PACK_WT, st);
  const int nb = (int)((p.NC + 255) / 256);
  k_pack_wt<R><<<nb, 256, 0, st>>>(static_cast<const R*>(W), static_cast<R*>(Wt), p.NC, p.P, p.NT * 16);
}

template <typename E>
static void launch_proj(const Plan& p, const StreamRows& src, const void* Wt, float* zpart, hipStream_t st,
                        xhc_timer* tm) {
  TimedLaunch tl(tm, KID_PROJ, st);
  const int nb = p.proj_tiles * p.SK;
  if (p.NT == 1)
    k_proj<E, 1><<<nb, 256, 0, st>>>(src, Wt, zpart, p.T, p.C, p.NC, p.ZST, p.proj_tiles);
  else if (p.NT == 2)
    k_proj<E, 2><<<nb, 256, 0, st>>>(src, Wt, zpart, p.T, p.C, p.NC, p.ZST, p.proj_tiles);
  else
    k_proj<E, 3><<<nb, 256, 0, st>>>(src, Wt, zpart, p.T, p.C, p.NC, p.ZST, p.proj_tiles);
}

template <typename E, typename R>
static int forward_impl(const Plan& p, const xhc_fwd_args* a, char* ws, hipStream_t st, xhc_timer* tm) {
  void* Wt = ws + p.off_wt;
  float* zpart = reinterpret_cast<float*>(ws + p.off_zpart);
  float* coef = reinterpret_cast<float*>(ws + p.off_coef);
  const int NTP = p.NT * 16;
  (void)sizeof(R);

  launch_pack_wt<R>(p, a->W, Wt, st, tm);
  launch_proj<E>(p, stream_rows(p, a->X, nullptr, a->active), Wt, zpart, st, tm);
  {
    TimedLaunch tl(tm, KID_COEF, st);
    k_coef<<<(p.T + 15) / 16, 256, 0, st>>>(zpart, p.SK, p.ZST, NTP, nullptr, a->bias, coef, a->z_save,
                                            p.T, p.N, p.k, p.nc, p.P, 1.0f / (float)p.NC, p.eps,
                                            p.iters, p.gate == XHC_GATE_UNIT);
  }
  {
    TimedLaunch tl(tm, KID_MIX, st);
    Active act;
    for (int b = 0; b < 4; ++b) act.id[b] = b < p.k ? a->active[b] : -1;
    dim3 grid(p.mix_cblocks, p.B * p.mix_segs);
    const int in_place = a->X_new == a->X;
    if (p.nc == 4)
      k_mix<E, 4><<<grid, MIX_THREADS, 0, st>>>(a->X, a->out, a->w4, a->w8, a->w12, coef, a->X_new, a->h_in,
                                                a->xact_save, p.S, p.C, p.N, p.k, act, in_place, p.mix_segs);
    else
      k_mix<E, 1><<<grid, MIX_THREADS, 0, st>>>(a->X, a->out, nullptr, nullptr, nullptr, coef, a->X_new,
                                                a->h_in, a->xact_save, p.S, p.C, p.N, p.k, act, in_place,
                                                p.mix_segs);
  }
  return hipGetLastError() == hipSuccess ? XHC_OK : XHC_ERR_HIP;
}

int launch_forward(const Plan& p, const xhc_fwd_args* a, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  if (p.dtype == XHC_BF16) return forward_impl<BF16, uint16_t>(p, a, w, st, a->timer);
  return forward_impl<F32, float>(p, a, w, st, a->timer);
}

// Backward helper: coefficients either from a forward's z_save or, when it
// is NULL, recomputed by the projection from the pre-update state.
int launch_coef_bwd(const Plan& p, const void* X, const void* xact, const int32_t* active, const void* W,
                    const float* bias, const float* z_save, void* ws, float* coef, float* z_out,
                    hipStream_t st, xhc_timer* tm) {
  char* w = static_cast<char*>(ws);
  float* zpart = nullptr;
  if (!z_save) {
    void* Wt = w + p.off_wt;
    zpart = reinterpret_cast<float*>(w + p.off_zpart);
    const StreamRows src = stream_rows(p, X, xact, active);
    if (p.dtype == XHC_BF16) {
      launch_pack_wt<uint16_t>(p, W, Wt, st, tm);
      launch_proj<BF16>(p, src, Wt, zpart, st, tm);
    } else {
      launch_pack_wt<float>(p, W, Wt, st, tm);
      launch_proj<F32>(p, src, Wt, zpart, st, tm);
    }
  }
  TimedLaunch tl(tm, KID_COEF, st);
  k_coef<<<(p.T + 15) / 16, 256, 0, st>>>(zpart, p.SK, p.ZST, p.NT * 16, z_save, bias, coef, z_out, p.T,
                                          p.N, p.k, p.nc, p.P, 1.0f / (float)p.NC, p.eps, p.iters,
                                          p.gate == XHC_GATE_UNIT);
  return hipGetLastError() == hipSuccess ? XHC_OK : XHC_ERR_HIP;
}

}  // namespace xhc

// Router kernels of the xHC sublayer update (gfx950): the pieces of the
// routed forward and backward that the fixed-list kernels do not cover.
//
// Source: the "xHC: Expanded Hyper-Connections" retrospective, section
// "模型可以拥有 16 条 streams，但每层只更新 4 条" -- k active streams of
// which some are fixed and the rest chosen per token by a sigmoid router
// over the LayerNorm'd flattened state; a routed stream's write-back is
// scaled by its score, and the score's gradient flows only through that
// scale.  With y = (x - mean) / sd the router's logits are
//   rho = y.Wr + b = (x.Wr - mean * colsum(Wr)) / sd + b,
// so the projection pass forms x.Wr on MFMA next to the other logits (and
// sum(x) beside sum(x^2)), and only Wr's column sums are needed apart
// (k_route_colsum).
//
//   k_route_colsum  W_route [NC, N] -> partial column sums [RCS_BLK][16],
//                   then (k_route_colsum_fin) the column sums [16]
//   k_route_pass    (backward) pass[t][b] = sum_a H_res[a, b] G_a, the
//                   gradient that reaches active row b through the mixing
//                   term, for the dX assembly of rows chosen per token
//   k_route_dwr     (backward) dW_route from the dX pass's partials minus
//                   the LayerNorm mean's share
//   k_route_scale_post (split forward, second call) the routed slots' post
//                   coefficients of a record rebuilt from saved logits,
//                   scaled by the saved scores as the router scaled them
#include <algorithm>

#include "xhc_device.h"
#include "xhc_launch.h"

namespace xhc {

__device__ inline float elem_to_float(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ inline float elem_to_float(float v) { return v; }

// Block b sums rows [b*per, (b+1)*per) of every column (columns >= N give 0):
// thread (row lane tid/16, column tid%16) walks every 16th row of the range,
// then the 16 row lanes are summed in lane order (deterministic).
template <typename R>
__global__ __launch_bounds__(256) void k_route_colsum(const R* __restrict__ Wr, int64_t NC, int N,
                                                      float* __restrict__ rcs) {
  __shared__ float part[16][17];
  const int c = threadIdx.x & 15, rl = threadIdx.x >> 4;
  const int64_t per = (NC + RCS_BLK - 1) / RCS_BLK;
  const int64_t r0 = (int64_t)blockIdx.x * per;
  const int64_t r1 = r0 + per < NC ? r0 + per : NC;
  float s = 0.f;
  if (c < N)
    for (int64_t j = r0 + rl; j < r1; j += 16) s += elem_to_float(Wr[j * N + c]);
  part[rl][c] = s;
  __syncthreads();
  if (threadIdx.x < 16) {
    float a = 0.f;
    for (int q = 0; q < 16; ++q) a += part[q][threadIdx.x];
    rcs[blockIdx.x * 16 + threadIdx.x] = a;
  }
}

// rcs[RCS_BLK][i] (the partials) -> rcs[RCS_BLK * 16 + i], in block order.
__global__ __launch_bounds__(256) void k_route_colsum_fin(float* __restrict__ rcs) {
  __shared__ float part[16][17];
  const int c = threadIdx.x & 15, rl = threadIdx.x >> 4;
  float s = 0.f;
  for (int b = rl; b < RCS_BLK; b += 16) s += rcs[b * 16 + c];
  part[rl][c] = s;
  __syncthreads();
  if (threadIdx.x < 16) {
    float a = 0.f;
    for (int q = 0; q < 16; ++q) a += part[q][threadIdx.x];
    rcs[RCS_BLK * 16 + threadIdx.x] = a;
  }
}

void launch_route_colsum(const Plan& p, const void* W_route, float* rcs, hipStream_t st) {
  if (p.dtype == XHC_BF16)
    k_route_colsum<uint16_t><<<RCS_BLK, 256, 0, st>>>(static_cast<const uint16_t*>(W_route), p.NC, p.N, rcs);
  else
    k_route_colsum<float><<<RCS_BLK, 256, 0, st>>>(static_cast<const float*>(W_route), p.NC, p.N, rcs);
  k_route_colsum_fin<<<1, 256, 0, st>>>(rcs);
}

// pass[t][b][c] = sum_a H_res[a, b] dX_new[t, i_a, c] for b < k (storage
// type, [T][k][C]).  Workgroup = one token and a block of RP_CH channels
// (8 per thread), so the token's active list and H_res ([T][16], row a at
// 4a, from the coefficient backward) are uniform loads.
constexpr int RP_CH = 256 * 8;
template <typename E>
__global__ __launch_bounds__(256) void k_route_pass(const void* __restrict__ dXn, const int32_t* __restrict__ ridx,
                                                    const float* __restrict__ hres, void* __restrict__ pass,
                                                    int64_t T, int C, int N, int k, int ncb) {
  const int64_t t = blockIdx.x / ncb;
  const int c = (int)(blockIdx.x - t * ncb) * RP_CH + threadIdx.x * 8;
  if (c >= C) return;
  int id[4];
  float h[16];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int v = a < k ? ridx[t * k + a] : 0;
    id[a] = (unsigned)v < (unsigned)N ? v : 0;
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) h[e] = (e >> 2) < k && (e & 3) < k ? hres[t * 16 + e] : 0.f;
  float g[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a) V8<E>::load(dXn, (size_t)(t * N + id[a]) * C + c).to_float(g[a]);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b < k) {
      float o[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float v = 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a) v = fmaf(h[a * 4 + b], g[a][q], v);   // rows a >= k have H_res 0
        o[q] = v;
      }
      V8<E>::from_float(o).store(pass, (size_t)(t * k + b) * C + c);
    }
  }
}

// dW_route[j][i] = sum over token splits of B2's router partials (column
// 48 + i of its 64-float rows) - rred[i] (the LayerNorm mean's share:
// sum_t mean_t drho[t, i] / sd_t, the same for every row j).
__global__ __launch_bounds__(256) void k_route_dwr(const float* __restrict__ dwp, int nsplit, int64_t NC, int N,
                                                   const float* __restrict__ rred, float* __restrict__ dWr,
                                                   int accumulate) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= NC * N) return;
  const int64_t j = g / N;
  const int i = (int)(g - j * N);
  float s = 0.f;
  #pragma unroll 8
  for (int q = 0; q < nsplit; ++q) s += dwp[((size_t)q * NC + j) * 64 + 48 + i];
  s -= rred[i];
  dWr[g] = (accumulate ? dWr[g] : 0.f) + s;
}

void launch_route_pass(const Plan& p, const void* dXn, const int32_t* ridx, const float* hres, void* pass,
                       hipStream_t st) {
  const int ncb = (p.C + RP_CH - 1) / RP_CH;
  const int64_t nb = (int64_t)p.T * ncb;
  if (p.dtype == XHC_BF16)
    k_route_pass<BF16><<<nb, 256, 0, st>>>(dXn, ridx, hres, pass, p.T, p.C, p.N, p.k, ncb);
  else
    k_route_pass<F32><<<nb, 256, 0, st>>>(dXn, ridx, hres, pass, p.T, p.C, p.N, p.k, ncb);
}

void launch_route_dwr(const Plan& p, const float* dwp, const float* rred, float* dWr, int accumulate,
                      hipStream_t st) {
  const int nb = (int)((p.NC * p.N + 255) / 256);
  k_route_dwr<<<nb, 256, 0, st>>>(dwp, p.b2_ts, p.NC, p.N, rred, dWr, accumulate);
}

// Per-token active lists (the caller's, or the router's handed back to the
// backward): one thread per token checks that its k ids lie in [0, N) and
// are distinct.  A bad token ORs its findings into status[0] and counts
// itself in status[1]; good tokens touch nothing, so the usual case costs
// one read of the lists.
__global__ __launch_bounds__(256) void k_check_lists(const int32_t* __restrict__ ids, int64_t T, int k, int N,
                                                     int32_t* __restrict__ status) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int v[4];
  int bad = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    v[b] = b < k ? ids[t * k + b] : 0;
    if (b < k && (unsigned)v[b] >= (unsigned)N) bad |= XHC_STATUS_ID_RANGE;
  }
#pragma unroll
  for (int b = 1; b < 4; ++b)
#pragma unroll
    for (int a = 0; a < b; ++a)
      if (b < k && v[a] == v[b]) bad |= XHC_STATUS_ID_REPEAT;
  if (bad) {
    atomicOr(status, bad);
    atomicAdd(status + 1, 1);
  }
}

void launch_check_lists(const Plan& p, const int32_t* ids, int32_t* status, hipStream_t st) {
  const int64_t nb = ((int64_t)p.T + 255) / 256;
  k_check_lists<<<nb, 256, 0, st>>>(ids, p.T, p.k, p.N, status);
}

// The split forward's second call rebuilds the coefficient records from the
// first call's saved logits; the routed slots' post coefficients are then
// scaled by s = sigmoid(rho) of the score saved for that slot (z_save's
// router record: rho of routed slot j at P + 3 + 3j), the same product the
// router formed.  One thread per (token, post entry a*4 + m).
__global__ __launch_bounds__(256) void k_route_scale_post(float* __restrict__ coef, const float* __restrict__ zin,
                                                          int64_t T, int zsv, int P, int nfix, int k) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= T * 16) return;
  const int64_t t = j >> 4;
  const int e = (int)(j & 15), a = e >> 2;
  if (a < nfix || a >= k) return;
  float* c = coef + (size_t)t * COEF_STRIDE + CO_POST + e;
  *c = *c * sigmoid(zin[(size_t)t * zsv + P + 3 + 3 * (a - nfix)]);
}

void launch_route_scale_post(const Plan& p, const float* z_save, float* coef, hipStream_t st) {
  const int64_t n = (int64_t)p.T * 16;
  k_route_scale_post<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(coef, z_save, (int64_t)p.T, p.zsv, p.P, p.nfix,
                                                                  p.k);
}

}  // namespace xhc

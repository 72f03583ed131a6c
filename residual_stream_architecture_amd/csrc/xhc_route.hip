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
// so the projection pass forms x.Wr and sum(x) on MFMA next to the other
// logits, and only Wr's column sums are needed apart (k_route_colsum).
//
//   k_route_colsum  W_route [NC, N] -> partial column sums [RCS_BLK][16]
//   k_route_pass    (backward) pass[t][b] = sum_a H_res[a, b] G_a, the
//                   gradient that reaches active row b through the mixing
//                   term, for the dX assembly of rows chosen per token
//   k_route_dwr     (backward) dW_route from the dX pass's partials minus
//                   the LayerNorm mean's share
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

void launch_route_colsum(const Plan& p, const void* W_route, float* rcs, hipStream_t st) {
  if (p.dtype == XHC_BF16)
    k_route_colsum<uint16_t><<<RCS_BLK, 256, 0, st>>>(static_cast<const uint16_t*>(W_route), p.NC, p.N, rcs);
  else
    k_route_colsum<float><<<RCS_BLK, 256, 0, st>>>(static_cast<const float*>(W_route), p.NC, p.N, rcs);
}

}  // namespace xhc

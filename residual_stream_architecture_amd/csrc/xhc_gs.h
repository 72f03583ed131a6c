// Modified Gram-Schmidt over the four write-back components, per token, in
// coefficient form (section "Conv 带来了新信息，也带来了新的麻烦" of the
// "xHC: Expanded Hyper-Connections" retrospective: the output is kept, and
// each conv component loses its projections on the components before it,
// removed one after another).
//
// Every u~_c is a combination of the raw components, u~_c = sum_m T[c][m] U_m
// with T unit lower triangular, and every inner product the procedure takes
// is one of the Gram matrix g[m][n] = <U_m, U_n> (sums over the C channels):
//   <a, u~_j> = a^T g T_j for a combination a.
// So a token's whole Gram-Schmidt is a 4 x 4 computation on g, and the write
// uses H_post T in place of H_post.  The removals, in the order of the
// method (component c receives j = 0, 1, .., c-1 in turn):
//   y_j = g T_j,  den_j = T_j . y_j + ceps           (ceps = C * gs_eps)
//   alpha_cj = (T_c . y_j) / den_j,  T_c -= alpha_cj T_j   for c > j.
// Arithmetic is fp32 with fixed-order sums, so every lane that runs it for a
// token gets the same bits.
#pragma once

namespace xhc {

struct GsFwd {
  float T[4][4];      // u~_c = sum_m T[c][m] U_m
  float y[3][4];      // y_j = g T_j
  float den[3];       // <u~_j, u~_j> + ceps
  float V[4][3][4];   // V[c][j] = T_c before the removal of u~_j (c > j)
  float al[4][3];     // alpha_cj
};

// g: the full symmetric Gram matrix.
__device__ inline void gs_forward(const float (&g)[4][4], float ceps, GsFwd& f) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m) f.T[c][m] = c == m ? 1.f : 0.f;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    float d = ceps;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float s = 0.f;
#pragma unroll
      for (int n = 0; n <= j; ++n) s = fmaf(g[m][n], f.T[j][n], s);
      f.y[j][m] = s;
    }
#pragma unroll
    for (int n = 0; n <= j; ++n) d = fmaf(f.T[j][n], f.y[j][n], d);
    f.den[j] = d;
    const float inv = 1.f / d;
#pragma unroll
    for (int c = j + 1; c < 4; ++c) {
      float num = 0.f;
#pragma unroll
      for (int n = 0; n <= c; ++n) num = fmaf(f.T[c][n], f.y[j][n], num);
      const float a = num * inv;
      f.al[c][j] = a;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        f.V[c][j][n] = f.T[c][n];
        if (n <= j) f.T[c][n] = fmaf(-a, f.T[j][n], f.T[c][n]);
      }
    }
  }
}

// Reverse mode of gs_forward: from dT (the gradient of T; entries m >= c are
// not variables and are ignored) to S = dg + dg^T, so that the gradient of
// the raw components through T is dU_m += sum_n S[m][n] U_n.
//   removal (c, j):  dalpha = -dT_c . T_j;  dT_j -= alpha dT_c;
//                    dnum = dalpha / den_j;  dden_j -= dalpha alpha / den_j;
//                    dT_c += dnum y_j;       dy_j += dnum V[c][j]
//   then for y_j, den_j:  dT_j += dden_j y_j + g dy_j;  dy_j += dden_j T_j;
//                         dg += dy_j T_j^T
// walked for j = 2, 1, 0: dT_j is complete once the removals that read T_j
// (c > j) and y_j, den_j are walked, before T_j's own removals (j' < j).
__device__ inline void gs_backward(const float (&g)[4][4], const GsFwd& f, const float (&dTin)[4][4],
                                   float (&S)[4][4]) {
  float dT[4][4], dg[4][4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      dT[c][m] = m < c ? dTin[c][m] : 0.f;
      dg[c][m] = 0.f;
    }
#pragma unroll
  for (int j = 2; j >= 0; --j) {
    float dy[4] = {0.f, 0.f, 0.f, 0.f};
    float dden = 0.f;
    const float inv = 1.f / f.den[j];
#pragma unroll
    for (int c = 3; c > j; --c) {
      float da = 0.f;
#pragma unroll
      for (int n = 0; n <= j; ++n) da = fmaf(-dT[c][n], f.T[j][n], da);
      const float a = f.al[c][j];
#pragma unroll
      for (int n = 0; n <= j; ++n) dT[j][n] = fmaf(-a, dT[c][n], dT[j][n]);
      const float dnum = da * inv;
      dden = fmaf(-dnum, a, dden);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        dT[c][n] = fmaf(dnum, f.y[j][n], dT[c][n]);
        dy[n] = fmaf(dnum, f.V[c][j][n], dy[n]);
      }
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) dy[n] = fmaf(dden, f.T[j][n], dy[n]);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      float s = dden * f.y[j][n];
#pragma unroll
      for (int m = 0; m < 4; ++m) s = fmaf(g[m][n], dy[m], s);
      dT[j][n] += s;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) dg[m][n] = fmaf(dy[m], f.T[j][n], dg[m][n]);
  }
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) S[m][n] = dg[m][n] + dg[n][m];
}

// Gram record of a token: the 10 entries m <= n in the order
// (0,0) (0,1) (0,2) (0,3) (1,1) (1,2) (1,3) (2,2) (2,3) (3,3).
__device__ constexpr int gram_idx(int m, int n) {
  return m <= n ? (m * (7 - m)) / 2 + n : (n * (7 - n)) / 2 + m;
}

}  // namespace xhc

// Backward kernels of the xHC sublayer update (gfx950).
//
// The gradients are those of the forward defined in the "xHC: Expanded
// Hyper-Connections" retrospective (sections "把 N 调大以后…" for the
// H_pre/H_post/H_res roles and Sinkhorn, "最便宜的新信息…" for TFA,
// "模型可以拥有 16 条 streams，但每层只更新 4 条" for the dense read and the
// sparse write), derived by hand.  With G_a = dX_new[t, i_a]:
//   dH_pre[i]    = <dh_in, X_i>          dH_res[a,b] = <G_a, X_{i_b}>
//   dH_post[a,m] = <G_a, U_m>            dU_m = sum_a H_post[a,m] G_a
//   dz = gate and unrolled-Sinkhorn backward of (dH_pre, dH_post, dH_res)
//   dX[i] = [i inactive] dX_new[i] + [i = i_b] sum_a H_res[a,b] G_a
//           + H_pre[i] dh_in + (dz W^T)_i / r - X_i * gamma,
//           gamma = dz.(z - bias) / (N*C*r^2)
//   dW = sum_t (X_t / r_t)^T dz_t,  db = sum_t dz_t
//   dout = dU_0 + sum_m (anti-causal correlation of dU_m with w_m)
//   dw_m[c,q] = sum_t dU_m[t,c] out[t-K_m+1+q, c]
//
// Pipeline of one backward call:
//   k_coef (shared)  coefficients from z_save (or a fresh projection)
//   k_pack_wp        W [N*C, P] -> Wp [N*C, 64] zero-padded A operand
//   k_bdots  (B1)    per (channel block, segment): the 48 dots per token
//                    (MFMA for the X dots, VALU for the TFA part), dout,
//                    conv-weight partials
//   k_bcoef          per token: reduce dots, gates' and Sinkhorn's backward,
//                    dz, dz/r (MFMA operands), gamma
//   k_bgrad  (B2)    per (row group, 64 channels, token split): dX assembly
//                    with the dz W^T term on MFMA, dW partials on MFMA
//   k_red_*          deterministic reductions of dW, db and dw partials
#include "xhc_device.h"
#include "xhc_launch.h"

namespace xhc {

struct Act4 { int id[4]; };
struct RowTable { int stream[5][4]; };   // row group -> 4 stream ids (-1 = none)

// ---------------------------------------------------------------------------
// W [NC, P] -> Wp [NC, 64], columns p >= P zero.
// ---------------------------------------------------------------------------
template <typename R>
__global__ void k_pack_wp(const R* __restrict__ W, R* __restrict__ Wp, int64_t NC, int P) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= NC * 64) return;
  const int64_t j = idx >> 6;
  const int p = (int)(idx & 63);
  Wp[idx] = p < P ? W[(size_t)j * P + p] : R(0);
}

// ---------------------------------------------------------------------------
// B1.  Workgroup = 4 waves on 4 consecutive 128-channel chunks of one
// sequence segment [s0, s1).  Per token:
//   * X dots on MFMA: A = the 16 state rows (K = the chunk's channels),
//     B columns = [dh_in, G_0..G_{k-1}, 0...]; D[i][0] = dH_pre[i] and
//     D[i_b][1+a] = dH_res[a][b] (partial over the chunk).
//   * TFA part (lane = 2 channels): U_m from a 12-row ring of `out`,
//     dH_post partials (wave-reduced), dU_m scattered into a 12-slot ring of
//     dout accumulators (anti-causal), conv-weight partials.
// The segment is followed by an 11-token lookahead that only scatters dU
// into the segment's last dout positions.  The 4 waves' partial dots are
// summed in LDS once per 12 tokens and written per channel block.
// ---------------------------------------------------------------------------
template <typename E, int NCOMP>
__global__ __launch_bounds__(256) void k_bdots(
    StreamRows src, const void* __restrict__ dXn, const void* __restrict__ dhin,
    const void* __restrict__ out, const float* __restrict__ w4, const float* __restrict__ w8,
    const float* __restrict__ w12, const float* __restrict__ coef, float* __restrict__ dpart,
    void* __restrict__ dout, float* __restrict__ dwpart, int T, int S, int C, int N, int k, Act4 act,
    int lseg, int segs_per_seq) {
  using V2 = Vec<E, B1_CH>;
  __shared__ float red[B1_WAVES][12][DOT_STRIDE];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cblock = blockIdx.x;
  const int c0 = (cblock * B1_WAVES + wave) * B1_WAVE_CH;
  const int seg = blockIdx.y;
  const int bseq = seg / segs_per_seq;
  const int s0 = (seg - bseq * segs_per_seq) * lseg;
  const int s1 = min(s0 + lseg, S);
  const size_t tok0 = (size_t)bseq * S;
  const int64_t NCs = (int64_t)N * C;

  // TFA lane channels
  const int cl = c0 + B1_CH * lane;
  const bool cv = cl < C;
  // MFMA lane roles
  const int r16 = lane & 15, g4 = lane >> 4;
  const int n_col = r16;   // B column: 0 = dh_in, 1..k = G_{n-1}
  const void* arow_base = src.base[r16];
  const int64_t arow_stride = src.stride[r16];
  const bool arow_valid = r16 < N;

  float wk[B1_CH][24];
  if (NCOMP == 4) {
#pragma unroll
    for (int ch = 0; ch < B1_CH; ++ch) {
      const int cc = cv ? cl + ch : 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) wk[ch][q] = w4[(size_t)cc * 4 + q];
#pragma unroll
      for (int q = 0; q < 8; ++q) wk[ch][4 + q] = w8[(size_t)cc * 8 + q];
#pragma unroll
      for (int q = 0; q < 12; ++q) wk[ch][12 + q] = w12[(size_t)cc * 12 + q];
    }
  }
  float ring[12][B1_CH], dacc[12][B1_CH], dw[B1_CH][24];
#pragma unroll
  for (int j = 0; j < 12; ++j) {
    const int s = s0 - 12 + j;
#pragma unroll
    for (int ch = 0; ch < B1_CH; ++ch) { ring[j][ch] = 0.f; dacc[j][ch] = 0.f; }
    if (NCOMP == 4 && j > 0 && s >= 0 && cv) {
      V2 v = V2::load(out, (tok0 + s) * C + cl);
      v.to_float(ring[j]);
    }
  }
#pragma unroll
  for (int ch = 0; ch < B1_CH; ++ch)
#pragma unroll
    for (int q = 0; q < 24; ++q) dw[ch][q] = 0.f;

  const int tend = s1 + 11;
  for (int g0 = s0; g0 < tend; g0 += 12) {
#pragma unroll
    for (int j = 0; j < 12; ++j) {
      const int s = g0 + j;
      if (s < tend) {
        const bool main_tok = s < s1;
        const bool live = s < S;              // lookahead tokens exist
        const size_t t = tok0 + (live ? s : 0);
        const float* co = coef + t * COEF_STRIDE;

        if (main_tok) {
          // ---- X dots on MFMA over this wave's 128 channels ----
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < B1_WAVE_CH / 32; ++ks) {
            const int cc = c0 + ks * 32 + 8 * g4;
            const bool kv = cc < C;
            V8<E> av = (kv && arow_valid) ? V8<E>::load(arow_base, t * arow_stride + cc) : V8<E>::zero();
            V8<E> bv = V8<E>::zero();
            if (kv) {
              if (n_col == 0) bv = V8<E>::load(dhin, t * C + cc);
              else if (n_col <= k) bv = V8<E>::load(dXn, (t * N + act.id[n_col - 1]) * C + cc);
            }
            acc = mma32(av, bv, acc);
          }
          // lane (n_col, g4) holds D[4*g4 + e][n_col]
          if (n_col == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) red[wave][j][4 * g4 + e] = acc[e];
          } else if (n_col <= 4) {
            const int a = n_col - 1;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const bool ok = a < k && b < k;
              const int ib = ok ? act.id[b] : 0;
              if (ok && (ib >> 2) == g4) {
                const int e = ib & 3;
                red[wave][j][16 + a * 4 + b] = e == 0 ? acc[0] : e == 1 ? acc[1] : e == 2 ? acc[2] : acc[3];
              } else if (!ok && g4 == 0) {
                red[wave][j][16 + a * 4 + b] = 0.f;
              }
            }
          }
        }

        // ---- TFA part ----
        float G[4][B1_CH];
        if (live) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            if (a < k && cv) {
              V2 gv = V2::load(dXn, (t * N + act.id[a]) * C + cl);
              gv.to_float(G[a]);
            } else {
#pragma unroll
              for (int ch = 0; ch < B1_CH; ++ch) G[a][ch] = 0.f;
            }
          }
        }
        if (main_tok) {
          if (cv) {
            V2 ov = V2::load(out, t * C + cl);
            ov.to_float(ring[j]);
          } else {
#pragma unroll
            for (int ch = 0; ch < B1_CH; ++ch) ring[j][ch] = 0.f;
          }
          // U_m for this token
          float U[4][B1_CH];
#pragma unroll
          for (int ch = 0; ch < B1_CH; ++ch) {
            U[0][ch] = ring[j][ch];
            if (NCOMP == 4) {
              float s4 = 0.f, s8 = 0.f, s12 = 0.f;
#pragma unroll
              for (int q = 0; q < 4; ++q) s4 = fmaf(wk[ch][q], ring[(j + 12 - 3 + q) % 12][ch], s4);
#pragma unroll
              for (int q = 0; q < 8; ++q) s8 = fmaf(wk[ch][4 + q], ring[(j + 12 - 7 + q) % 12][ch], s8);
#pragma unroll
              for (int q = 0; q < 12; ++q) s12 = fmaf(wk[ch][12 + q], ring[(j + 12 - 11 + q) % 12][ch], s12);
              U[1][ch] = s4; U[2][ch] = s8; U[3][ch] = s12;
            }
          }
          // dH_post partials v[a*4+m], reduced over the wave by halving
          float v[16];
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              float d = 0.f;
              if (m < NCOMP) {
#pragma unroll
                for (int ch = 0; ch < B1_CH; ++ch) d = fmaf(G[a][ch], U[m][ch], d);
              }
              v[a * 4 + m] = d;
            }
          {
            const bool h5 = lane & 32;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const float send = h5 ? v[q] : v[8 + q];
              const float keep = h5 ? v[8 + q] : v[q];
              v[q] = keep + shfl_xor(send, 32);
            }
            const bool h4 = lane & 16;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float send = h4 ? v[q] : v[4 + q];
              const float keep = h4 ? v[4 + q] : v[q];
              v[q] = keep + shfl_xor(send, 16);
            }
            const bool h3 = lane & 8;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const float send = h3 ? v[q] : v[2 + q];
              const float keep = h3 ? v[2 + q] : v[q];
              v[q] = keep + shfl_xor(send, 8);
            }
            const bool h2 = lane & 4;
            {
              const float send = h2 ? v[0] : v[1];
              const float keep = h2 ? v[1] : v[0];
              v[0] = keep + shfl_xor(send, 4);
            }
            v[0] += shfl_xor(v[0], 1);
            v[0] += shfl_xor(v[0], 2);
            if ((lane & 3) == 0) {
              const int idx = ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1);
              red[wave][j][32 + idx] = v[0];
            }
          }
          // conv-weight partials: dw_m[c,q] += dU_m[t] * out[t-K_m+1+q]
        }
        if (live) {
          float dU[4][B1_CH];
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int ch = 0; ch < B1_CH; ++ch) {
              float d = 0.f;
              if (m < NCOMP) {
#pragma unroll
                for (int a = 0; a < 4; ++a)
                  if (a < k) d = fmaf(co[CO_POST + a * 4 + m], G[a][ch], d);
              }
              dU[m][ch] = d;
            }
          if (main_tok && NCOMP == 4) {
#pragma unroll
            for (int ch = 0; ch < B1_CH; ++ch) {
#pragma unroll
              for (int q = 0; q < 4; ++q) dw[ch][q] = fmaf(dU[1][ch], ring[(j + 12 - 3 + q) % 12][ch], dw[ch][q]);
#pragma unroll
              for (int q = 0; q < 8; ++q) dw[ch][4 + q] = fmaf(dU[2][ch], ring[(j + 12 - 7 + q) % 12][ch], dw[ch][4 + q]);
#pragma unroll
              for (int q = 0; q < 12; ++q) dw[ch][12 + q] = fmaf(dU[3][ch], ring[(j + 12 - 11 + q) % 12][ch], dw[ch][12 + q]);
            }
          }
          // scatter into dout accumulators of positions s - lag (lag < K_m)
          if (main_tok) {
#pragma unroll
            for (int ch = 0; ch < B1_CH; ++ch) dacc[j][ch] += dU[0][ch];
          }
          if (NCOMP == 4) {
#pragma unroll
            for (int lag = 0; lag < 12; ++lag) {
              const int pos = s - lag;
              if (pos >= s0 && pos < s1) {
                const int slot = (j + 12 - lag) % 12;
#pragma unroll
                for (int ch = 0; ch < B1_CH; ++ch) {
                  float d = dacc[slot][ch];
                  if (lag < 4) d = fmaf(wk[ch][3 - lag], dU[1][ch], d);
                  if (lag < 8) d = fmaf(wk[ch][4 + 7 - lag], dU[2][ch], d);
                  d = fmaf(wk[ch][12 + 11 - lag], dU[3][ch], d);
                  dacc[slot][ch] = d;
                }
              }
            }
          }
        }
        // position s-11 is complete: emit it
        {
          const int pos = s - 11;
          const int slot = (j + 1) % 12;
          if (pos >= s0 && pos < s1) {
            if (cv) V2::from_float(dacc[slot]).store(dout, (tok0 + pos) * C + cl);
#pragma unroll
            for (int ch = 0; ch < B1_CH; ++ch) dacc[slot][ch] = 0.f;
          }
        }
      }
    }
    // ---- sum the 4 waves' dots of this group's tokens ----
    __syncthreads();
    for (int idx = threadIdx.x; idx < 12 * DOT_STRIDE; idx += 256) {
      const int jj = idx / DOT_STRIDE, q = idx - jj * DOT_STRIDE;
      const int s = g0 + jj;
      if (s < s1) {
        const float sum = (red[0][jj][q] + red[1][jj][q]) + (red[2][jj][q] + red[3][jj][q]);
        dpart[((size_t)cblock * T + tok0 + s) * DOT_STRIDE + q] = sum;
      }
    }
    __syncthreads();
  }
  if (NCOMP == 4 && cv) {
#pragma unroll
    for (int ch = 0; ch < B1_CH; ++ch) {
      float* dst = dwpart + ((size_t)seg * C + cl + ch) * 24;
#pragma unroll
      for (int q = 0; q < 24; q += 4)
        *reinterpret_cast<f32x4*>(dst + q) = f32x4{dw[ch][q], dw[ch][q + 1], dw[ch][q + 2], dw[ch][q + 3]};
    }
  }
}

// ---------------------------------------------------------------------------
// Coefficient backward.  16 lanes per token, lane e owns pre slot e, post
// slot (a, m) = (e/4, e%4) and Sinkhorn entry (a, b) = (e/4, e%4).  The
// Sinkhorn iterates after every column step are kept in LDS and walked back:
//   column step Mc = R / colsum(R):  dR = (dMc - colsum(dMc*Mc)) / colsum(R)
//   row step    R  = M / rowsum(M):  dM = (dR - rowsum(dR*R))  / rowsum(M)
//   dL = dM_0 * M_0 (the row-max shift cancels in the first row step).
// ---------------------------------------------------------------------------
constexpr int BCOEF_TOK = 4;

template <typename E>
__global__ __launch_bounds__(64) void k_bcoef(const float* __restrict__ dpart, int ncb, const float* __restrict__ zin,
                                              const float* __restrict__ bias, float* __restrict__ coef,
                                              float* __restrict__ dz_out, void* __restrict__ dzr,
                                              void* __restrict__ dzrt, int T, int64_t Tpad, int N, int k, int nc,
                                              int P, float inv_nc_total, int iters, int unit_gates) {
  extern __shared__ float hist[];   // [BCOEF_TOK][iters+1][16]
  __shared__ float dzs[BCOEF_TOK][64];
  const int e = threadIdx.x & 15, tok = threadIdx.x >> 4;
  const int64_t t = (int64_t)blockIdx.x * BCOEF_TOK + tok;
  const bool tv = t < T;
  const int64_t tc = tv ? t : 0;
  float* H = hist + (size_t)tok * (iters + 1) * 16;

  // reduce the per-chunk dots
  float dpre = 0.f, dres = 0.f, dpost = 0.f;
  for (int cb = 0; cb < ncb; ++cb) {
    const float* d = dpart + ((size_t)cb * T + tc) * DOT_STRIDE;
    dpre += d[e];
    dres += d[16 + e];
    dpost += d[32 + e];
  }
  const float* co = coef + tc * COEF_STRIDE;
  const float* z = zin + tc * (P + 1);
  const float r = co[CO_R];

  // gates
  float dz_pre = 0.f, dz_post = 0.f;
  if (!unit_gates) {
    const float hp = co[CO_PRE + e];
    dz_pre = e < N ? dpre * hp * (1.f - hp) : 0.f;
    const float hq = co[CO_POST + e];
    dz_post = ((e >> 2) < k && (e & 3) < nc) ? dpost * hq * (1.f - hq) : 0.f;
  }

  // Sinkhorn backward
  const int a = e >> 2, b = e & 3;
  const bool valid = a < k && b < k;
  {
    const float L = valid ? z[N + k * nc + a * k + b] : -INFINITY;
    float mx = fmaxf(L, shfl_xor(L, 1));
    mx = fmaxf(mx, shfl_xor(mx, 2));
    float M = valid ? expf(L - mx) : 0.f;
    H[e] = M;
    for (int it = 0; it < iters; ++it) {
      float rs = M + shfl_xor(M, 1);
      rs += shfl_xor(rs, 2);
      M = valid ? M / rs : 0.f;
      float cs = M + shfl_xor(M, 4);
      cs += shfl_xor(cs, 8);
      M = valid ? M / cs : 0.f;
      H[(it + 1) * 16 + e] = M;
    }
  }
  float g = valid ? dres : 0.f;
  for (int it = iters; it >= 1; --it) {
    const float Mp = H[(it - 1) * 16 + e];
    float rs = Mp + shfl_xor(Mp, 1);
    rs += shfl_xor(rs, 2);
    const float R = valid ? Mp / rs : 0.f;
    float cs = R + shfl_xor(R, 4);
    cs += shfl_xor(cs, 8);
    const float Mc = valid ? R / cs : 0.f;
    float t1 = g * Mc;
    t1 += shfl_xor(t1, 4);
    t1 += shfl_xor(t1, 8);
    const float gR = valid ? (g - t1) / cs : 0.f;
    float t2 = gR * R;
    t2 += shfl_xor(t2, 1);
    t2 += shfl_xor(t2, 2);
    g = valid ? (gR - t2) / rs : 0.f;
  }
  const float dL = g * H[e];

  // assemble dz in the logit column layout
  dzs[tok][e] = 0.f; dzs[tok][16 + e] = 0.f; dzs[tok][32 + e] = 0.f; dzs[tok][48 + e] = 0.f;
  __syncthreads();
  if (e < N) dzs[tok][e] = dz_pre;
  if (a < k && b < nc) dzs[tok][N + a * nc + b] = dz_post;
  if (valid) dzs[tok][N + k * nc + a * k + b] = dL;
  __syncthreads();

  // gamma = dz.(z - bias) / (N*C*r^2)
  float al = 0.f;
#pragma unroll
  for (int n = 0; n < 3; ++n) {
    const int p = e + 16 * n;
    if (p < P) al = fmaf(dzs[tok][p], z[p] - (bias ? bias[p] : 0.f), al);
  }
  al += shfl_xor(al, 1);
  al += shfl_xor(al, 2);
  al += shfl_xor(al, 4);
  al += shfl_xor(al, 8);
  const float inv_r = 1.f / r;
  if (tv) {
    if (e == 0) coef[t * COEF_STRIDE + CO_GAMMA] = al * inv_nc_total * inv_r * inv_r;
#pragma unroll
    for (int n = 0; n < 3; ++n) dz_out[t * 48 + e + 16 * n] = dzs[tok][e + 16 * n];
  }
  // MFMA operands: dzr [T][64] (B operand of dz W^T) and its transpose
  // [48][Tpad] (operand of dW); t in [T, Tpad) is written as zero.  In bf16
  // mode each is stored as hi and lo halves (hi at offset 0, lo after it):
  // the dz values of saturated Sinkhorn entries are large, and the products
  // must keep fp32 accuracy.
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int p = e + 16 * n;
    const float v = tv ? dzs[tok][p] * inv_r : 0.f;
    if constexpr (E::bytes == 2) {
      __bf16 hi, lo;
      split_bf16(v, hi, lo);
      if (tv) {
        reinterpret_cast<__bf16*>(dzr)[t * 64 + p] = hi;
        reinterpret_cast<__bf16*>(dzr)[((size_t)T + t) * 64 + p] = lo;
      }
      if (p < 48 && t < Tpad) {
        reinterpret_cast<__bf16*>(dzrt)[(size_t)p * Tpad + t] = hi;
        reinterpret_cast<__bf16*>(dzrt)[(size_t)(48 + p) * Tpad + t] = lo;
      }
    } else {
      if (tv) reinterpret_cast<float*>(dzr)[t * 64 + p] = v;
      if (p < 48 && t < Tpad) reinterpret_cast<float*>(dzrt)[(size_t)p * Tpad + t] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// B2.  Workgroup = (row group, 64 channels, token split); wave w handles the
// group's row w.  Per 32-token tile:
//   proj[c][t] = sum_p W[i*C+c, p] dzr[t, p] on MFMA, with A rows permuted so
//   that lane (t = lane%16, g = lane/16) ends up owning channels 16g..16g+16
//   of tokens t and t+16 -- the layout of its own vector loads;
//   dX = pass + H_pre dh_in + proj - X gamma;
//   dW[i*C+c][p] += sum_t X[t, c] dzr[t, p] on MFMA (A = X^T through LDS,
//   dzr as bf16 hi + lo).
// For the active group all rows are read before any is written (barrier), so
// dX may alias dX_new.
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void k_bgrad(
    StreamRows src, const void* __restrict__ dXn, const void* __restrict__ dhin,
    const float* __restrict__ coef, const void* __restrict__ Wp, const void* __restrict__ dzr,
    const void* __restrict__ dzrt, void* dX, float* __restrict__ dwp, int T, int64_t Tpad, int C, int N,
    int k, Act4 act, RowTable rows, int nrg, int ncb, int tok_per_split) {
  constexpr bool BF = E::bytes == 2;
  constexpr int XS_LD = B2_CB + 8;                         // padded LDS row (elements)
  __shared__ __attribute__((aligned(16))) unsigned char xs_raw[4][B2_TT][XS_LD * E::bytes];

  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int rg = lb % nrg;
  const int cb = (lb / nrg) % ncb;
  const int ts = lb / (nrg * ncb);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int stream = rows.stream[rg][wave];
  const bool wv = stream >= 0;
  const int srow = wv ? stream : 0;
  const bool active_grp = rg == 0;
  const int c0 = cb * B2_CB;
  const int64_t NCs = (int64_t)N * C;
  const size_t jbase = (size_t)srow * C + c0;   // flattened row index of channel c0

  // proj A operand: W rows, permuted: A row m of j-tile jt -> channel
  // 16*(m/4) + 4*jt + m%4 ; K = 64 logits in two steps.
  V8<E> wa[4][2];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    const int ch = 16 * (r16 >> 2) + 4 * jt + (r16 & 3);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      wa[jt][ks] = (wv && c0 + ch < C) ? V8<E>::load(Wp, (jbase + ch) * 64 + 32 * ks + 8 * g4) : V8<E>::zero();
  }
  f32x4 dwacc[4][3];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int pt = 0; pt < 3; ++pt) dwacc[jt][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const void* xbase = src.base[srow];
  const int64_t xstride = src.stride[srow];
  const int cl = c0 + 16 * g4;                  // this lane's 16 channels
  const bool cv = wv && cl < C;                 // C % 8 == 0: 8-wide halves
  const bool cv2 = wv && cl + 8 < C;
  unsigned char (*xs)[XS_LD * E::bytes] = xs_raw[wave];

  const int tbeg = ts * tok_per_split;
  const int tfin = min(tbeg + tok_per_split, T);
  for (int t0 = tbeg; t0 < tfin; t0 += B2_TT) {
    // ---- proj on MFMA: D[c][t] for 4 j-tiles x 2 token tiles ----
    f32x4 pj[4][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tb = t0 + 16 * tt + r16;
      V8<E> bz[2], bzl[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bz[ks] = tb < T ? V8<E>::load(dzr, (size_t)tb * 64 + 32 * ks + 8 * g4) : V8<E>::zero();
        if constexpr (BF)
          bzl[ks] = tb < T ? V8<E>::load(dzr, ((size_t)T + tb) * 64 + 32 * ks + 8 * g4) : V8<E>::zero();
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma32(wa[jt][0], bz[0], acc);
        acc = mma32(wa[jt][1], bz[1], acc);
        if constexpr (BF) {
          acc = mma32(wa[jt][0], bzl[0], acc);
          acc = mma32(wa[jt][1], bzl[1], acc);
        }
        pj[jt][tt] = acc;
      }
    }
    // ---- loads for the elementwise assembly ----
    V8<E> xv[2][2], dv[2][2], hv[2][2];
    float hpre[2], gam[2], hres[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tk = t0 + 16 * tt + r16;
      const bool tv = tk < T;
      const size_t tkc = tv ? tk : 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool ok = tv && (h ? cv2 : cv);
        xv[tt][h] = ok ? V8<E>::load(xbase, tkc * xstride + cl + 8 * h) : V8<E>::zero();
        hv[tt][h] = ok ? V8<E>::load(dhin, tkc * C + cl + 8 * h) : V8<E>::zero();
        dv[tt][h] = (ok && !active_grp) ? V8<E>::load(dXn, (tkc * N + srow) * C + cl + 8 * h) : V8<E>::zero();
      }
      const float* co = coef + tkc * COEF_STRIDE;
      hpre[tt] = co[CO_PRE + srow];
      gam[tt] = co[CO_GAMMA];
#pragma unroll
      for (int a = 0; a < 4; ++a) hres[tt][a] = (active_grp && a < k) ? co[CO_RES + a * 4 + wave] : 0.f;
    }
    // active group: pass term sum_a H_res[a][wave] G_a
    float pass[2][16];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float d[8];
        dv[tt][h].to_float(d);
#pragma unroll
        for (int q = 0; q < 8; ++q) pass[tt][8 * h + q] = d[q];
      }
    }
    if (active_grp) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int tk = t0 + 16 * tt + r16;
        const bool tv = tk < T;
        const size_t tkc = tv ? tk : 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) pass[tt][q] = 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          if (a < k) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const bool ok = tv && (h ? cv2 : cv);
              V8<E> gv = ok ? V8<E>::load(dXn, (tkc * N + act.id[a]) * C + cl + 8 * h) : V8<E>::zero();
              float gf[8];
              gv.to_float(gf);
#pragma unroll
              for (int q = 0; q < 8; ++q) pass[tt][8 * h + q] = fmaf(hres[tt][a], gf[q], pass[tt][8 * h + q]);
            }
          }
        }
      }
      __syncthreads();   // every G row of the tile is read before any dX row is written
    }
    // ---- assemble and store dX; stage X into LDS for the dW operand ----
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tk = t0 + 16 * tt + r16;
      const bool tv = tk < T;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float xf[8], hf[8], o[8];
        xv[tt][h].to_float(xf);
        hv[tt][h].to_float(hf);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int cidx = 8 * h + q;                 // channel offset within the lane's 16
          const int jt = (cidx >> 2) & 3, e = cidx & 3;
          float v = pass[tt][cidx];
          v = fmaf(hpre[tt], hf[q], v);
          v += pj[jt][tt][e];
          v = fmaf(-gam[tt], xf[q], v);
          o[q] = v;
        }
        if (tv && (h ? cv2 : cv)) V8<E>::from_float(o).store(dX, ((size_t)tk * N + srow) * C + cl + 8 * h);
        *reinterpret_cast<V8<E>*>(&xs[16 * tt + r16][(16 * g4 + 8 * h) * E::bytes]) = xv[tt][h];
      }
    }
    __syncthreads();
    // ---- dW on MFMA: A = X^T (rows = channels, K = 32 tokens) ----
    V8<E> bh[3], bl[3];
#pragma unroll
    for (int pt = 0; pt < 3; ++pt) {
      const size_t off = (size_t)(16 * pt + r16) * Tpad + t0 + 8 * g4;
      bh[pt] = V8<E>::load(dzrt, off);
      if constexpr (BF) bl[pt] = V8<E>::load(dzrt, off + (size_t)48 * Tpad);
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      V8<E> xa;
      if constexpr (BF) {
        const uint16_t* col = reinterpret_cast<const uint16_t*>(&xs[0][0]) + 16 * jt + r16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const unsigned lo16 = col[(size_t)(8 * g4 + 2 * q) * XS_LD];
          const unsigned hi16 = col[(size_t)(8 * g4 + 2 * q + 1) * XS_LD];
          xa.w[q] = lo16 | (hi16 << 16);
        }
      } else {
        const float* col = reinterpret_cast<const float*>(&xs[0][0]) + 16 * jt + r16;
#pragma unroll
        for (int q = 0; q < 8; ++q) reinterpret_cast<float*>(&xa)[q] = col[(size_t)(8 * g4 + q) * XS_LD];
      }
#pragma unroll
      for (int pt = 0; pt < 3; ++pt) {
        dwacc[jt][pt] = mma32(xa, bh[pt], dwacc[jt][pt]);
        if constexpr (BF) dwacc[jt][pt] = mma32(xa, bl[pt], dwacc[jt][pt]);
      }
    }
    __syncthreads();
  }
  // dW partial rows: D row 4*g4+e of j-tile jt = channel 16*jt + 4*g4 + e
  if (wv) {
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = 16 * jt + 4 * g4 + e;
        if (c0 + ch < C) {
          float* dst = dwp + ((size_t)ts * NCs + jbase + ch) * 48;
#pragma unroll
          for (int pt = 0; pt < 3; ++pt) dst[16 * pt + r16] = dwacc[jt][pt][e];
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Deterministic reductions (fixed order, no atomics).
// ---------------------------------------------------------------------------
__global__ void k_red_dw(const float* __restrict__ part, int nsplit, int64_t NC, int P, float* __restrict__ dW,
                         int accumulate) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= NC * P) return;
  const int64_t j = idx / P;
  const int p = (int)(idx - j * P);
  float s = accumulate ? dW[idx] : 0.f;
  for (int q = 0; q < nsplit; ++q) s += part[((size_t)q * NC + j) * 48 + p];
  dW[idx] = s;
}

__global__ void k_red_db(const float* __restrict__ dz, int T, float* __restrict__ db, int accumulate) {
  __shared__ float sm[256];
  const int p = blockIdx.x;
  float s = 0.f;
  for (int t = threadIdx.x; t < T; t += 256) s += dz[(size_t)t * 48 + p];
  sm[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) sm[threadIdx.x] += sm[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) db[p] = (accumulate ? db[p] : 0.f) + sm[0];
}

__global__ void k_red_conv(const float* __restrict__ part, int nseg, int C, float* __restrict__ dw4,
                           float* __restrict__ dw8, float* __restrict__ dw12, int accumulate) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)C * 24) return;
  const int c = (int)(idx / 24), q = (int)(idx - (int64_t)c * 24);
  float s = 0.f;
  for (int g = 0; g < nseg; ++g) s += part[((size_t)g * C + c) * 24 + q];
  float* dst = q < 4 ? dw4 + (size_t)c * 4 + q : q < 12 ? dw8 + (size_t)c * 8 + (q - 4) : dw12 + (size_t)c * 12 + (q - 12);
  *dst = (accumulate ? *dst : 0.f) + s;
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <typename E, typename R>
static int backward_impl(const Plan& p, const xhc_bwd_args* a, char* ws, hipStream_t st) {
  xhc_timer* tm = a->timer;
  float* coef = reinterpret_cast<float*>(ws + p.off_coef);
  const float* zin = a->z_save;
  if (!zin) zin = reinterpret_cast<const float*>(ws + p.off_zbuf);
  int rc = launch_coef_bwd(p, a->X, a->xact, a->active, a->W, a->bias, a->z_save, ws, coef,
                           a->z_save ? nullptr : reinterpret_cast<float*>(ws + p.off_zbuf), st, tm);
  if (rc) return rc;

  void* Wp = ws + p.off_wp;
  float* dpart = reinterpret_cast<float*>(ws + p.off_dpart);
  float* dwpart = reinterpret_cast<float*>(ws + p.off_dwpart);
  float* dz = reinterpret_cast<float*>(ws + p.off_dz);
  void* dzr = ws + p.off_dzr;
  void* dzrt = ws + p.off_dzrt;
  float* dwp = reinterpret_cast<float*>(ws + p.off_dwpart2);
  const StreamRows src = stream_rows(p, a->X, a->xact, a->active);
  Act4 act;
  for (int b = 0; b < 4; ++b) act.id[b] = b < p.k ? a->active[b] : 0;

  {
    TimedLaunch tl(tm, KID_PACK_WP, st);
    const int64_t n = p.NC * 64;
    k_pack_wp<R><<<(int)((n + 255) / 256), 256, 0, st>>>(static_cast<const R*>(a->W), static_cast<R*>(Wp), p.NC, p.P);
  }
  {
    TimedLaunch tl(tm, KID_BDOTS, st);
    dim3 grid(p.b1_cblocks, p.B * p.b1_segs);
    if (p.nc == 4)
      k_bdots<E, 4><<<grid, 256, 0, st>>>(src, a->dX_new, a->dh_in, a->out, a->w4, a->w8, a->w12, coef, dpart,
                                          a->dout, dwpart, p.T, p.S, p.C, p.N, p.k, act, p.b1_lseg, p.b1_segs);
    else
      k_bdots<E, 1><<<grid, 256, 0, st>>>(src, a->dX_new, a->dh_in, a->out, nullptr, nullptr, nullptr, coef,
                                          dpart, a->dout, dwpart, p.T, p.S, p.C, p.N, p.k, act, p.b1_lseg,
                                          p.b1_segs);
  }
  {
    TimedLaunch tl(tm, KID_BCOEF, st);
    const int nb = (int)((p.Tpad + BCOEF_TOK - 1) / BCOEF_TOK);
    const size_t shm = (size_t)BCOEF_TOK * (p.iters + 1) * 16 * sizeof(float);
    k_bcoef<E><<<nb, 64, shm, st>>>(dpart, p.b1_cblocks, zin, a->bias, coef, dz, dzr, dzrt, p.T, p.Tpad, p.N,
                                    p.k, p.nc, p.P, 1.0f / (float)p.NC, p.iters, p.gate == XHC_GATE_UNIT);
  }
  {
    TimedLaunch tl(tm, KID_BGRAD, st);
    RowTable rows;
    for (int g = 0; g < 5; ++g)
      for (int w = 0; w < 4; ++w) rows.stream[g][w] = -1;
    for (int w = 0; w < p.k; ++w) rows.stream[0][w] = a->active[w];
    int nxt = 0;
    for (int i = 0; i < p.N; ++i) {
      bool is_act = false;
      for (int b = 0; b < p.k; ++b) is_act |= a->active[b] == i;
      if (is_act) continue;
      rows.stream[1 + nxt / 4][nxt % 4] = i;
      ++nxt;
    }
    const int nb = p.b2_rowgroups * p.b2_cblocks * p.b2_ts;
    k_bgrad<E><<<nb, 256, 0, st>>>(src, a->dX_new, a->dh_in, coef, Wp, dzr, dzrt, a->dX, dwp, p.T, p.Tpad, p.C,
                                   p.N, p.k, act, rows, p.b2_rowgroups, p.b2_cblocks, p.b2_tok_per_split);
  }
  {
    TimedLaunch tl(tm, KID_BREDUCE, st);
    const int64_t n = p.NC * p.P;
    k_red_dw<<<(int)((n + 255) / 256), 256, 0, st>>>(dwp, p.b2_ts, p.NC, p.P, a->dW, a->accumulate);
    if (a->db) k_red_db<<<p.P, 256, 0, st>>>(dz, p.T, a->db, a->accumulate);
    if (p.nc == 4) {
      const int64_t m = (int64_t)p.C * 24;
      k_red_conv<<<(int)((m + 255) / 256), 256, 0, st>>>(dwpart, p.B * p.b1_segs, p.C, a->dw4, a->dw8, a->dw12,
                                                          a->accumulate);
    }
  }
  return hipGetLastError() == hipSuccess ? XHC_OK : XHC_ERR_HIP;
}

int launch_backward(const Plan& p, const xhc_bwd_args* a, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  if (p.dtype == XHC_BF16) return backward_impl<BF16, uint16_t>(p, a, w, st);
  return backward_impl<F32, float>(p, a, w, st);
}

}  // namespace xhc

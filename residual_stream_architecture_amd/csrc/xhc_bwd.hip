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
//   (k_coef path)    only when no logits were saved: a fresh projection
//   k_bxdots (B1x)   per (512 channels, 64 tokens): dH_pre and dH_res on MFMA;
//                    also packs W for B2 and writes the post gates for B1
//   k_bdots  (B1)    per (512 channels, sequence segment): TFA backward --
//                    dH_post partials, dout, conv-weight partials
//   k_bcoef          per token: reduce the dots, gates' and Sinkhorn's
//                    backward, dz, B2's per-tile record (dz/r, gates, gamma)
//   k_bgrad  (B2)    per (row group, 64 channels, token split): dX assembly
//                    with the dz W^T term on MFMA, dW partials on MFMA
//   k_reduce         deterministic reductions of the dW, db and dconv partials
#include "xhc_device.h"
#include "xhc_gs.h"
#include "xhc_launch.h"

namespace xhc {

struct Act4 { int id[4]; };

struct RowTable { int stream[5][4]; };   // row group -> 4 stream ids (-1 = none)

// ---------------------------------------------------------------------------
// W [NC, P] -> Wp [NC, 64], columns p >= P zero.
// ---------------------------------------------------------------------------

// B2's projection operand, elements [beg, end) of Wp [NC][64] from W [NC][P]
// (zero padded past P; with a router columns 48.. hold W_route), by `nth`
// threads of which this is `tid`.  Each thread's PK elements are loaded
// together (clamped, always valid addresses) before any is stored: one
// memory latency per PK elements instead of one per element.
template <typename R, bool ROUTE>
__device__ inline void pack_wp(const R* __restrict__ W, R* __restrict__ Wp, const R* __restrict__ Wr, int P, int N,
                               int64_t NC, int64_t beg, int64_t end, int tid, int nth) {
  constexpr int PK = 8;
  for (int64_t i0 = beg + tid; i0 < end; i0 += (int64_t)nth * PK) {
    R w[PK], wr[PK];
#pragma unroll
    for (int u = 0; u < PK; ++u) {
      const int64_t idx = i0 + (int64_t)u * nth;
      const int64_t j = min(idx >> 6, NC - 1);
      const int pp = (int)(idx & 63);
      w[u] = W[(size_t)j * P + min(pp, P - 1)];
      // (given per-token lists run this path without a router: no W_route)
      if constexpr (ROUTE) wr[u] = Wr ? Wr[(size_t)j * N + min(max(pp - 48, 0), N - 1)] : R(0);
    }
#pragma unroll
    for (int u = 0; u < PK; ++u) {
      const int64_t idx = i0 + (int64_t)u * nth;
      const int pp = (int)(idx & 63);
      R x = pp < P ? w[u] : R(0);
      if (ROUTE && pp >= 48) x = pp - 48 < N ? wr[u] : R(0);
      if (idx < end) Wp[idx] = x;
    }
  }
}

// ---------------------------------------------------------------------------
// The backward's preparation, ahead of the TFA backward:
//   blocks [0, nbg): post gates for B1, hpost[t][a*4 + m] = H_post[a][m],
//     recomputed from the saved logits as the forward computed them (routed
//     slots scaled by their scores), zero past k and nc; one thread per
//     entry (none when hpost is NULL);
//   the other blocks: B2's projection operand Wp (pack_wp), which nothing
//     reads before B2.
// Both are small; in one launch they cost one launch.
// ---------------------------------------------------------------------------
template <typename R, bool ROUTE>
__global__ __launch_bounds__(256) void k_bwd_prep(const float* __restrict__ zin, float* __restrict__ hpost, int T,
                                                  int N, int k, int P, int nc, int unit_gates, int zsv, int nfix,
                                                  int nbg, const R* __restrict__ W, R* __restrict__ Wp,
                                                  const R* __restrict__ Wr, int64_t NC) {
  if ((int)blockIdx.x < nbg) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= (int64_t)T * 16) return;
    const int64_t t = j >> 4;
    const int e = (int)(j & 15), a = e >> 2, m = e & 3;
    const float* zt = zin + (size_t)t * zsv;
    float h = 0.f;
    if (a < k && m < nc) h = unit_gates ? 1.f : sigmoid(zt[N + a * nc + m]);
    if (ROUTE && a >= nfix && a < k) h *= sigmoid(zt[P + 3 + 3 * (a - nfix)]);
    hpost[j] = h;
  } else {
    const int nbp = (int)gridDim.x - nbg, bp = (int)blockIdx.x - nbg;
    const int64_t nwp = NC * 64;
    const int64_t per = (nwp + nbp - 1) / nbp;
    const int64_t beg = (int64_t)bp * per, end = min(beg + per, nwp);
    pack_wp<R, ROUTE>(W, Wp, Wr, P, N, NC, beg, end, threadIdx.x, 256);
  }
}

// ---------------------------------------------------------------------------
// B1x.  The backward's state dots on MFMA.  Workgroup = (channel block of
// BX_CB = 8 x 64 channels, tile of BX_TOK tokens); wave w owns channels
// cb*BX_CB + 64w .. +64 (two K=32 steps).  Per token:
//   D[i][col] = sum_c X[t, i, c] B[c][col],  B columns = [dh_in, G_0..G_{k-1}, ...]
// so D[i][0] = dH_pre[i] and D[i_b][1+a] = dH_res[a][b] over the wave's
// channels (columns past k and rows past N are never read).  Each wave keeps
// the loads of RING-1 tokens in flight; the loop holds no global stores, so
// loads complete in order and the waits are exact.  Every BX_GRP tokens the
// 8 waves' partials are summed in LDS in a fixed order (deterministic) into
// the tile's result buffer, written out once at the end:
//   dpa[cb][t][0..16) = dH_pre,  dpa[cb][t][16 + a*4 + b] = dH_res[a][b].
// ROUTE: the active list is per token (route_idx, staged for the tile in
// LDS), B2's Wp gets the router's columns (W_route, stream i at column
// 48 + i) and the post gates of routed slots are scaled by their scores
// s = sigmoid(rho) from z_save's router record, as in the forward.
// ---------------------------------------------------------------------------
template <typename E, typename R, bool ROUTE>
__global__ __launch_bounds__(64 * BX_WAVES) void k_bxdots(StreamRows src, const void* __restrict__ dXn,
                                                          const void* __restrict__ dhin, float* __restrict__ dpa,
                                                          int T, int C, int N, int k, Act4 act, int ncb, int P,
                                                          const R* __restrict__ W, R* __restrict__ Wp, int64_t NC,
                                                          const int32_t* __restrict__ ridx,
                                                          const R* __restrict__ Wr, const void* __restrict__ xact,
                                                          int pack) {
  constexpr int EB = E::bytes;
  constexpr int RING = EB == 2 ? 4 : 2;
  static_assert(BX_GRP % RING == 0 && BX_TOK % BX_GRP == 0, "ring slots must be static in a group");
  __shared__ float red[BX_GRP][BX_WAVES][80];
  __shared__ float res[BX_TOK][BX_OUT];
  __shared__ int tid_s[BX_TOK][4];            // ROUTE: the tile's active lists

  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int cb = lb % ncb;
  const int tile = lb / ncb;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int c0 = cb * BX_CB + wave * BX_WCH;
  const int t0 = tile * BX_TOK;
  const int tn = min(BX_TOK, T - t0);

  // B2's projection operand, this workgroup's slice of it (when the
  // backward's preparation kernel has not packed it)
  if (pack) {
    const int64_t nwp = NC * 64;
    const int64_t per = (nwp + gridDim.x - 1) / gridDim.x;
    const int64_t beg = (int64_t)lb * per, end = min(beg + per, nwp);
    pack_wp<R, ROUTE>(W, Wp, Wr, P, N, NC, beg, end, threadIdx.x, 64 * BX_WAVES);
  }
  if constexpr (ROUTE) {
    for (int j = threadIdx.x; j < BX_TOK * 4; j += 64 * BX_WAVES) {
      const int tt = j >> 2, a = j & 3;
      int v = 0;
      if (tt < tn && a < k) v = ridx[(size_t)(t0 + tt) * k + a];
      tid_s[tt][a] = (unsigned)v < (unsigned)N ? v : 0;     // never a row outside the state
    }
    __syncthreads();
  }

  // A row r = stream r; B column r = dh_in (r = 0) or G_{r-1}
  const bool arow = r < N;
  const void* abase = src.base[arow ? r : 0];
  const int64_t astr = src.stride[arow ? r : 0];
  // (columns past k repeat G_0's row: their loads touch no further lines)
  const int brow = (!ROUTE && r >= 1) ? act.id[r <= k ? r - 1 : 0] : 0;
  const void* bbase = r == 0 ? dhin : dXn;
  const int64_t bstr = r == 0 ? (int64_t)C : (int64_t)N * C;
  const int64_t boff = r == 0 ? 0 : (int64_t)brow * C;
  int cofs[2];
  bool kv[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int cc = c0 + 32 * ks + 8 * g;
    kv[ks] = cc < C;
    cofs[ks] = kv[ks] ? cc : 0;
  }

  V8<E> av[RING][2], bv[RING][2];
  // token t0 + tt (clamped to the tile) -> ring slot q.  The ring holds the
  // loads as they arrive: channels past C are zeroed in A at the MFMA, not
  // here, since a select on a prefetched value would make the loop wait
  // for it where the ring is carried to the next group
  auto load = [&](int tt, int q) {
    const int ttc = min(tt, tn - 1);
    const int64_t t = t0 + ttc;
    int64_t bo = boff;
    const void* ab = abase;
    int64_t ao = t * astr;
    if constexpr (ROUTE) {
      bo = r >= 1 ? (int64_t)tid_s[ttc][r <= k ? min(r - 1, 3) : 0] * C : 0;
      if (xact) {
        // after an in-place forward, stream r's old row is saved at its slot
        int slot = -1;
#pragma unroll
        for (int a = 0; a < 4; ++a)
          if (a < k && tid_s[ttc][a] == r) slot = a;
        if (slot >= 0) { ab = xact; ao = (t * k + slot) * C; }
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      av[q][ks] = V8<E>::load(ab, (size_t)(ao + cofs[ks]));
      bv[q][ks] = V8<E>::load(bbase, (size_t)(t * bstr + bo + cofs[ks]));
    }
  };

  // this thread's entry of the cross-wave sums: D[i][0] = dH_pre[i] for
  // o < 16, D[i_b][1 + a] = dH_res[a][b] after (fixed lists: formed here
  // once -- indexing the by-value list with a run-time index reads the
  // kernel arguments from memory, and that load's wait in the loop would
  // also wait for the whole prefetch ring)
  int red_idx = -1;
  {
    const int o = threadIdx.x % BX_OUT;
    if (o < 16) {
      red_idx = o < N ? o : -1;
    } else if (!ROUTE) {
      const int a = (o - 16) >> 2, b = (o - 16) & 3;
      int ib = act.id[0];
#pragma unroll
      for (int bb = 1; bb < 4; ++bb)
        if (b == bb) ib = act.id[bb];
      red_idx = (a < k && b < k) ? (1 + a) * 16 + ib : -1;
    }
  }
#pragma unroll
  for (int q = 0; q < RING - 1; ++q) load(q, q);
  // every group of the tile runs (a short last tile works on copies of its
  // last token, whose sums are not written out), fully unrolled: at the head
  // of a loop the compiler cannot tell which ring slot each outstanding load
  // fills and waits for all of them, which drained the ring once per group
#pragma unroll
  for (int tg = 0; tg < BX_TOK; tg += BX_GRP) {
#pragma unroll
    for (int u = 0; u < BX_GRP; ++u) {
      const int q = u % RING;
      load(tg + u + RING - 1, (u + RING - 1) % RING);
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
      d = mma32(kv[0] ? av[q][0] : V8<E>::zero(), bv[q][0], d);
      d = mma32(kv[1] ? av[q][1] : V8<E>::zero(), bv[q][1], d);
      // lane (r, g) holds D[4g + e][r]: column r, rows 4g..4g+3
      if (r <= 4) *reinterpret_cast<f32x4*>(&red[u][wave][r * 16 + 4 * g]) = d;
    }
    __syncthreads();
    if (threadIdx.x < BX_GRP * BX_OUT) {
      const int u = threadIdx.x / BX_OUT, o = threadIdx.x % BX_OUT;
      int idx = red_idx;
      if (ROUTE && o >= 16) {
        const int a = (o - 16) >> 2, b = (o - 16) & 3;
        idx = (a < k && b < k) ? (1 + a) * 16 + tid_s[tg + u][b] : -1;   // D[i_b][1 + a]
      }
      float sum = 0.f;
      if (idx >= 0) {
#pragma unroll
        for (int w = 0; w < BX_WAVES; ++w) sum += red[u][w][idx];
      }
      res[tg + u][o] = sum;
    }
    __syncthreads();
  }
  for (int j = threadIdx.x; j < tn * BX_OUT; j += 64 * BX_WAVES)
    dpa[((size_t)cb * T + t0 + j / BX_OUT) * BX_OUT + j % BX_OUT] = res[j / BX_OUT][j % BX_OUT];
}

// ---------------------------------------------------------------------------
// B1.  TFA backward.  Workgroup = 4 waves on 4 consecutive 128-channel
// chunks of one sequence segment [s0, s1).  Per token (lane = 2 channels):
//   U_m from a 12-row window of `out`, dH_post partials (wave-reduced),
//   dU_m scattered into a 12-slot window of dout accumulators (anti-causal),
//   conv-weight partials.
// Both windows shift by one slot per token (slot 11 = current position).
// The segment is followed by an 11-token lookahead that only scatters dU
// into the segment's last dout positions.  The 4 waves' partial dH_post are
// summed in LDS once per 12 tokens and written per channel block.  All
// loads are unconditional (clamped addresses, masked values) and the next
// token's loads are issued before the current token's arithmetic.
//
// MODE selects the pass (Gram-Schmidt over the components, xhc_gs.h, needs
// the full-C inner products of the components before any gradient of them):
//   BD_FULL    no Gram-Schmidt: all of the above in one pass
//   BD_GSDOTS  <G_a, U_m> and the Gram record <U_m, U_n> only
//   BD_GSGRAD  dout and conv-weight partials from
//              dU_m = sum_a Ht[a][m] G_a + sum_n Sg[m][n] U_n,
//              Ht = H_post T and Sg from the coefficient backward; U is then
//              also formed for the lookahead tokens
//   BD_GRAM    (forward) the Gram record only; G is not read
// Dot records: dpart[cb][t][DOT_STRIDE] with <G_a, U_m> at 32 + 4a + m and
// the Gram record at 0..10 (BD_GRAM: dpart[cb][t][16], Gram at 0..10).
// ROUTE: the rows G_a come from each token's active list (route_idx; uniform
// scalar loads one token ahead of the loads they address).
// hpost holds each token's post coefficients (16 floats, a-major) every
// hstride floats: B1x's [T][16] gate records, or the coefficient records of
// the split backward's first call.
// ---------------------------------------------------------------------------
enum { BD_FULL = 0, BD_GSDOTS = 1, BD_GSGRAD = 2, BD_GRAM = 3 };
constexpr int GRAM_SPLIT = 8;   // segments of the forward Gram pass per backward segment

// Sum of 16 per-lane values over the wave by halving exchanges (lanes are
// paired by xor 32, 16, 15, 7, then quads are summed): afterwards lane l with
// l % 4 == 0 holds the sum of value reduce16_slot(l).
__device__ inline float wave_reduce16(float (&v)[16], int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = halve32(v[i], v[8 + i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = halve16(v[i], v[4 + i]);
  const bool h3 = lane & 8;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float send = h3 ? v[i] : v[2 + i];
    const float keep = h3 ? v[2 + i] : v[i];
    v[i] = keep + dpp_xor15(send);
  }
  const bool h2 = lane & 4;
  {
    const float send = h2 ? v[0] : v[1];
    const float keep = h2 ? v[1] : v[0];
    v[0] = keep + dpp_xor7(send);
  }
  v[0] += dpp_xor1(v[0]);
  v[0] += dpp_xor2(v[0]);
  return v[0];
}
__device__ inline int reduce16_slot(int lane) {
  return ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1);
}

template <typename E, int NCOMP, bool FAST, int MODE, bool ROUTE>
__global__ __launch_bounds__(256) void k_bdots(
    StreamRows src, const void* __restrict__ dXn, const void* __restrict__ dhin,
    const void* __restrict__ out, const float* __restrict__ w4, const float* __restrict__ w8,
    const float* __restrict__ w12, const float* __restrict__ hpost, const float* __restrict__ gsS,
    float* __restrict__ dpart, void* __restrict__ dout, float* __restrict__ dwpart, int T, int S, int C, int N,
    int kk, Act4 act, int lseg, int segs_per_seq, const int32_t* __restrict__ ridx, int hstride) {
  using V2 = Vec<E, B1_CH>;
  constexpr int EB = E::bytes;
  constexpr bool GS = MODE != BD_FULL;
  constexpr bool NEED_G = MODE != BD_GRAM;
  constexpr bool NEED_H = MODE == BD_FULL || MODE == BD_GSGRAD;
  constexpr bool DOTS = MODE == BD_FULL || MODE == BD_GSDOTS;       // <G_a, U_m>
  constexpr bool GRAMR = MODE == BD_GSDOTS || MODE == BD_GRAM;      // <U_m, U_n>
  constexpr bool GRAD = MODE == BD_FULL || MODE == BD_GSGRAD;       // dout, dw
  constexpr int NRED = (DOTS ? 16 : 0) + (GRAMR ? 16 : 0);
  constexpr int RSTRIDE = MODE == BD_GRAM ? 16 : DOT_STRIDE;
  static_assert(!GS || NCOMP == 4, "Gram-Schmidt needs the four components");
  __shared__ float red[B1_WAVES][12][NRED > 0 ? NRED : 1];
  const int k = FAST ? 4 : kk;
  (void)N;
  const int NS = FAST ? 16 : N;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cblock = blockIdx.x;
  const int c0 = (cblock * B1_WAVES + wave) * B1_WAVE_CH;
  const int seg = blockIdx.y;
  const int bseq = seg / segs_per_seq;
  const int s0 = (seg - bseq * segs_per_seq) * lseg;
  const int s1 = min(s0 + lseg, S);
  const int tend = GRAD ? s1 + 11 : s1;
  const size_t tok0 = (size_t)bseq * S;
  const uint32_t rowb = (uint32_t)C * EB;
  const uint32_t tokb = (uint32_t)NS * rowb;

  // TFA lane channels (clamped for idle lanes)
  const int clraw = c0 + B1_CH * lane;
  const bool cv = clraw < C;
  const int cl = cv ? clraw : 0;
  const uint32_t voff = (uint32_t)cl * EB;

  float wk[B1_CH][24];
  if constexpr (NCOMP == 4) {
#pragma unroll
    for (int ch = 0; ch < B1_CH; ++ch) {
#pragma unroll
      for (int q = 0; q < 4; ++q) wk[ch][q] = w4[(size_t)(cl + ch) * 4 + q];
#pragma unroll
      for (int q = 0; q < 8; ++q) wk[ch][4 + q] = w8[(size_t)(cl + ch) * 8 + q];
#pragma unroll
      for (int q = 0; q < 12; ++q) wk[ch][12 + q] = w12[(size_t)(cl + ch) * 12 + q];
    }
  }
  const rsrc_t rout = make_rsrc(static_cast<const char*>(out) + tok0 * rowb, (uint32_t)S * rowb);
  float win[12][B1_CH], dacc[12][B1_CH], dw[B1_CH][24];
#pragma unroll
  for (int j = 0; j < 12; ++j)
#pragma unroll
    for (int ch = 0; ch < B1_CH; ++ch) { win[j][ch] = 0.f; dacc[j][ch] = 0.f; }
#pragma unroll
  for (int ch = 0; ch < B1_CH; ++ch)
#pragma unroll
    for (int q = 0; q < 24; ++q) dw[ch][q] = 0.f;
  if constexpr (NCOMP == 4) {
#pragma unroll
    for (int j = 0; j < 11; ++j) {
      const int s = s0 - 11 + j;
      V2 v = bload<E, B1_CH>(rout, voff, (uint32_t)(s >= 0 ? s : 0) * rowb);
      float f[B1_CH];
      v.to_float(f);
#pragma unroll
      // ring slot of position s0-11+j; lanes past C hold zeros, as in the
      // loop, so that their components vanish in the Gram record
      for (int ch = 0; ch < B1_CH; ++ch) win[j][ch] = (s >= 0 && cv) ? f[ch] : 0.f;
    }
  }

  // loads of one token (clamped to the sequence) into ring slot q; the ring
  // keeps PF tokens of loads in flight
  constexpr int PF = 3;
  V2 gq[PF + 1][4], oq[PF + 1];
  int nid[4];                       // ROUTE: active list of the token loaded next
#pragma unroll
  for (int a = 0; a < 4; ++a) nid[a] = act.id[a < k ? a : 0];
  auto next_ids = [&](int s) {
    if constexpr (ROUTE && NEED_G) {
      const size_t t = tok0 + min(s, S - 1);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int v = ridx[t * k + (a < k ? a : 0)];
        nid[a] = (unsigned)v < (unsigned)NS ? v : 0;
      }
    }
  };
  // One buffer resource per row read, sized to the row, or to nothing for a
  // position past the sequence: lanes past C and such positions read zeros,
  // with no per-value selects in the token loop.  The second Gram-Schmidt
  // pass holds more uniform values (Sg), and there the extra resources
  // spill scalar registers: it reads through one resource per token and
  // masks the values instead (ZMASK).
  constexpr bool ZMASK = MODE == BD_GSGRAD;
  const uint32_t voffr = (uint32_t)clraw * EB;
  auto load_tok = [&](int s, int q) {
    const bool lv = s < S;
    const size_t t = tok0 + min(s, S - 1);
    if constexpr (ZMASK) {
      if constexpr (NEED_G) {
        const rsrc_t rg = make_rsrc(static_cast<const char*>(dXn) + t * tokb, tokb);
#pragma unroll
        for (int a = 0; a < 4; ++a) gq[q][a] = bload<E, B1_CH>(rg, voff, (uint32_t)nid[a] * rowb);
      }
      oq[q] = bload<E, B1_CH>(rout, voff, (uint32_t)min(s, S - 1) * rowb);
    } else {
      if constexpr (NEED_G) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const rsrc_t rg =
              make_rsrc(static_cast<const char*>(dXn) + t * tokb + (size_t)nid[a] * rowb, lv ? rowb : 0u);
          gq[q][a] = bload<E, B1_CH>(rg, voffr, 0);
        }
      }
      const rsrc_t ro = make_rsrc(static_cast<const char*>(out) + t * rowb, lv ? rowb : 0u);
      oq[q] = bload<E, B1_CH>(ro, voffr, 0);
    }
    next_ids(s + 1);
  };
  // post coefficients (and Sg) of one token (uniform: scalar loads), one token ahead
  float Hn[4][4], Sn[4][4];
  auto load_h = [&](int s) {
    if constexpr (NEED_H) {
      const size_t t = tok0 + min(s, S - 1);
      const f32x4* hp = reinterpret_cast<const f32x4*>(hpost + t * hstride);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 v = hp[a];
#pragma unroll
        for (int m = 0; m < 4; ++m) Hn[a][m] = v[m];
      }
      if constexpr (MODE == BD_GSGRAD) {
        const f32x4* sp = reinterpret_cast<const f32x4*>(gsS + t * 16);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f32x4 v = sp[m];
#pragma unroll
          for (int n = 0; n < 4; ++n) Sn[m][n] = v[n];
        }
      }
    }
  };
  next_ids(s0);
#pragma unroll
  for (int q = 0; q < PF; ++q) load_tok(s0 + q, q);
  load_h(s0);

  // Tokens go in groups of 12 aligned to s0, fully unrolled, so that both
  // 12-slot windows are rings with static slots: at group position j,
  //   `out` of position s - 11 + i sits in win[(j + i) % 12]  (i = 11: s)
  //   the dout accumulator of position s - 11 + i in dacc[(j + 1 + i) % 12].
  // Positions completed during a group are held in registers and stored at
  // the group's end, so that the loop issues no store between a load and its
  // use (loads and stores share one completion counter).
  for (int sg = s0; sg < tend; sg += 12) {
    V2 pend[12];
    static_for<0, 12>([&](auto J) {
      constexpr int j = decltype(J)::value;
      constexpr int q = j % (PF + 1);
      const int s = sg + j;
      const bool main_tok = s < s1;
      const bool in_seg = s < tend;
      const bool live = s < S;
      load_tok(s + PF, (j + PF) % (PF + 1));
      float H[4][4], Sg[4][4];
      if constexpr (NEED_H) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            H[a][m] = Hn[a][m];
            if constexpr (MODE == BD_GSGRAD) Sg[a][m] = Sn[a][m];
          }
        load_h(s + 1);
      }

      float G[4][B1_CH], of[B1_CH];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if constexpr (NEED_G) {
          gq[q][a].to_float(G[a]);
        }
        if (!NEED_G || !(a < k && (!ZMASK || (cv && live)))) {
#pragma unroll
          for (int ch = 0; ch < B1_CH; ++ch) G[a][ch] = 0.f;
        }
      }
      oq[q].to_float(of);

      // U of this token: main tokens, and in BD_GSGRAD the lookahead too
      const bool need_u = MODE == BD_GSGRAD ? in_seg : main_tok;
      float U[4][B1_CH];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int ch = 0; ch < B1_CH; ++ch) U[m][ch] = 0.f;
      if (need_u) {
#pragma unroll
        for (int ch = 0; ch < B1_CH; ++ch) win[(j + 11) % 12][ch] = (!ZMASK || cv) ? of[ch] : 0.f;
#pragma unroll
        for (int ch = 0; ch < B1_CH; ++ch) {
          U[0][ch] = win[(j + 11) % 12][ch];
          if constexpr (NCOMP == 4) {
            float s4 = 0.f, s8 = 0.f, s12 = 0.f;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) s4 = fmaf(wk[ch][qq], win[(j + 8 + qq) % 12][ch], s4);
#pragma unroll
            for (int qq = 0; qq < 8; ++qq) s8 = fmaf(wk[ch][4 + qq], win[(j + 4 + qq) % 12][ch], s8);
#pragma unroll
            for (int qq = 0; qq < 12; ++qq) s12 = fmaf(wk[ch][12 + qq], win[(j + qq) % 12][ch], s12);
            U[1][ch] = s4; U[2][ch] = s8; U[3][ch] = s12;
          }
        }
      }
      if (main_tok) {
        if constexpr (DOTS) {
          // dH_post partials v[a*4+m]
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
          const float r = wave_reduce16(v, lane);
          if ((lane & 3) == 0) red[wave][j][reduce16_slot(lane)] = r;
        }
        if constexpr (GRAMR) {
          // Gram record partials (entries 10..15 are zero)
          float v[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) v[i] = 0.f;
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = m; n < 4; ++n) {
              float d = 0.f;
#pragma unroll
              for (int ch = 0; ch < B1_CH; ++ch) d = fmaf(U[m][ch], U[n][ch], d);
              v[gram_idx(m, n)] = d;
            }
          const float r = wave_reduce16(v, lane);
          if ((lane & 3) == 0) red[wave][j][(DOTS ? 16 : 0) + reduce16_slot(lane)] = r;
        }
      }
      if constexpr (GRAD) {
        // dU_m for this token (zero for tokens past the sequence)
        float dU[4][B1_CH];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int ch = 0; ch < B1_CH; ++ch) {
            float d = 0.f;
            if (m < NCOMP) {
#pragma unroll
              for (int a = 0; a < 4; ++a)
                if (a < k) d = fmaf(H[a][m], G[a][ch], d);
              if constexpr (MODE == BD_GSGRAD) {
                float e = 0.f;
#pragma unroll
                for (int n = 0; n < 4; ++n) e = fmaf(Sg[m][n], U[n][ch], e);
                d += (live && (!ZMASK || cv)) ? e : 0.f;   // U past the sequence still sees real ones
              }
            }
            dU[m][ch] = d;
          }
        if (main_tok && NCOMP == 4) {
#pragma unroll
          for (int ch = 0; ch < B1_CH; ++ch) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) dw[ch][qq] = fmaf(dU[1][ch], win[(j + 8 + qq) % 12][ch], dw[ch][qq]);
#pragma unroll
            for (int qq = 0; qq < 8; ++qq)
              dw[ch][4 + qq] = fmaf(dU[2][ch], win[(j + 4 + qq) % 12][ch], dw[ch][4 + qq]);
#pragma unroll
            for (int qq = 0; qq < 12; ++qq)
              dw[ch][12 + qq] = fmaf(dU[3][ch], win[(j + qq) % 12][ch], dw[ch][12 + qq]);
          }
        }
        if (in_seg) {
          // scatter into the dout accumulators of positions s - lag (positions
          // before s0 receive terms too; they are never emitted)
          if (main_tok) {
#pragma unroll
            for (int ch = 0; ch < B1_CH; ++ch) dacc[j % 12][ch] += dU[0][ch];
          }
          if constexpr (NCOMP == 4) {
#pragma unroll
            for (int lag = 0; lag < 12; ++lag) {
#pragma unroll
              for (int ch = 0; ch < B1_CH; ++ch) {
                float d = dacc[(j + 12 - lag) % 12][ch];
                if (lag < 4) d = fmaf(wk[ch][3 - lag], dU[1][ch], d);
                if (lag < 8) d = fmaf(wk[ch][4 + 7 - lag], dU[2][ch], d);
                d = fmaf(wk[ch][12 + 11 - lag], dU[3][ch], d);
                dacc[(j + 12 - lag) % 12][ch] = d;
              }
            }
          }
        }
        // position s - 11 is complete: hold it for the group's store, clear its slot
        pend[j] = V2::from_float(dacc[(j + 1) % 12]);
#pragma unroll
        for (int ch = 0; ch < B1_CH; ++ch) dacc[(j + 1) % 12][ch] = 0.f;
      }
    });
    // group end: completed positions sg - 11 .. sg (those in [s0, s1)) and
    // the waves' dot sums of the group's main tokens
    if constexpr (GRAD) {
      if (cv) {
#pragma unroll
        for (int j = 0; j < 12; ++j) {
          const int pos = sg + j - 11;
          if (pos >= s0 && pos < s1) pend[j].store(dout, (tok0 + pos) * C + cl);
        }
      }
    }
    if constexpr (NRED > 0) {
      if (sg < s1) {
        __syncthreads();
        const int nmain = min(12, s1 - sg);
        for (int idx = threadIdx.x; idx < nmain * NRED; idx += 64 * B1_WAVES) {
          const int jj = idx / NRED, q = idx - jj * NRED;
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < B1_WAVES; ++w) sum += red[w][jj][q];
          // q < 16 with DOTS: <G_a, U_m>; otherwise the Gram record
          const int col = (DOTS && q < 16) ? 32 + q : q - (DOTS ? 16 : 0);
          if (!(GRAMR && col < 16 && col >= 10))
            dpart[((size_t)cblock * T + tok0 + sg + jj) * RSTRIDE + col] = sum;
        }
        __syncthreads();
      }
    }
  }
  if constexpr (GRAD) {
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
}

// ---------------------------------------------------------------------------
// Coefficient backward.  16 lanes per token, lane e owns pre slot e, post
// slot (a, m) = (e/4, e%4) and Sinkhorn entry (a, b) = (e/4, e%4).  The
// Sinkhorn iterates after every column step are kept in LDS and walked back:
//   column step Mc = R / colsum(R):  dR = (dMc - colsum(dMc*Mc)) / colsum(R)
//   row step    R  = M / rowsum(M):  dM = (dR - rowsum(dR*R))  / rowsum(M)
//   dL = dM_0 * M_0 (the row-max shift cancels in the first row step).
// With Gram-Schmidt (GS, xhc_gs.h) the B1 dots are D[a][m] = <G_a, U_m> over
// the raw components, and with u~ = T U:
//   dH_post[a][c] = sum_m T[c][m] D[a][m]
//   dT[c][m]      = sum_a H_post[a][c] D[a][m]   -> Sg = dg + dg^T
// and the kernel writes, for the second B1 pass, Ht = H_post T over hpost
// and Sg to gss ([T][16] each), so that dU_m = sum_a Ht[a][m] G_a +
// sum_n Sg[m][n] U_n.
// ---------------------------------------------------------------------------
constexpr int BCOEF_TOK = 16;   // tokens per workgroup (16 lanes each)

// ROUTE: the routed slots' write-back scale s_a = sigmoid(rho_a) enters as
// in the forward (the effective post coefficient is s_a H_post[a, m]); with
// dq[a, m] the gradient of that coefficient, dH_post = s_a dq and
// ds_a = sum_m H_post[a, m] dq[a, m], drho_a = ds_a s_a (1 - s_a).  The
// LayerNorm backward, with dy = drho W_route^T, y = (x - mean) / sd,
//   dx = dy / sd - mean(dy) / sd - (x - mean) mean(dy y) / sd^2,
//   mean(dy) = sum_a drho_a colsum_a / NC,  mean(dy y) = sum_a drho_a (rho_a - b_a) / NC,
// goes to B2 as: the router's logit columns of its record (drho / sd at
// column 48 + stream), gamma += mean(dy y) / sd^2 and a constant
// mean * mean(dy y) / sd^2 - mean(dy) / sd added to every element.  dz_out
// (DZ_R floats per token) also gets drho and mean * drho / sd per stream for
// db_route and for dW_route's mean term; hres gets H_res for the pass kernel.
template <typename E, bool GS, bool ROUTE>
__global__ __launch_bounds__(16 * BCOEF_TOK) void k_bcoef(const float* __restrict__ dpa, int ncba, const float* __restrict__ dpart,
                                              int ncb, const float* __restrict__ zin,
                                              const float* __restrict__ bias,
                                              float* __restrict__ dz_out, void* __restrict__ rec,
                                              int T, int64_t Tpad, int N, int k, int nc,
                                              int P, float inv_nc_total, int iters, int unit_gates,
                                              float gs_ceps, float* __restrict__ hpost, float* __restrict__ gss,
                                              int zsv, int dzstride, const int32_t* __restrict__ ridx, int nfix,
                                              float* __restrict__ hres, int has_router, HresActive ha) {
  extern __shared__ float hist[];   // [BCOEF_TOK][iters+1][16]
  __shared__ float dzs[BCOEF_TOK][64];
  const int e = threadIdx.x & 15, tok = threadIdx.x >> 4;
  const int64_t t = (int64_t)blockIdx.x * BCOEF_TOK + tok;
  const bool tv = t < T;
  const int64_t tc = tv ? t : 0;
  float* H = hist + (size_t)tok * (iters + 1) * 16;

  // reduce the per-chunk dots
  float dpre = 0.f, dres = 0.f, dpost = 0.f;
  #pragma unroll 8
  for (int cb = 0; cb < ncba; ++cb) {
    const float* d = dpa + ((size_t)cb * T + tc) * BX_OUT;
    dpre += d[e];
    dres += d[16 + e];
  }
  #pragma unroll 8
  for (int cb = 0; cb < ncb; ++cb) dpost += dpart[((size_t)cb * T + tc) * DOT_STRIDE + 32 + e];
  const float* z = zin + tc * zsv;
  const float r = z[P];
  const float r_act = ha.mask ? z[P + 1] : r;     // hres_active: the res logits' normaliser

  // gates (recomputed from the logits, as the forward computed them)
  const bool pre_ok = e < N;
  const bool post_ok = (e >> 2) < k && (e & 3) < nc;
  const float hp = pre_ok ? (unit_gates ? 1.f : sigmoid(z[e])) : 0.f;
  const float hq = post_ok ? (unit_gates ? 1.f : sigmoid(z[N + (e >> 2) * nc + (e & 3)])) : 0.f;
  // routed slots' scores and write-back scales (1 for fixed slots)
  float sa[4];
  int sid[4];
#pragma unroll
  for (int a2 = 0; a2 < 4; ++a2) {
    sa[a2] = 1.f;
    sid[a2] = 0;
    if constexpr (ROUTE) {
      if (a2 >= nfix && a2 < k) sa[a2] = sigmoid(z[P + 3 + 3 * (a2 - nfix)]);
      if (a2 < k) {
        const int v = ridx[(size_t)tc * k + a2];
        sid[a2] = (unsigned)v < (unsigned)N ? v : 0;
      }
    }
  }
  float my_s = sa[0];
#pragma unroll
  for (int a2 = 1; a2 < 4; ++a2)
    if ((e >> 2) == a2) my_s = sa[a2];
  if constexpr (GS) {
    // the token's 16 lanes share one wave: gather its records
    float gsum = 0.f;
    if (e < 10)
      #pragma unroll 8
      for (int cb = 0; cb < ncb; ++cb) gsum += dpart[((size_t)cb * T + tc) * DOT_STRIDE + e];
    const int base = (threadIdx.x & 63) & ~15;
    float g[4][4], D[4][4], Hp[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        if (n >= m) {
          g[m][n] = __shfl(gsum, base + gram_idx(m, n), 64);
          g[n][m] = g[m][n];
        }
        D[m][n] = __shfl(dpost, base + m * 4 + n, 64);
        Hp[m][n] = __shfl(hq, base + m * 4 + n, 64) * sa[m];    // the effective coefficients
      }
    GsFwd f;
    gs_forward(g, gs_ceps, f);
    float dT[4][4], Sg[4][4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float v = 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a) v = fmaf(Hp[a][c], D[a][m], v);
        dT[c][m] = v;
      }
    gs_backward(g, f, dT, Sg);
    const int a = e >> 2, q = e & 3;
    float dh = 0.f, ht = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) dh = fmaf(f.T[q][m], D[a][m], dh);
#pragma unroll
    for (int c = 0; c < 4; ++c) ht = fmaf(Hp[a][c], f.T[c][q], ht);
    float sv = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        if (m == a && n == q) sv = Sg[m][n];
    dpost = dh;
    if (tv) {
      hpost[t * 16 + e] = ht;
      gss[t * 16 + e] = sv;
    }
  } else {
    (void)gs_ceps; (void)hpost; (void)gss;
  }
  // dpost is now the gradient of the effective post coefficient s_a H_post
  float dz_pre = 0.f, dz_post = 0.f;
  if (!unit_gates) {
    dz_pre = pre_ok ? dpre * hp * (1.f - hp) : 0.f;
    dz_post = post_ok ? (ROUTE ? my_s * dpost : dpost) * hq * (1.f - hq) : 0.f;
  }
  // router: drho per slot, then per stream
  float drs = 0.f, gam_r = 0.f, cst = 0.f;   // this lane's stream: drho; LN gamma and constant
  float rmu = 0.f, rsd = 1.f;
  if constexpr (ROUTE) {
    float v = hq * dpost;                    // ds_a over the quad of lanes of row a
    v += row_xor<1>(v);
    v += row_xor<2>(v);
    const int base = (threadIdx.x & 63) & ~15;
    if (has_router) {                        // (given lists: no router record, no routed slots)
      rmu = z[P + 1];
      rsd = z[P + 2];
    }
    float m1 = 0.f, m2 = 0.f;
#pragma unroll
    for (int a2 = 0; a2 < 4; ++a2) {
      const float ds = __shfl(v, base + 4 * a2, 64);
      if (a2 >= nfix && a2 < k) {
        const float dr = ds * sa[a2] * (1.f - sa[a2]);
        const int j = a2 - nfix;
        m1 = fmaf(dr, z[P + 5 + 3 * j], m1);
        m2 = fmaf(dr, z[P + 4 + 3 * j], m2);
        if (sid[a2] == e) drs += dr;
      }
    }
    m1 *= inv_nc_total;
    m2 *= inv_nc_total;
    const float isd = 1.f / rsd;
    gam_r = m2 * isd * isd;
    cst = rmu * gam_r - m1 * isd;
  }

  // Sinkhorn backward
  const int a = e >> 2, b = e & 3;
  const bool valid = a < k && b < k;
  {
    const float L = valid ? z[N + k * nc + a * k + b] : -INFINITY;
    float mx = fmaxf(L, row_xor<1>(L));
    mx = fmaxf(mx, row_xor<2>(mx));
    float M = valid ? expf(L - mx) : 0.f;
    H[e] = M;
    for (int it = 0; it < iters; ++it) {
      float rs = M + row_xor<1>(M);
      rs += row_xor<2>(rs);
      M = valid ? M / rs : 0.f;
      float cs = M + row_xor<4>(M);
      cs += row_xor<8>(cs);
      M = valid ? M / cs : 0.f;
      H[(it + 1) * 16 + e] = M;
    }
  }
  float g = valid ? dres : 0.f;
  for (int it = iters; it >= 1; --it) {
    const float Mp = H[(it - 1) * 16 + e];
    float rs = Mp + row_xor<1>(Mp);
    rs += row_xor<2>(rs);
    const float R = valid ? Mp / rs : 0.f;
    float cs = R + row_xor<4>(R);
    cs += row_xor<8>(cs);
    const float Mc = valid ? R / cs : 0.f;
    float t1 = g * Mc;
    t1 += row_xor<4>(t1);
    t1 += row_xor<8>(t1);
    const float gR = valid ? (g - t1) / cs : 0.f;
    float t2 = gR * R;
    t2 += row_xor<1>(t2);
    t2 += row_xor<2>(t2);
    g = valid ? (gR - t2) / rs : 0.f;
  }
  const float dL = g * H[e];
  if (ROUTE && tv) hres[t * 16 + e] = H[iters * 16 + e];

  // assemble dz in the logit column layout
  dzs[tok][e] = 0.f; dzs[tok][16 + e] = 0.f; dzs[tok][32 + e] = 0.f; dzs[tok][48 + e] = 0.f;
  __syncthreads();
  if (e < N) dzs[tok][e] = dz_pre;
  if (a < k && b < nc) dzs[tok][N + a * nc + b] = dz_post;
  if (valid) dzs[tok][N + k * nc + a * k + b] = dL;
  __syncthreads();

  // gamma = dz.(z - bias) / (N*C*r^2); with hres_active the res logits'
  // share goes to gamma_act = dz_res.(z_res - bias) / (k*C*r_act^2), which
  // only the active rows receive
  float al = 0.f, al_act = 0.f;
#pragma unroll
  for (int n = 0; n < 3; ++n) {
    const int p = e + 16 * n;
    const float v = p < P ? dzs[tok][p] * (z[p] - (bias ? bias[p] : 0.f)) : 0.f;
    if (ha.mask && p >= ha.res0 && p < ha.res1) al_act += v;
    else al += v;
  }
  al += row_xor<1>(al);
  al += row_xor<2>(al);
  al += row_xor<4>(al);
  al += row_xor<8>(al);
  al_act += row_xor<1>(al_act);
  al_act += row_xor<2>(al_act);
  al_act += row_xor<4>(al_act);
  al_act += row_xor<8>(al_act);
  const float inv_r = 1.f / r;
  const float inv_ra = 1.f / r_act;
  if (tv) {
#pragma unroll
    for (int n = 0; n < 3; ++n) dz_out[t * dzstride + e + 16 * n] = dzs[tok][e + 16 * n];
    if constexpr (ROUTE) {
      dz_out[t * dzstride + 48 + e] = drs;
      dz_out[t * dzstride + 64 + e] = rmu * drs / rsd;
    }
  }
  // B2's tile record (layout next to REC_BYTES); t in [T, Tpad) is written
  // as zeros.  In bf16 mode dz/r is stored as hi and lo bf16 halves: the dz
  // values of saturated Sinkhorn entries are large, and the products must
  // keep fp32 accuracy.
  if (t < Tpad) {
    constexpr int EB = E::bytes;
    constexpr int NT_REC = ROUTE ? 4 : 3;
    unsigned char* rb = static_cast<unsigned char*>(rec) + (size_t)(t / B2_TT) * (ROUTE ? REC_R_BYTES : REC_BYTES);
    const int tt = (int)(t % B2_TT);
#pragma unroll
    for (int n = 0; n < NT_REC; ++n) {
      const int p = e + 16 * n;                      // logits 0..47 (router: 48..63 = drho / sd per stream)
      const float inv_n = (ha.mask && p >= ha.res0 && p < ha.res1) ? inv_ra : inv_r;
      const float v = tv ? (n < 3 ? dzs[tok][p] * inv_n : drs / rsd) : 0.f;
      size_t o_dzr, dzr_half;
      if (p < 32) {
        o_dzr = REC_DZR0 + ((size_t)(((p >> 3) * 16 + tt) * 8 + (p & 7))) * EB;
        dzr_half = rec_dzr0_half(EB);
      } else if (ROUTE) {
        o_dzr = RR_DZR1 + ((size_t)((((p - 32) >> 3) * 16 + tt) * 8 + ((p - 32) & 7))) * EB;
        dzr_half = rec_dzr0_half(EB);
      } else {
        o_dzr = REC_DZR1 + ((size_t)((((p - 32) >> 2) * 16 + tt) * 4 + ((p - 32) & 3))) * EB;
        dzr_half = rec_dzr1_half(EB);
      }
      const int pt = p >> 4, rr = p & 15, gt = tt >> 2, e4 = tt & 3;
      const size_t o_dzrt = (ROUTE ? RR_DZRT : REC_DZRT) + ((size_t)((pt * 4 + gt) * 16 + rr) * 4 + e4) * EB;
      const size_t dzrt_half = (size_t)NT_REC * 4 * 16 * 4 * EB;
      if constexpr (EB == 2) {
        __bf16 hi, lo;
        split_bf16(v, hi, lo);
        *reinterpret_cast<__bf16*>(rb + o_dzr) = hi;
        *reinterpret_cast<__bf16*>(rb + o_dzr + dzr_half) = lo;
        *reinterpret_cast<__bf16*>(rb + o_dzrt) = hi;
        *reinterpret_cast<__bf16*>(rb + o_dzrt + dzrt_half) = lo;
      } else {
        *reinterpret_cast<float*>(rb + o_dzr) = v;
        *reinterpret_cast<float*>(rb + o_dzrt) = v;
      }
    }
    const float gam = al * inv_nc_total * inv_r * inv_r + gam_r;
    if constexpr (ROUTE) {
      float* rco = reinterpret_cast<float*>(rb + RR_CO);
      rco[(RRF_PRE + e) * B2_TT + tt] = tv ? hp : 0.f;
      if (e < RRF_NF - RRF_GAMMA)
        rco[(RRF_GAMMA + e) * B2_TT + tt] = tv ? (e == 0 ? gam : e == 1 ? cst : 0.f) : 0.f;
    } else {
      float* rco = reinterpret_cast<float*>(rb + REC_CO);
      rco[(RF_PRE + e) * B2_TT + tt] = tv ? hp : 0.f;
      rco[(RF_RES + e) * B2_TT + tt] = tv ? H[iters * 16 + e] : 0.f;
      const float gam_act = al_act * ha.inv_kc * inv_ra * inv_ra;
      if (e < REC_NF - RF_GAMMA)
        rco[(RF_GAMMA + e) * B2_TT + tt] = tv ? (e == 0 ? gam : e == 1 ? gam_act : 0.f) : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// B2.  Workgroup = (row group, B2_CB = 64 channels, token split), 8 waves:
// wave w computes row w%4 of the group on channel half w/4.  Its loads and
// stores instead cover token half w/4 of the tile in whole 128-byte lines
// (both channel halves), exchanged with the other wave of the row through
// the LDS row tiles: an instruction that reads or writes half lines, the
// other half coming from another wave, moves HBM data markedly slower.
// Per tile of B2_TT = 16 tokens:
//   proj[c][t] = sum_p W[i*C+c, p] dz_r[t, p] on MFMA (dz/r as bf16 hi + lo),
//   with A rows permuted so that lane (t = lane%16, g = lane/16) ends up
//   owning channels 8g..8g+8 of token t -- the layout of its row tile slots;
//   dX = pass + H_pre dh_in + proj - X gamma;
//   dW[i*C+c][p] += sum_t X[t, c] dz_r[t, p] on MFMA (K = the tile's tokens,
//   A = X^T through LDS).
// The tile's shared operands (dz/r in both fragment orders, the coefficients)
// arrive as one contiguous record in LDS order, copied global -> LDS by the
// LDS-DMA form of the load one tile ahead (double-buffered); each lane
// prefetches its own state, dX_new and dh_in pieces one tile ahead.  A
// tile's dX is stored at the start of the next iteration, ahead of that
// iteration's prefetch, so the wait at the top of the loop never waits on a
// store issued after the loads it needs (the routed form stores the first
// tile of a step as soon as it is done).  The active rows' upstream
// gradients G_a are exchanged through LDS; all of a tile's rows are read (a
// tile earlier) before any is written, so dX may alias dX_new.
// ROUTE: the active rows differ per token, so the row groups are simply
// streams 4g..4g+3, and a lane's "pass" row is either dX_new[t, i] (i not
// active for its token) or pass[t][b] = sum_a H_res[a, b] G_a (i = i_b),
// formed beforehand by k_route_pass; the choice is made per lane from the
// token's active list (loaded one step ahead of the addresses it selects).
// The projection's K is 64 (the router's logit columns 48.. carry
// drho / sd), dX also receives the LayerNorm constant, and dW has a fourth
// 16-column tile (the router's, rows of 64 partials).
// ---------------------------------------------------------------------------
template <typename E> struct B2Lds {
  static constexpr int EB = E::bytes;
  // per-wave row tiles ([g][t] x 8 elements, group stride padded by 16 B)
  static constexpr int GSTRIDE = 16 * 8 * EB + 16;
  static constexpr int ROWTILE = 4 * GSTRIDE;
};

// LDS of the row-group body: the double-buffered tile records with the dh_in
// blocks, then the published dX_new and X row tiles.
template <typename E, bool ROUTE>
constexpr int bgrad_sbuf() {
  return (ROUTE ? REC_R_USED : REC_USED) + B2_TT * B2_CB * E::bytes;
}
template <typename E, bool ROUTE>
constexpr int bgrad_lds_bytes() {
  return 2 * B2_SUB * bgrad_sbuf<E, ROUTE>() + 2 * B2_SUB * B2_WAVES * B2Lds<E>::ROWTILE;
}

template <typename E, bool ROUTE>
__device__ __forceinline__ void bgrad_body(
    StreamRows src, const void* __restrict__ dXn, const void* __restrict__ dhin, const void* __restrict__ Wp,
    const unsigned char* __restrict__ rec, int ntiles, void* dX, float* __restrict__ dwp, int T, int C, int N, int k,
    RowTable rows, int rg, int cb, int ts, int tok_per_split, const void* __restrict__ passbuf,
    const int32_t* __restrict__ ridx, const void* __restrict__ xact, int wz0, int wz1, unsigned char* smem) {
  constexpr bool BF = E::bytes == 2;
  constexpr int EB = E::bytes;
  using LY = B2Lds<E>;
  constexpr int RUSED = ROUTE ? REC_R_USED : REC_USED;     // record bytes copied to LDS
  constexpr int RSTRIDE = ROUTE ? REC_R_BYTES : REC_BYTES; // record bytes per tile
  constexpr int RCO = ROUTE ? RR_CO : REC_CO;
  constexpr int RDZRT = ROUTE ? RR_DZRT : REC_DZRT;
  constexpr int NPT = ROUTE ? 4 : 3;                       // 16-logit tiles of dz/r
  constexpr int F_PRE = ROUTE ? RRF_PRE : RF_PRE;
  constexpr int F_GAMMA = ROUTE ? RRF_GAMMA : RF_GAMMA;
  constexpr int DHB = B2_TT * B2_CB * EB;              // dh_in block of one tile ([t][B2_CB])
  constexpr int SBUF = RUSED + DHB;                    // LDS bytes of one tile's shared operands
  constexpr int NREC = (RUSED + 1023) / 1024;          // wave-wide copies of the record (last one partial)
  constexpr int NCH = NREC + DHB / 1024;
  constexpr int STEP = B2_TT * B2_SUB;
  static_assert(RUSED % 16 == 0 && DHB % 1024 == 0 && RUSED <= RSTRIDE, "record copy split");
  static_assert(SBUF == bgrad_sbuf<E, ROUTE>(), "LDS layout");
  typedef unsigned char RbufT[B2_SUB][SBUF];
  typedef unsigned char RowT[B2_WAVES][LY::ROWTILE];
  RbufT* rbuf = reinterpret_cast<RbufT*>(smem);                                     // [2] tile records + dh_in
  RowT* gsh = reinterpret_cast<RowT*>(smem + 2 * B2_SUB * SBUF);                    // [B2_SUB] dX_new rows
  RowT* xsh = reinterpret_cast<RowT*>(smem + 2 * B2_SUB * SBUF + B2_SUB * sizeof(RowT));   // [B2_SUB] X rows

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: rsrc and M0 stay scalar
  const int slot = wave & 3, chalf = wave >> 2;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int stream = rows.stream[rg][slot];
  const bool wv = stream >= 0;
  const int srow = wv ? stream : 0;
  const bool active_grp = !ROUTE && rg == 0;
  const int c0 = cb * B2_CB + chalf * B2_WAVE_CH;   // this wave's channels c0 .. c0+32
  const int64_t NCs = (int64_t)N * C;
  const size_t jbase = (size_t)srow * C + c0;
  const int cl = c0 + 8 * g4;                        // this lane's 8 channels (in the row tiles)
  const uint32_t tokb = (uint32_t)N * C * EB;        // bytes of one token's state

  // proj A operand: W rows, permuted: A row m of j-tile jt -> channel
  // 8*(m/4) + 4*jt + m%4 ; K = 48 logits as a K=32 step (wa) and a K=16
  // step (wb)
  // (ROUTE: K = 64 as two K=32 steps, wa and wc)
  V8<E> wa[2], wc[2];
  Vec<E, 4> wb[2];
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    const int ch = 8 * (r16 >> 2) + 4 * jt + (r16 & 3);
    const bool ok = wv && c0 + ch < C;
    const size_t row = (ok ? jbase + ch : 0) * 64;
    const V8<E> va = V8<E>::load(Wp, row + 8 * g4);
    wa[jt] = ok ? va : V8<E>::zero();
    if constexpr (ROUTE) {
      const V8<E> vc = V8<E>::load(Wp, row + 32 + 8 * g4);
      wc[jt] = ok ? vc : V8<E>::zero();
    } else {
      const Vec<E, 4> vb = Vec<E, 4>::load(Wp, row + 32 + 4 * g4);
      wb[jt] = ok ? vb : Vec<E, 4>::zero();
    }
  }
  if (!ROUTE && !active_grp && wz0 < wz1) {
    // hres_active: the res logits [wz0, wz1) do not read the untouched rows
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      float fa[8], fb[4];
      wa[jt].to_float(fa);
      wb[jt].to_float(fb);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (8 * g4 + j >= wz0 && 8 * g4 + j < wz1) fa[j] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (32 + 4 * g4 + j >= wz0 && 32 + 4 * g4 + j < wz1) fb[j] = 0.f;
      wa[jt] = V8<E>::from_float(fa);
      wb[jt] = Vec<E, 4>::from_float(fb);
    }
  }
  f32x4 dwacc[2][NPT];
#pragma unroll
  for (int jt = 0; jt < 2; ++jt)
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) dwacc[jt][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const void* xbase = src.base[srow];
  const int64_t xstride = src.stride[srow];
  const int tbeg = ts * tok_per_split;
  const int tfin = min(tbeg + tok_per_split, T);

  // The B2_SUB tiles from t0 -> rbuf[b]: each tile's record, then this
  // workgroup's dh_in block, by wave-wide 16-byte LDS-DMA copies of 1 KiB
  // (the record's last copy is partial).  Every copy goes through a buffer
  // resource based at its tile whose size ends at the data's end, so tiles
  // and tokens past the end read zeros.
  const uint32_t dhrowb = (uint32_t)C * EB;
  auto dma = [&](int t0, int b) {
#pragma unroll
    for (int s = 0; s < B2_SUB; ++s) {
      const int ta = t0 + s * B2_TT;
      const int tile = ta / B2_TT;
      const rsrc_t rrec = make_rsrc(rec + (size_t)tile * RSTRIDE, tile < ntiles ? (uint32_t)RSTRIDE : 0u);
      const rsrc_t rdh = make_rsrc(static_cast<const char*>(dhin) + (size_t)ta * dhrowb,
                                   clamp_bytes(ta < T ? T - ta : 0, dhrowb));
#pragma unroll
      for (int q = 0; q < (NCH + B2_WAVES - 1) / B2_WAVES; ++q) {
        const int c = wave + q * B2_WAVES;
        if (c < NREC) {
          if (c * 1024 + lane * 16 < RUSED)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rrec, (lds_void_t*)&rbuf[b][s][c * 1024], 16,
                                                     c * 1024 + lane * 16, 0, 0, 0);
        } else if (c < NCH) {
          constexpr int PPT = B2_CB * EB / 16;             // 16-byte pieces per token
          const int e = (c - NREC) * 64 + lane;
          const uint32_t voff = ((uint32_t)(e / PPT) * C + cb * B2_CB + (e % PPT) * (16 / EB)) * EB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rdh, (lds_void_t*)&rbuf[b][s][RUSED + (c - NREC) * 1024], 16,
                                                   voff, 0, 0, 0);
        }
      }
    }
  };
  // own rows of the B2_SUB tiles from t0 (tokens past the end read zeros,
  // or are masked when published).  These are the pass's last reads of the
  // state, of dX_new and of the pass rows: non-temporal.  The two waves of a
  // row split its tile by tokens rather than by channel halves when loading,
  // so that every load instruction covers whole lines: lane (token
  // lt = 8 chalf + lane/8, piece lp = lane%8) reads channels
  // cb*B2_CB + 8 lp .. + 8 and publishes them into the row tile of the wave
  // that owns that half, at that wave's slot for (token lt, group lp%4).
  V8<E> xo[B2_SUB], dvo[B2_SUB];
  const uint32_t xrowb = (uint32_t)xstride * EB;
  const int lt = 8 * chalf + (lane >> 3);
  const int lp = lane & 7;
  const int lc = cb * B2_CB + 8 * lp;
  const bool lcv = wv && lc < C;
  const int lcc = lcv ? lc : 0;
  const int pubw = slot + 4 * (lp >> 2);
  const int puboff = (lp & 3) * LY::GSTRIDE + lt * 8 * EB;
  const uint32_t vx = ((uint32_t)lt * (uint32_t)xstride + lcc) * EB;
  const uint32_t vd = (((uint32_t)lt * N + srow) * (uint32_t)C + lcc) * EB;
  // ROUTE: this lane's tokens' active lists for the step loaded next, and
  // from them the slot of this lane's stream (-1: not active).  The slots
  // are formed right after the top-of-step wait, before any memory operation
  // of the step: a first use of the lists after this step's store and copies
  // would make the compiler wait for all of them (loads and stores share one
  // counter), exposing the copies' latency every step.
  int nid[B2_SUB][4], nslot[B2_SUB];
#pragma unroll
  for (int s = 0; s < B2_SUB; ++s) {
    nslot[s] = -1;
#pragma unroll
    for (int a = 0; a < 4; ++a) nid[s][a] = -1;
  }
  auto form_slots = [&]() {
    if constexpr (ROUTE) {
#pragma unroll
      for (int s = 0; s < B2_SUB; ++s) {
        int slot = -1;
#pragma unroll
        for (int a = 0; a < 4; ++a)
          if (nid[s][a] == srow) slot = a;
        nslot[s] = slot;
      }
    }
  };
  // (the routed loads go through buffer resources based at each tile, with
  // 32-bit per-lane offsets; a list of a token past the end reads zeros)
  auto load_ids = [&](int t0) {
    if constexpr (ROUTE) {
#pragma unroll
      for (int s = 0; s < B2_SUB; ++s) {
        const int ta = t0 + s * B2_TT;
        const rsrc_t ri = make_rsrc(ridx + (size_t)ta * k, clamp_bytes(ta < T ? T - ta : 0, (uint32_t)k * 4));
        if (k == 4) {                                  // the token's list in one 16-byte load
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ri, (uint32_t)lt * 16, 0, 0);
          nid[s][0] = (int)v[0]; nid[s][1] = (int)v[1]; nid[s][2] = (int)v[2]; nid[s][3] = (int)v[3];
        } else {
#pragma unroll
          for (int a = 0; a < 4; ++a)
            nid[s][a] = a < k ? (int)__builtin_amdgcn_raw_buffer_load_b32(ri, ((uint32_t)lt * k + a) * 4, 0, 0) : -1;
        }
      }
    }
  };
  auto load_own = [&](int t0) {
#pragma unroll
    for (int s = 0; s < B2_SUB; ++s) {
      const int ta = t0 + s * B2_TT;
      const int left = ta < T ? T - ta : 0;
      const rsrc_t rx = make_rsrc(static_cast<const char*>(xbase) + (size_t)ta * xrowb, clamp_bytes(left, xrowb));
      const rsrc_t rd = make_rsrc(static_cast<const char*>(dXn) + (size_t)ta * tokb, clamp_bytes(left, tokb));
      if (!ROUTE) xo[s] = bload<E, 8, CP_NT>(rx, vx, 0);
      if constexpr (ROUTE) {
        // the slot of this lane's stream in its token's list (-1: not
        // active) picks the row: pass[t][slot] or dX_new[t][stream], read
        // through a per-lane address (tokens past the end read token T-1;
        // their values are masked when published)
        const int slot = nslot[s];
        const size_t tk = (size_t)(ta + lt < T ? ta + lt : T - 1);
        const char* src_row = slot >= 0
            ? static_cast<const char*>(passbuf) + ((tk * k + slot) * (size_t)C + lcc) * EB
            : static_cast<const char*>(dXn) + ((tk * N + srow) * (size_t)C + lcc) * EB;
        dvo[s] = V8<E>::load_nt(src_row, 0);
        // the state row: saved at its slot after an in-place forward
        const char* x_row = (xact && slot >= 0)
            ? static_cast<const char*>(xact) + ((tk * k + slot) * (size_t)C + lcc) * EB
            : static_cast<const char*>(xbase) + (tk * (size_t)xstride + lcc) * EB;
        xo[s] = V8<E>::load_nt(x_row, 0);
      } else {
        dvo[s] = bload<E, 8, CP_NT>(rd, vd, 0);
      }
    }
  };
  // dX of finished tiles, by buffer stores based at each tile: an
  // out-of-range offset (ragged token or channel tail, or no tile yet) is
  // dropped by the hardware.  A tile's dX goes out in whole lines, in the
  // load mapping: each wave leaves its dX in its own X row tile (the tile's
  // dW runs first, so the X values are no longer needed), and after the
  // step's closing barrier each lane stores the piece (token lt, piece lp)
  // it loaded, both tiles at the top of the next step, ahead of the
  // prefetch.  It reads them before it publishes the next rows into the
  // same places (the other wave of the row writes only the other token
  // half).  The stores are non-temporal: dX is not read again in the pass.
  auto staged = [&](int s) { return *reinterpret_cast<const V8<E>*>(&xsh[s][pubw][puboff]); };
  auto store_staged = [&](const V8<E>& v, int ta, bool have) {
    const rsrc_t rdx = make_rsrc(static_cast<char*>(dX) + (size_t)ta * tokb, (uint32_t)B2_TT * tokb);
    bstore<E, 8, CP_NT>(v, rdx, (have && ta + lt < T && lcv) ? vd : 0x80000000u, 0);
  };
  const int rowoff = g4 * LY::GSTRIDE + r16 * 8 * EB;      // this lane's slot in a row tile

  if (tbeg < tfin) {
    dma(tbeg, 0);
    load_ids(tbeg);
    form_slots();
    load_own(tbeg);
    load_ids(tbeg + STEP);
  }
  int buf = 0;
  int last_t0 = tbeg;
  for (int t0 = tbeg; t0 < tfin; t0 += STEP) {
    // these tiles' copies and own loads (issued one iteration ago) have
    // landed; the other waves' copies are covered by the barrier below
    wait_vmcnt<0>();
    form_slots();                    // (the next step's lists landed with them)
    // publish the own rows (zero outside the sequence or the channels), which
    // frees their registers for the next prefetch; each tile's place first
    // gives up the previous step's staged dX
#pragma unroll
    for (int s = 0; s < B2_SUB; ++s) {
      const V8<E> d = staged(s);
      const bool ok = t0 + s * B2_TT + lt < T && lcv;
      *reinterpret_cast<V8<E>*>(&xsh[s][pubw][puboff]) = ok ? xo[s] : V8<E>::zero();
      *reinterpret_cast<V8<E>*>(&gsh[s][pubw][puboff]) = ok ? dvo[s] : V8<E>::zero();
      store_staged(d, t0 - STEP + s * B2_TT, t0 > tbeg);
    }
    {
      // next tiles' loads; the last step reloads itself so that every wave
      // issues the same memory operations in every iteration
      const int tn = t0 + STEP < tfin ? t0 + STEP : t0;
      dma(tn, buf ^ 1);
      load_own(tn);
      load_ids(tn + STEP);
    }
    // the published rows and this step's copies (waited above) are visible
    // to every wave; the next step's copies and loads stay in flight
    lds_barrier();
#pragma unroll
    for (int s = 0; s < B2_SUB; ++s) {
      __builtin_amdgcn_sched_barrier(0);      // keep the tiles' live ranges apart
      const unsigned char* rb = rbuf[buf][s];

      // ---- dW on MFMA: A = X^T (rows = channels, K = 16 tokens) ----
      {
        Vec<E, 4> bh[NPT], bl[NPT];
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const int off = RDZRT + ((pt * 4 + g4) * 16 + r16) * 4 * EB;
          bh[pt] = *reinterpret_cast<const Vec<E, 4>*>(rb + off);
          if constexpr (BF) bl[pt] = *reinterpret_cast<const Vec<E, 4>*>(rb + off + NPT * 4 * 16 * 4 * EB);
        }
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          // channel cc = 16*jt + r16 of tokens 4*g4 .. 4*g4+3: entry [cc/8][t], element cc%8
          const int cc = 16 * jt + r16;
          const unsigned char* colp = &xsh[s][wave][(cc >> 3) * LY::GSTRIDE + (cc & 7) * EB];
          Vec<E, 4> xa;
          if constexpr (BF) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const unsigned lo16 = *reinterpret_cast<const uint16_t*>(colp + (4 * g4 + 2 * q) * 8 * EB);
              const unsigned hi16 = *reinterpret_cast<const uint16_t*>(colp + (4 * g4 + 2 * q + 1) * 8 * EB);
              xa.w[q] = lo16 | (hi16 << 16);
            }
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) xa.x[q] = *reinterpret_cast<const float*>(colp + (4 * g4 + q) * 8 * EB);
          }
#pragma unroll
          for (int pt = 0; pt < NPT; ++pt) {
            dwacc[jt][pt] = mma16(xa, bh[pt], dwacc[jt][pt]);
            if constexpr (BF) dwacc[jt][pt] = mma16(xa, bl[pt], dwacc[jt][pt]);
          }
        }
      }
      // ---- proj on MFMA: D[c][t], 2 j-tiles; K = 48 logits as 32 + 16 ----
      f32x4 pj[2];
      if constexpr (ROUTE) {
        V8<E> bz0, bz0l, bz2, bz2l;
        const int off0 = REC_DZR0 + (g4 * 16 + r16) * 8 * EB;
        const int off2 = RR_DZR1 + (g4 * 16 + r16) * 8 * EB;
        bz0 = *reinterpret_cast<const V8<E>*>(rb + off0);
        bz2 = *reinterpret_cast<const V8<E>*>(rb + off2);
        if constexpr (BF) {
          bz0l = *reinterpret_cast<const V8<E>*>(rb + off0 + rec_dzr0_half(EB));
          bz2l = *reinterpret_cast<const V8<E>*>(rb + off2 + rec_dzr0_half(EB));
        }
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          acc = mma32(wa[jt], bz0, acc);
          acc = mma32(wc[jt], bz2, acc);
          if constexpr (BF) {
            acc = mma32(wa[jt], bz0l, acc);
            acc = mma32(wc[jt], bz2l, acc);
          }
          pj[jt] = acc;
        }
      } else {
        V8<E> bz0, bz0l;
        Vec<E, 4> bz1, bz1l;
        {
          const int off0 = REC_DZR0 + (g4 * 16 + r16) * 8 * EB;
          const int off1 = REC_DZR1 + (g4 * 16 + r16) * 4 * EB;
          bz0 = *reinterpret_cast<const V8<E>*>(rb + off0);
          bz1 = *reinterpret_cast<const Vec<E, 4>*>(rb + off1);
          if constexpr (BF) {
            bz0l = *reinterpret_cast<const V8<E>*>(rb + off0 + rec_dzr0_half(EB));
            bz1l = *reinterpret_cast<const Vec<E, 4>*>(rb + off1 + rec_dzr1_half(EB));
          }
        }
        // the K = 32 and K = 16 steps accumulate apart and are added on the
        // VALU: an MFMA of one shape accumulating onto the result of the
        // other shape needs wait states that the compiler does not insert
        // (such a chain gave timing-dependent wrong sums)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          f32x4 a32 = {0.f, 0.f, 0.f, 0.f}, a16 = {0.f, 0.f, 0.f, 0.f};
          a32 = mma32(wa[jt], bz0, a32);
          a16 = mma16(wb[jt], bz1, a16);
          if constexpr (BF) {
            a32 = mma32(wa[jt], bz0l, a32);
            a16 = mma16(wb[jt], bz1l, a16);
          }
          pj[jt] = a32 + a16;
        }
      }
      // ---- assemble dX for (token t0 + s*B2_TT + r16, channels cl..cl+8) ----
      {
        const float* co = reinterpret_cast<const float*>(rb + RCO);
        const float hpre = co[(F_PRE + srow) * B2_TT + r16];
        // the active rows also take gamma_act (hres_active; 0 otherwise)
        const float gam = co[F_GAMMA * B2_TT + r16] + ((!ROUTE && active_grp) ? co[(F_GAMMA + 1) * B2_TT + r16] : 0.f);
        const float cst = ROUTE ? co[RRF_CONST * B2_TT + r16] : 0.f;
        float pass[8];
        if (active_grp) {
          // all four rows' reads first (rows past k were published as zeros
          // and get coefficient 0), then the sums
          V8<E> gv[4];
          float hh[4];
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            gv[a] = *reinterpret_cast<const V8<E>*>(&gsh[s][a + 4 * chalf][rowoff]);
            const float h = co[(RF_RES + a * 4 + slot) * B2_TT + r16];
            hh[a] = a < k ? h : 0.f;
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) pass[q] = 0.f;
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            float gf[8];
            gv[a].to_float(gf);
#pragma unroll
            for (int q = 0; q < 8; ++q) pass[q] = fmaf(hh[a], gf[q], pass[q]);
          }
        } else {
          const V8<E> gv = *reinterpret_cast<const V8<E>*>(&gsh[s][wave][rowoff]);
          gv.to_float(pass);
        }
        const V8<E> hv =
            *reinterpret_cast<const V8<E>*>(rb + RUSED + (r16 * B2_CB + chalf * B2_WAVE_CH + 8 * g4) * EB);
        const V8<E> xv = *reinterpret_cast<const V8<E>*>(&xsh[s][wave][rowoff]);
        float xf[8], hf[8], o[8];
        xv.to_float(xf);
        hv.to_float(hf);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int jt = q >> 2, e = q & 3;              // channel 8*g4 + q = 8*g4 + 4*jt + e
          float v = pass[q];
          v = fmaf(hpre, hf[q], v);
          v += pj[jt][e];
          v = fmaf(-gam, xf[q], v);
          if constexpr (ROUTE) v += cst;
          o[q] = v;
        }
        // staged in this wave's X row tile, over the value just read (the
        // tile's dW, above, has read the rest of it)
        *reinterpret_cast<V8<E>*>(&xsh[s][wave][rowoff]) = V8<E>::from_float(o);
      }
    }
    // every read of this step's buffers and row tiles is done, and the staged
    // dX is visible to the other wave of the row
    lds_barrier();
    buf ^= 1;
    last_t0 = t0;
  }
  if (tbeg < tfin) {
#pragma unroll
    for (int s = 0; s < B2_SUB; ++s) store_staged(staged(s), last_t0 + s * B2_TT, true);
  }
  // dW partial rows: D row 4*g4+e of j-tile jt = channel 16*jt + 4*g4 + e
  if (wv) {
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = 16 * jt + 4 * g4 + e;
        if (c0 + ch < C) {
          float* dst = dwp + ((size_t)ts * NCs + jbase + ch) * (NPT * 16);
#pragma unroll
          for (int pt = 0; pt < NPT; ++pt) dst[16 * pt + r16] = dwacc[jt][pt][e];
        }
      }
  }
}

// The B2 kernels: the fixed-list form and the routed form (every row group
// in the row-group body), both held to four waves per SIMD (at most 128
// VGPRs, no spills) so that two workgroups share a CU.
template <typename E>
__global__ __launch_bounds__(512, 4) void k_bgrad(
    StreamRows src, const void* __restrict__ dXn, const void* __restrict__ dhin, const void* __restrict__ Wp,
    const unsigned char* __restrict__ rec, int ntiles, void* dX, float* __restrict__ dwp, int T, int C, int N, int k,
    RowTable rows, int nrg, int ncb, int tok_per_split, int wz0, int wz1) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[bgrad_lds_bytes<E, false>()];
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int rg = lb % nrg;
  const int cb = (lb / nrg) % ncb;
  const int ts = lb / (nrg * ncb);
  bgrad_body<E, false>(src, dXn, dhin, Wp, rec, ntiles, dX, dwp, T, C, N, k, rows, rg, cb, ts, tok_per_split,
                       nullptr, nullptr, nullptr, wz0, wz1, smem);
}
template <typename E>
__global__ __launch_bounds__(512, 4) void k_bgrad_route(
    StreamRows src, const void* __restrict__ dXn, const void* __restrict__ dhin, const void* __restrict__ Wp,
    const unsigned char* __restrict__ rec, int ntiles, void* dX, float* __restrict__ dwp, int T, int C, int N, int k,
    RowTable rows, int nrg, int ncb, int tok_per_split, const void* __restrict__ passbuf,
    const int32_t* __restrict__ ridx, const void* __restrict__ xact) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[bgrad_lds_bytes<E, true>()];
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int rg = lb % nrg;
  const int cb = (lb / nrg) % ncb;
  const int ts = lb / (nrg * ncb);
  bgrad_body<E, true>(src, dXn, dhin, Wp, rec, ntiles, dX, dwp, T, C, N, k, rows, rg, cb, ts, tok_per_split, passbuf,
                      ridx, xact, 0, 0, smem);
}

// ---------------------------------------------------------------------------
// Deterministic reductions (fixed order, no atomics).
// ---------------------------------------------------------------------------
constexpr int RED_CONV_LANES = 4;   // threads per conv-weight gradient (quad, summed with DPP)

// One launch for the three parameter-gradient reductions; workgroup ranges:
//   [0, nb_dw)              dW[j][p] = sum over token splits (B2 partials)
//   [nb_dw, nb_dw + P)      db[p]    = sum over tokens of dz (one block per p)
//   [nb_dw + P, .. + nb_conv) dconv  = sum over sequence segments (B1 partials),
//                            4 threads per output, each summing every 4th segment
//   [.., + 32)              router: db_route[i] = sum_t drho[t, i] (blocks 0..15)
//                            and rred[i] = sum_t mean drho[t, i] / sd (16..31)
// dwp rows hold dwr floats, dz records dzs floats.  The launch runs the
// few long-latency sums over tokens (db, router) first, so that they overlap
// the bandwidth-bound dW blocks instead of trailing them.
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ dwp, int nsplit, int64_t NC, int P,
                                                float* __restrict__ dW, const float* __restrict__ dz, int T,
                                                float* __restrict__ db, const float* __restrict__ cpart, int nseg,
                                                int C, float* __restrict__ dw4, float* __restrict__ dw8,
                                                float* __restrict__ dw12, int nb_dw, int accumulate, int dwr,
                                                int dzs, int nb_conv, float* __restrict__ db_route,
                                                float* __restrict__ rred, int N, HresActive ha) {
  __shared__ float sm[256];
  const int nrt = (int)gridDim.x - (nb_dw + P + nb_conv);     // router sums (0 or 32)
  const int nfirst = P + nrt;                                   // db and router blocks go first
  int bid = blockIdx.x;
  if (bid < nfirst) bid = bid < P ? nb_dw + bid : nb_dw + P + nb_conv + (bid - P);
  else bid = bid - nfirst < nb_dw ? bid - nfirst : bid - nfirst + P;   // dW, then dconv
  if (bid >= nb_dw + P + nb_conv) {
    const int q = bid - (nb_dw + P + nb_conv);
    const int i = q & 15;
    float s = 0.f;
    #pragma unroll 8
    for (int t = threadIdx.x; t < T; t += 256) s += dz[(size_t)t * dzs + (q < 16 ? 48 : 64) + i];
    sm[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) sm[threadIdx.x] += sm[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0 && i < N) {
      if (q >= 16) rred[i] = sm[0];
      else if (db_route) db_route[i] = (accumulate ? db_route[i] : 0.f) + sm[0];
    }
    return;
  }
  if (bid < nb_dw) {
    // four consecutive logits of one row per thread (P <= 48 and the
    // partial rows are 48 floats, so a group of 4 never crosses a row)
    const int64_t g = (int64_t)bid * 256 + threadIdx.x;
    const int gpr = (P + 3) >> 2;                   // groups per row
    if (g >= NC * gpr) return;
    const int64_t j = g / gpr;
    const int p0 = (int)(g - j * gpr) * 4;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll 8
    for (int q = 0; q < nsplit; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(dwp + ((size_t)q * NC + j) * dwr + p0);
      s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
    }
    float* dst = dW + (size_t)j * P + p0;
    // hres_active: the res columns of the untouched streams' rows get no gradient
    const bool untouched = ha.mask && !((ha.mask >> (int)(j / C)) & 1u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool zero = untouched && p0 + e >= ha.res0 && p0 + e < ha.res1;
      if (p0 + e < P) dst[e] = (accumulate ? dst[e] : 0.f) + (zero ? 0.f : s[e]);
    }
    return;
  }
  if (bid < nb_dw + P) {
    if (!db) return;
    const int p = bid - nb_dw;
    float s = 0.f;
    #pragma unroll 8
    for (int t = threadIdx.x; t < T; t += 256) s += dz[(size_t)t * dzs + p];
    sm[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) sm[threadIdx.x] += sm[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) db[p] = (accumulate ? db[p] : 0.f) + sm[0];
    return;
  }
  if (!cpart) return;
  const int64_t oid = ((int64_t)(bid - nb_dw - P) * 256 + threadIdx.x) / RED_CONV_LANES;
  const int sub = threadIdx.x % RED_CONV_LANES;
  const bool ok = oid < (int64_t)C * 24;
  const int c = ok ? (int)(oid / 24) : 0, q = ok ? (int)(oid - (int64_t)c * 24) : 0;
  float s = 0.f;
  if (ok)
    #pragma unroll 8
    for (int g = sub; g < nseg; g += RED_CONV_LANES) s += cpart[((size_t)g * C + c) * 24 + q];
  s += dpp_xor1(s);
  s += dpp_xor2(s);
  if (ok && sub == 0) {
    float* dst = q < 4 ? dw4 + (size_t)c * 4 + q : q < 12 ? dw8 + (size_t)c * 8 + (q - 4) : dw12 + (size_t)c * 12 + (q - 12);
    *dst = (accumulate ? *dst : 0.f) + s;
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
static void dots_segments(const Plan& p, int& lseg, int& segs);

template <typename E, typename R>
static int backward_impl(const Plan& p, const xhc_bwd_args* a, char* ws, hipStream_t st) {
  xhc_timer* tm = a->timer;
  if (p.pt && a->status) {
    TimedLaunch tl(tm, KID_CHECK, st);
    launch_check_lists(p, a->route_idx, a->status, st);
  }
  const float* zin = a->z_save;
  if (!zin) {
    // no saved logits: recompute them (projection and coefficient passes)
    float* zbuf = reinterpret_cast<float*>(ws + p.off_zbuf);
    float* coef = reinterpret_cast<float*>(ws + p.off_coef);
    const int rc = launch_coef_bwd(p, a->X, a->xact, a->active, a->W, a->bias, nullptr, ws, coef, zbuf, st, tm,
                                   p.R ? a->W_route : nullptr, p.R ? a->b_route : nullptr,
                                   p.R ? a->route_idx : nullptr);
    if (rc) return rc;
    zin = zbuf;
  }

  const bool rt = p.pt;                      // per-token lists (router or caller)
  void* Wp = ws + p.off_wp;
  float* dpart = reinterpret_cast<float*>(ws + p.off_dpart);
  float* dpa = reinterpret_cast<float*>(ws + p.off_dpa);
  float* hpost = reinterpret_cast<float*>(ws + p.off_coef);     // [T][16] post gates for B1
  float* dwpart = reinterpret_cast<float*>(ws + p.off_dwpart);
  float* dz = reinterpret_cast<float*>(ws + p.off_dz);
  unsigned char* rec = reinterpret_cast<unsigned char*>(ws + p.off_rec);
  float* dwp = reinterpret_cast<float*>(ws + p.off_dwpart2);
  float* hres = reinterpret_cast<float*>(ws + p.off_hres);
  void* pass = ws + p.off_pass;
  float* rred = reinterpret_cast<float*>(ws + p.off_rred);
  const int32_t* ridx = rt ? a->route_idx : nullptr;
  // with a router the saved rows are mapped per token inside the kernels
  const StreamRows src = stream_rows(p, a->X, rt ? nullptr : a->xact, a->active);
  Act4 act;
  for (int b = 0; b < 4; ++b) act.id[b] = b < p.k && !rt ? a->active[b] : 0;
  const HresActive ha = hres_active(p, a->active);

  float* gss = reinterpret_cast<float*>(ws + p.off_gss);        // [T][16] Sg (Gram-Schmidt)
  const dim3 b1grid(p.b1_cblocks, p.B * p.b1_segs);
  const bool fast = p.N == 16 && p.k == 4;
#define XHC_BDOTS_G(GRID, NCOMP, FAST, MODE, LSEG, SEGS, RT)                                                    \
  k_bdots<E, NCOMP, FAST, MODE, RT><<<GRID, 256, 0, st>>>(src, a->dX_new, a->dh_in, a->out, a->w4, a->w8, a->w12, \
                                                          hpost, gss, dpart, a->dout, dwpart, p.T, p.S, p.C, p.N,  \
                                                          p.k, act, LSEG, SEGS, ridx, 16)
#define XHC_BDOTS(NCOMP, MODE)                                                                                 \
  do {                                                                                                         \
    if (rt) {                                                                                                  \
      if (fast) XHC_BDOTS_G(b1grid, NCOMP, true, MODE, p.b1_lseg, p.b1_segs, true);                            \
      else XHC_BDOTS_G(b1grid, NCOMP, false, MODE, p.b1_lseg, p.b1_segs, true);                                \
    } else {                                                                                                   \
      if (fast) XHC_BDOTS_G(b1grid, NCOMP, true, MODE, p.b1_lseg, p.b1_segs, false);                           \
      else XHC_BDOTS_G(b1grid, NCOMP, false, MODE, p.b1_lseg, p.b1_segs, false);                               \
    }                                                                                                          \
  } while (0)
  // The TFA backward runs first: it is bound by arithmetic rather than by
  // memory, so the write-back of whatever ran before the call drains while
  // it runs instead of slowing the state dots.  Its post gates (with
  // Gram-Schmidt the first pass needs none) and B2's projection operand come
  // from one small preparation kernel ahead of it.
  {
    TimedLaunch tl(tm, KID_BPREP, st);
    const int nbg = p.gs ? 0 : (int)(((int64_t)p.T * 16 + 255) / 256);
    const int nbp = (int)std::min<int64_t>(4096, (p.NC * 64 + 2047) / 2048);   // one round of PK loads each
    const R* Wr = static_cast<const R*>(p.R ? a->W_route : nullptr);
    if (rt)
      k_bwd_prep<R, true><<<nbg + nbp, 256, 0, st>>>(zin, p.gs ? nullptr : hpost, p.T, p.N, p.k, p.P, p.nc,
                                                     p.gate == XHC_GATE_UNIT, p.zsv, p.nfix, nbg,
                                                     static_cast<const R*>(a->W), static_cast<R*>(Wp), Wr, p.NC);
    else
      k_bwd_prep<R, false><<<nbg + nbp, 256, 0, st>>>(zin, p.gs ? nullptr : hpost, p.T, p.N, p.k, p.P, p.nc,
                                                      p.gate == XHC_GATE_UNIT, p.zsv, p.nfix, nbg,
                                                      static_cast<const R*>(a->W), static_cast<R*>(Wp), Wr, p.NC);
  }
  {
    TimedLaunch tl(tm, KID_BDOTS, st);
    if (p.gs) {
      int lseg, segs;
      dots_segments(p, lseg, segs);
      const dim3 g2(p.b1_cblocks, p.B * segs);
      if (rt) {
        if (fast) XHC_BDOTS_G(g2, 4, true, BD_GSDOTS, lseg, segs, true);
        else XHC_BDOTS_G(g2, 4, false, BD_GSDOTS, lseg, segs, true);
      } else {
        if (fast) XHC_BDOTS_G(g2, 4, true, BD_GSDOTS, lseg, segs, false);
        else XHC_BDOTS_G(g2, 4, false, BD_GSDOTS, lseg, segs, false);
      }
    } else if (p.nc == 4) {
      XHC_BDOTS(4, BD_FULL);
    } else {
      XHC_BDOTS(1, BD_FULL);
    }
  }
  {
    TimedLaunch tl(tm, KID_BXDOTS, st);
#define XHC_BX(RT)                                                                                             \
  k_bxdots<E, R, RT><<<p.bx_cblocks * p.bx_tiles, 64 * BX_WAVES, 0, st>>>(                                      \
      src, a->dX_new, a->dh_in, dpa, p.T, p.C, p.N, p.k, act, p.bx_cblocks, p.P, static_cast<const R*>(a->W),   \
      static_cast<R*>(Wp), p.NC, ridx, static_cast<const R*>(p.R ? a->W_route : nullptr), rt ? a->xact : nullptr, \
      0)
    if (rt) XHC_BX(true); else XHC_BX(false);
#undef XHC_BX
  }
  {
    TimedLaunch tl(tm, KID_BCOEF, st);
    const int nb = (int)((p.Tpad + BCOEF_TOK - 1) / BCOEF_TOK);
    const size_t shm = (size_t)BCOEF_TOK * (p.iters + 1) * 16 * sizeof(float);
#define XHC_BCOEF(GS, RT)                                                                                       \
  k_bcoef<E, GS, RT><<<nb, 16 * BCOEF_TOK, shm, st>>>(dpa, p.bx_cblocks, dpart, p.b1_cblocks, zin, a->bias, dz, rec, p.T,  \
                                          p.Tpad, p.N, p.k, p.nc, p.P, 1.0f / (float)p.NC, p.iters,            \
                                          p.gate == XHC_GATE_UNIT, GS ? p.gs_ceps : 0.f, hpost,                \
                                          GS ? gss : nullptr, p.zsv, p.dzs, ridx, p.nfix, hres, p.R > 0, ha)
    if (p.gs) {
      if (rt) XHC_BCOEF(true, true); else XHC_BCOEF(true, false);
    } else {
      if (rt) XHC_BCOEF(false, true); else XHC_BCOEF(false, false);
    }
#undef XHC_BCOEF
  }
  if (p.gs) {
    TimedLaunch tl(tm, KID_BDOTS_GS, st);
    XHC_BDOTS(4, BD_GSGRAD);
  }
#undef XHC_BDOTS
#undef XHC_BDOTS_G
  if (rt) {
    TimedLaunch tl(tm, KID_RPASS, st);
    launch_route_pass(p, a->dX_new, ridx, hres, pass, st);
  }
  {
    TimedLaunch tl(tm, KID_BGRAD, st);
    RowTable rows;
    for (int g = 0; g < 5; ++g)
      for (int w = 0; w < 4; ++w) rows.stream[g][w] = -1;
    if (rt) {
      for (int i = 0; i < p.N; ++i) rows.stream[i / 4][i % 4] = i;
    } else {
      for (int w = 0; w < p.k; ++w) rows.stream[0][w] = a->active[w];
      int nxt = 0;
      for (int i = 0; i < p.N; ++i) {
        bool is_act = false;
        for (int b = 0; b < p.k; ++b) is_act |= a->active[b] == i;
        if (is_act) continue;
        rows.stream[1 + nxt / 4][nxt % 4] = i;
        ++nxt;
      }
    }
    if (rt) {
      const int nb = p.b2_rowgroups * p.b2_cblocks * p.b2_ts;
      k_bgrad_route<E><<<nb, 64 * B2_WAVES, 0, st>>>(src, a->dX_new, a->dh_in, Wp, rec, (int)(p.Tpad / B2_TT),
                                                     a->dX, dwp, p.T, p.C, p.N, p.k, rows, p.b2_rowgroups,
                                                     p.b2_cblocks, p.b2_tok_per_split, pass, ridx, a->xact);
    } else {
      const int nb = p.b2_rowgroups * p.b2_cblocks * p.b2_ts;
      k_bgrad<E><<<nb, 64 * B2_WAVES, 0, st>>>(src, a->dX_new, a->dh_in, Wp, rec, (int)(p.Tpad / B2_TT), a->dX,
                                               dwp, p.T, p.C, p.N, p.k, rows, p.b2_rowgroups, p.b2_cblocks,
                                               p.b2_tok_per_split, ha.res0, ha.mask ? ha.res1 : ha.res0);
    }
  }
  {
    TimedLaunch tl(tm, KID_BREDUCE, st);
    const int nb_dw = (int)((p.NC * ((p.P + 3) / 4) + 255) / 256);
    const int nb_conv = p.nc == 4 ? (int)(((int64_t)p.C * 24 * RED_CONV_LANES + 255) / 256) : 0;
    k_reduce<<<nb_dw + p.P + nb_conv + (rt ? 32 : 0), 256, 0, st>>>(
        dwp, p.b2_ts, p.NC, p.P, a->dW, dz, p.T, a->db, p.nc == 4 ? dwpart : nullptr, p.B * p.b1_segs, p.C, a->dw4,
        a->dw8, a->dw12, nb_dw, a->accumulate, p.dwr, p.dzs, nb_conv, p.R ? a->db_route : nullptr, rred, p.N, ha);
  }
  if (p.R) {
    TimedLaunch tl(tm, KID_RDWR, st);
    launch_route_dwr(p, dwp, rred, a->dW_route, a->accumulate, st);
  }
  return hipGetLastError() == hipSuccess ? XHC_OK : XHC_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Split backward.  xhc_backward_post (first in backpropagation): from dX_new
// and the forward's z_save, the TFA backward -- dout, the conv-weight
// gradients and the dots <G_a, U_m> -- with the dots left in the caller's
// bwd_state.  xhc_backward_pre (after the sublayer's own backward has turned
// dout into dh_in): the state dots, the coefficient backward from both sets
// of dots, the dX assembly and dW, db.  Together the kernels and their
// order are those of backward_impl.
// ---------------------------------------------------------------------------
template <typename E, typename R>
static int backward_post_impl(const Plan& p, const xhc_bwd_post_args* a, char* ws, hipStream_t st) {
  xhc_timer* tm = a->timer;
  const bool rt = p.pt;                        // per-token lists (router or caller)
  float* coef = reinterpret_cast<float*>(ws + p.off_coef);        // [T][64] records, or [T][16] post gates
  float* dwpart = reinterpret_cast<float*>(ws + p.off_dwpart);
  float* dpart = static_cast<float*>(a->bwd_state);
  const int32_t* ridx = rt ? a->route_idx : nullptr;
  if (rt && a->status) {
    TimedLaunch tl(tm, KID_CHECK, st);
    launch_check_lists(p, a->route_idx, a->status, st);
  }
  const StreamRows src{};     // the rows of the state are not read here
  Act4 act;
  for (int b = 0; b < 4; ++b) act.id[b] = b < p.k && !rt ? a->active[b] : 0;
  const dim3 b1grid(p.b1_cblocks, p.B * p.b1_segs);
  const bool fast = p.N == 16 && p.k == 4;
#define XHC_BDP(GRID, NCOMP, FAST, MODE, LSEG, SEGS, RT, HP, GSS, HSTRIDE)                                      \
  k_bdots<E, NCOMP, FAST, MODE, RT><<<GRID, 256, 0, st>>>(src, a->dX_new, nullptr, a->out, a->w4, a->w8, a->w12, \
                                                          HP, GSS, dpart, a->dout, dwpart, p.T, p.S, p.C, p.N,   \
                                                          p.k, act, LSEG, SEGS, ridx, HSTRIDE)
#define XHC_BDP_RT(GRID, NCOMP, MODE, LSEG, SEGS, HP, GSS, HSTRIDE)                                             \
  do {                                                                                                         \
    if (rt) {                                                                                                  \
      if (fast) XHC_BDP(GRID, NCOMP, true, MODE, LSEG, SEGS, true, HP, GSS, HSTRIDE);                          \
      else XHC_BDP(GRID, NCOMP, false, MODE, LSEG, SEGS, true, HP, GSS, HSTRIDE);                              \
    } else {                                                                                                   \
      if (fast) XHC_BDP(GRID, NCOMP, true, MODE, LSEG, SEGS, false, HP, GSS, HSTRIDE);                         \
      else XHC_BDP(GRID, NCOMP, false, MODE, LSEG, SEGS, false, HP, GSS, HSTRIDE);                             \
    }                                                                                                          \
  } while (0)
  if (p.gs) {
    // Gram-Schmidt: the gradient through T needs the full-C dots <G_a, U_m>
    // and the Gram record (first pass, into bwd_state), then Ht = H_post T
    // and Sg from the coefficient backward's Gram-Schmidt part -- which reads
    // only those dots and the saved logits, not the state dots that need
    // dh_in -- and dout from the second pass.  The coefficient backward runs
    // here with no state-dot blocks for those records alone (its dz and
    // tile records are formed again, in full, by xhc_backward_pre).
    float* hpost = coef;
    float* gss = reinterpret_cast<float*>(ws + p.off_gss);
    {
      TimedLaunch tl(tm, KID_BDOTS, st);
      int lseg, segs;
      dots_segments(p, lseg, segs);
      const dim3 g2(p.b1_cblocks, p.B * segs);
      XHC_BDP_RT(g2, 4, BD_GSDOTS, lseg, segs, hpost, gss, 16);
    }
    {
      TimedLaunch tl(tm, KID_BCOEF, st);
      float* dpa = reinterpret_cast<float*>(ws + p.off_dpa);
      float* dz = reinterpret_cast<float*>(ws + p.off_dz);
      unsigned char* rec = reinterpret_cast<unsigned char*>(ws + p.off_rec);
      float* hres = reinterpret_cast<float*>(ws + p.off_hres);
      const int nb = (int)((p.Tpad + BCOEF_TOK - 1) / BCOEF_TOK);
      const size_t shm = (size_t)BCOEF_TOK * (p.iters + 1) * 16 * sizeof(float);
#define XHC_BCOEF_GS(RT)                                                                                        \
  k_bcoef<E, true, RT><<<nb, 16 * BCOEF_TOK, shm, st>>>(                                                         \
      dpa, 0, dpart, p.b1_cblocks, a->z_save, nullptr, dz, rec, p.T, p.Tpad, p.N, p.k, p.nc, p.P,                \
      1.0f / (float)p.NC, p.iters, p.gate == XHC_GATE_UNIT, p.gs_ceps, hpost, gss, p.zsv, p.dzs, ridx, p.nfix, \
      hres, p.R > 0, HresActive{})
      if (rt) XHC_BCOEF_GS(true); else XHC_BCOEF_GS(false);
#undef XHC_BCOEF_GS
    }
    {
      TimedLaunch tl(tm, KID_BDOTS_GS, st);
      XHC_BDP_RT(b1grid, 4, BD_GSGRAD, p.b1_lseg, p.b1_segs, hpost, gss, 16);
    }
  } else {
    const float* hpost = coef + CO_POST;
    int hstride = COEF_STRIDE;
    if (rt) {
      // the post gates as the full backward forms them (routed slots scaled
      // by their saved scores); no projection operand to pack here
      TimedLaunch tl(tm, KID_BPREP, st);
      const int nbg = (int)(((int64_t)p.T * 16 + 255) / 256);
      k_bwd_prep<R, true><<<nbg, 256, 0, st>>>(a->z_save, coef, p.T, p.N, p.k, p.P, p.nc, p.gate == XHC_GATE_UNIT,
                                               p.zsv, p.nfix, nbg, nullptr, nullptr, nullptr, p.NC);
      hpost = coef;
      hstride = 16;
    } else {
      const int rc = launch_coef_saved(p, a->z_save, coef, st, tm);
      if (rc) return rc;
    }
    TimedLaunch tl(tm, KID_BDOTS, st);
    if (p.nc == 4) XHC_BDP_RT(b1grid, 4, BD_FULL, p.b1_lseg, p.b1_segs, hpost, nullptr, hstride);
    else XHC_BDP_RT(b1grid, 1, BD_FULL, p.b1_lseg, p.b1_segs, hpost, nullptr, hstride);
  }
#undef XHC_BDP_RT
#undef XHC_BDP
  if (p.nc == 4) {
    TimedLaunch tl(tm, KID_BREDUCE, st);
    const int nb_conv = (int)(((int64_t)p.C * 24 * RED_CONV_LANES + 255) / 256);
    k_reduce<<<p.P + nb_conv, 256, 0, st>>>(nullptr, 0, p.NC, p.P, nullptr, nullptr, p.T, nullptr, dwpart,
                                           p.B * p.b1_segs, p.C, a->dw4, a->dw8, a->dw12, 0, a->accumulate, p.dwr,
                                           p.dzs, nb_conv, nullptr, nullptr, p.N, HresActive{});
  }
  return hipGetLastError() == hipSuccess ? XHC_OK : XHC_ERR_HIP;
}

template <typename E, typename R>
static int backward_pre_impl(const Plan& p, const xhc_bwd_pre_args* a, char* ws, hipStream_t st) {
  xhc_timer* tm = a->timer;
  const bool rt = p.pt;                        // per-token lists (router or caller)
  const float* zin = a->z_save;
  void* Wp = ws + p.off_wp;
  float* dpa = reinterpret_cast<float*>(ws + p.off_dpa);
  float* hpost = reinterpret_cast<float*>(ws + p.off_coef);
  float* dz = reinterpret_cast<float*>(ws + p.off_dz);
  unsigned char* rec = reinterpret_cast<unsigned char*>(ws + p.off_rec);
  float* dwp = reinterpret_cast<float*>(ws + p.off_dwpart2);
  float* hres = reinterpret_cast<float*>(ws + p.off_hres);
  void* pass = ws + p.off_pass;
  float* rred = reinterpret_cast<float*>(ws + p.off_rred);
  const float* dpart = static_cast<const float*>(a->bwd_state);
  const int32_t* ridx = rt ? a->route_idx : nullptr;
  // with per-token lists the saved rows are mapped per token inside the kernels
  const StreamRows src = stream_rows(p, a->X, rt ? nullptr : a->xact, a->active);
  Act4 act;
  for (int b = 0; b < 4; ++b) act.id[b] = b < p.k && !rt ? a->active[b] : 0;
  const HresActive ha = hres_active(p, a->active);
  {
    TimedLaunch tl(tm, KID_BXDOTS, st);
#define XHC_BX(RT)                                                                                             \
  k_bxdots<E, R, RT><<<p.bx_cblocks * p.bx_tiles, 64 * BX_WAVES, 0, st>>>(                                      \
      src, a->dX_new, a->dh_in, dpa, p.T, p.C, p.N, p.k, act, p.bx_cblocks, p.P, static_cast<const R*>(a->W),   \
      static_cast<R*>(Wp), p.NC, ridx, static_cast<const R*>(p.R ? a->W_route : nullptr), rt ? a->xact : nullptr, \
      1)
    if (rt) XHC_BX(true); else XHC_BX(false);
#undef XHC_BX
  }
  {
    TimedLaunch tl(tm, KID_BCOEF, st);
    const int nb = (int)((p.Tpad + BCOEF_TOK - 1) / BCOEF_TOK);
    const size_t shm = (size_t)BCOEF_TOK * (p.iters + 1) * 16 * sizeof(float);
    float* gss = reinterpret_cast<float*>(ws + p.off_gss);
#define XHC_BCOEF(GS, RT)                                                                                       \
  k_bcoef<E, GS, RT><<<nb, 16 * BCOEF_TOK, shm, st>>>(                                                           \
      dpa, p.bx_cblocks, dpart, p.b1_cblocks, zin, a->bias, dz, rec, p.T, p.Tpad, p.N, p.k, p.nc, p.P,           \
      1.0f / (float)p.NC, p.iters, p.gate == XHC_GATE_UNIT, GS ? p.gs_ceps : 0.f, hpost, GS ? gss : nullptr,    \
      p.zsv, p.dzs, ridx, p.nfix, hres, p.R > 0, ha)
    if (p.gs) {
      if (rt) XHC_BCOEF(true, true); else XHC_BCOEF(true, false);
    } else {
      if (rt) XHC_BCOEF(false, true); else XHC_BCOEF(false, false);
    }
#undef XHC_BCOEF
  }
  if (rt) {
    TimedLaunch tl(tm, KID_RPASS, st);
    launch_route_pass(p, a->dX_new, ridx, hres, pass, st);
  }
  {
    TimedLaunch tl(tm, KID_BGRAD, st);
    RowTable rows;
    for (int g = 0; g < 5; ++g)
      for (int w = 0; w < 4; ++w) rows.stream[g][w] = -1;
    const int nb = p.b2_rowgroups * p.b2_cblocks * p.b2_ts;
    if (rt) {
      for (int i = 0; i < p.N; ++i) rows.stream[i / 4][i % 4] = i;
      k_bgrad_route<E><<<nb, 64 * B2_WAVES, 0, st>>>(src, a->dX_new, a->dh_in, Wp, rec, (int)(p.Tpad / B2_TT),
                                                     a->dX, dwp, p.T, p.C, p.N, p.k, rows, p.b2_rowgroups,
                                                     p.b2_cblocks, p.b2_tok_per_split, pass, ridx, a->xact);
    } else {
      for (int w = 0; w < p.k; ++w) rows.stream[0][w] = a->active[w];
      int nxt = 0;
      for (int i = 0; i < p.N; ++i) {
        bool is_act = false;
        for (int b = 0; b < p.k; ++b) is_act |= a->active[b] == i;
        if (is_act) continue;
        rows.stream[1 + nxt / 4][nxt % 4] = i;
        ++nxt;
      }
      k_bgrad<E><<<nb, 64 * B2_WAVES, 0, st>>>(src, a->dX_new, a->dh_in, Wp, rec, (int)(p.Tpad / B2_TT), a->dX,
                                               dwp, p.T, p.C, p.N, p.k, rows, p.b2_rowgroups, p.b2_cblocks,
                                               p.b2_tok_per_split, ha.res0, ha.mask ? ha.res1 : ha.res0);
    }
  }
  {
    TimedLaunch tl(tm, KID_BREDUCE, st);
    const int nb_dw = (int)((p.NC * ((p.P + 3) / 4) + 255) / 256);
    k_reduce<<<nb_dw + p.P + (rt ? 32 : 0), 256, 0, st>>>(
        dwp, p.b2_ts, p.NC, p.P, a->dW, dz, p.T, a->db, nullptr, 0, p.C, nullptr, nullptr, nullptr, nb_dw,
        a->accumulate, p.dwr, p.dzs, 0, p.R ? a->db_route : nullptr, rred, p.N, ha);
  }
  if (p.R) {
    TimedLaunch tl(tm, KID_RDWR, st);
    launch_route_dwr(p, dwp, rred, a->dW_route, a->accumulate, st);
  }
  return hipGetLastError() == hipSuccess ? XHC_OK : XHC_ERR_HIP;
}

int launch_backward_post(const Plan& p, const xhc_bwd_post_args* a, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  if (p.dtype == XHC_BF16) return backward_post_impl<BF16, uint16_t>(p, a, w, st);
  return backward_post_impl<F32, float>(p, a, w, st);
}

int launch_backward_pre(const Plan& p, const xhc_bwd_pre_args* a, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  if (p.dtype == XHC_BF16) return backward_pre_impl<BF16, uint16_t>(p, a, w, st);
  return backward_pre_impl<F32, float>(p, a, w, st);
}

// Segments of the passes that write per-token records only (BD_GRAM,
// BD_GSDOTS): GRAM_SPLIT times the backward's, as these passes need few
// registers and more, shorter segments keep more waves in flight.
static void dots_segments(const Plan& p, int& lseg, int& segs) {
  lseg = std::max(12, (p.b1_lseg / GRAM_SPLIT + 11) / 12 * 12);
  segs = (p.S + lseg - 1) / lseg;
}

void launch_gram(const Plan& p, const void* out, const float* w4, const float* w8, const float* w12, float* gram,
                 hipStream_t st) {
  int lseg, segs;
  dots_segments(p, lseg, segs);
  const dim3 grid(p.b1_cblocks, p.B * segs);
  StreamRows none{};
  Act4 act{};
  if (p.dtype == XHC_BF16)
    k_bdots<BF16, 4, false, BD_GRAM, false><<<grid, 256, 0, st>>>(none, nullptr, nullptr, out, w4, w8, w12, nullptr,
                                                                  nullptr, gram, nullptr, nullptr, p.T, p.S, p.C,
                                                                  p.N, p.k, act, lseg, segs, nullptr, 16);
  else
    k_bdots<F32, 4, false, BD_GRAM, false><<<grid, 256, 0, st>>>(none, nullptr, nullptr, out, w4, w8, w12, nullptr,
                                                                 nullptr, gram, nullptr, nullptr, p.T, p.S, p.C,
                                                                 p.N, p.k, act, lseg, segs, nullptr, 16);
}

int launch_backward(const Plan& p, const xhc_bwd_args* a, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  if (p.dtype == XHC_BF16) return backward_impl<BF16, uint16_t>(p, a, w, st);
  return backward_impl<F32, float>(p, a, w, st);
}

}  // namespace xhc

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
#include "xhc_gs.h"
#include "xhc_launch.h"

namespace xhc {

// ---------------------------------------------------------------------------
// W [NC, P] (row j = i*C + c) -> Wf, the MFMA B operand in fragment order:
// for stream i, K-step ks (channels ks*32 .. ks*32+32 of the stream) and
// logit tile n, one 512-element block in which lane l holds the 8 channels
// 8*(l/16) .. +8 of logit column 16n + l%16.  A wave then loads one B
// fragment as one contiguous 1 KiB access.  Entries past C or P are zero.
// One workgroup per (i, ks): the 32 x P source rows are one contiguous run
// of W, read coalesced into LDS, and the NT fragments are written from there
// as 8-element vectors.
// With a router (Wr != NULL, NT == 4) logit tile 3 holds the router's
// candidate columns, column 48 + e = Wr column cand(e) for e < ncand (up to
// all 16 streams), then zeros.
// ---------------------------------------------------------------------------
template <typename R>
__global__ __launch_bounds__(256) void k_pack_wt(const R* __restrict__ W, R* __restrict__ Wf, int C, int P, int NT,
                                                 int nks, const R* __restrict__ Wr, int N, RowOrder cand,
                                                 int ncand) {
  __shared__ R tile[32][16 * NT_MAX + 1];
  const int i = blockIdx.x / nks, ks = blockIdx.x - (blockIdx.x / nks) * nks;
  const int c0 = ks * 32;
  const int rows = min(32, C - c0);
  const R* src = W + ((size_t)i * C + c0) * P;
  // the rows * P source elements are one contiguous, 16-byte aligned run
  // (C % 8 == 0 makes rows a multiple of 8): 16-byte loads; rows past C are 0
  constexpr int VE = 16 / sizeof(R);
  for (int v = threadIdx.x; v < rows * P / VE; v += 256) {
    R val[VE];
    __builtin_memcpy(val, src + (size_t)v * VE, 16);
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const int idx = v * VE + e;
      const int rr = idx / P;
      tile[rr][idx - rr * P] = val[e];
    }
  }
  for (int idx = rows * P + threadIdx.x; idx < 32 * P; idx += 256) {
    const int rr = idx / P;
    tile[rr][idx - rr * P] = R(0);
  }
  if (Wr) {
    const R* rsrc = Wr + ((size_t)i * C + c0) * N;
    for (int idx = threadIdx.x; idx < 32 * 16; idx += 256) {
      const int rr = idx >> 4, e = idx & 15;
      R v = R(0);
      if (rr < rows && e < ncand) v = rsrc[(size_t)rr * N + row_of(cand, e)];
      tile[rr][48 + e] = v;
    }
  }
  const int PW = Wr ? 64 : P;    // columns held in the tile
  __syncthreads();
  R* dst = Wf + (size_t)blockIdx.x * NT * 512;
  for (int idx = threadIdx.x; idx < NT * 64; idx += 256) {
    const int n = idx >> 6, l = idx & 63;
    const int p = 16 * n + (l & 15), r0 = 8 * (l >> 4);
    R v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (p < P || (p >= 48 && p < PW)) ? tile[r0 + e][p] : R(0);
    __builtin_memcpy(dst + (size_t)idx * 8, v, sizeof(v));
  }
}

// ---------------------------------------------------------------------------
// Projection partials.  Workgroup = (stream `split`, tile of PROJ_TOK
// tokens), PROJ_WAVES waves; wave w owns two 16-token MFMA row blocks
// (tokens base + 32w + 16f + l%16, f = 0, 1).  The K loop walks the stream's
// channels in stages of PU K-steps of 32:
//   * the stage's W fragments (the same for every wave) are copied once per
//     workgroup into an LDS ring by LDS-DMA loads;
//   * each lane's state pieces go to a register ring;
// and the ring keeps PNS-1 stages in flight ahead of the one being
// multiplied.  The loop holds no stores, so loads complete in order and the
// per-stage waits count only the younger stages' loads.
// Stream rows come from `src` (the state, or after an in-place forward the
// saved active rows for the active streams).
// Output zpart[split][t][0..16NT) = sum_c X[t,split,c] W[split*C+c, p],
//        zpart[split][t][16NT]    = sum_c X[t,split,c]^2,
// and with the router's tile (NT == 4)
//        zpart[split][t][16NT+1]  = sum_c X[t,split,c]   (for the LayerNorm mean).
// ---------------------------------------------------------------------------
// PU K-steps per stage, PNS stages in the ring: one K-step in a six-deep ring
// when the grid has several workgroups per CU (N >= 8 stream splits), two in
// a four-deep ring when it has one (more bytes in flight per workgroup).
template <typename E, int NT, int PU, int PNS>
__global__ __launch_bounds__(64 * PROJ_WAVES) void k_proj(StreamRows src, const void* __restrict__ Wf,
                                                          float* __restrict__ zpart, int T, int C, int ZST,
                                                          int ntiles) {
  constexpr int EB = E::bytes;
  constexpr int FB = 512 * EB;                       // bytes of one W fragment
  constexpr int WST = PU * NT * FB;                  // W bytes per stage
  constexpr int NCH = WST / 1024;                    // wave-wide 1 KiB copies per stage
  constexpr int XOPS = PU * 2 * (EB == 2 ? 1 : 2);  // state loads per lane per stage
  static_assert(WST % 1024 == 0, "stage copy split");
  __shared__ __attribute__((aligned(16))) unsigned char wring[PNS][WST];

  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int split = lb / ntiles;
  const int tile = lb - split * ntiles;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int tbase = tile * PROJ_TOK + wave * 32;
  const void* X = src.base[split];
  const int64_t xs = src.stride[split];
  size_t xrow[2];
  bool tv[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int t = tbase + 16 * f + r;
    tv[f] = t < T;
    xrow[f] = (size_t)(tv[f] ? t : 0) * xs;
  }
  const int nks = (C + 31) >> 5;
  const int nst = (nks + PU - 1) / PU;                 // stages
  const unsigned char* wsplit = static_cast<const unsigned char*>(Wf) + (size_t)split * nks * NT * FB;
  // this wave's share of each stage's W copies: chunks wave, wave + PROJ_WAVES, ...
  const int nmine = NCH > wave ? (NCH - wave + PROJ_WAVES - 1) / PROJ_WAVES : 0;

  f32x4 acc[2][NT];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[f][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss[2] = {0.f, 0.f};
  constexpr bool SUMX = NT == 4;                     // the router's LayerNorm needs sum(x)
  float sx[2] = {0.f, 0.f};

  V8<E> a[PNS][PU][2];
  // stage j -> ring slot q: W copies, then this lane's state pieces.  Stages
  // past the end reload K-step 0 (valid addresses); their data is unused.
  // Workgroups start their K walk at different stages (and wrap), so that
  // at any moment the chip reads many different column offsets of the
  // token rows instead of one column of every row.
  const int jofs = (int)(((unsigned)tile * 5u + (unsigned)split * 3u) % (unsigned)nst);
  auto issue = [&](int jv, int q) {
    const int j = jv + jofs < nst ? jv + jofs : jv + jofs - nst;
#pragma unroll
    for (int i = 0; i < (NCH + PROJ_WAVES - 1) / PROJ_WAVES; ++i) {
      const int c = wave + i * PROJ_WAVES;
      if (c < NCH) {
        const int fr = c * 1024 / FB;                    // fragment (u, n) of the stage
        const int u = fr / NT, n = fr - u * NT;
        const int ks = j * PU + u;
        const int kw = ks < nks ? ks : 0;
        const unsigned char* gsrc = wsplit + ((size_t)kw * NT + n) * FB + (c * 1024 - fr * FB) + lane * 16;
        __builtin_amdgcn_global_load_lds((const gbl_void_t*)gsrc, (lds_void_t*)&wring[q][c * 1024], 16, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      const int ks = j * PU + u;
      const int kb = ks * 32 + 8 * g;
      const bool kv = ks < nks && kb < C;
      const int kc = kv ? kb : 0;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        V8<E> v = V8<E>::load(X, xrow[f] + kc);
        a[q][u][f] = (kv && tv[f]) ? v : V8<E>::zero();
      }
    }
  };
  auto compute = [&](int q) {
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      V8<E> b[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) b[n] = *reinterpret_cast<const V8<E>*>(&wring[q][(u * NT + n) * FB + lane * 8 * EB]);
#pragma unroll
      for (int f = 0; f < 2; ++f) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float v = a[q][u][f].f(j);
          ss[f] = fmaf(v, v, ss[f]);
          if constexpr (SUMX) sx[f] += v;
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[f][n] = mma32(a[q][u][f], b[n], acc[f][n]);
      }
    }
  };
  // wait for stage j's loads with `younger` later stages issued after it
  auto wait_stage = [&]() {
    // per stage this wave issued nmine W copies and XOPS state loads;
    // PNS - 2 younger stages are in flight when a stage is consumed
    static_assert(PNS >= 3 && (PNS - 2) * (XOPS + 2) < 64, "ring depth");
    if (nmine == 2) wait_vmcnt<(PNS - 2) * (XOPS + 2)>();
    else if (nmine == 1) wait_vmcnt<(PNS - 2) * (XOPS + 1)>();
    else wait_vmcnt<(PNS - 2) * XOPS>();
  };

#pragma unroll
  for (int q = 0; q < PNS - 1; ++q) issue(q < nst ? q : 0, q);
  // steady state, unrolled by the ring size so that ring slots are static
  for (int j = 0; j < nst; j += PNS) {
#pragma unroll
    for (int q = 0; q < PNS; ++q) {
      const int jj = j + q;
      if (jj < nst) {
        wait_stage();
        __syncthreads();                           // stage jj's W copies from every wave are in LDS;
                                                   // every wave is done with slot (q-1)%PNS
        issue(jj + PNS - 1 < nst ? jj + PNS - 1 : 0, (q + PNS - 1) % PNS);
        compute(q);
      }
    }
  }
  wait_vmcnt<0>();

#pragma unroll
  for (int f = 0; f < 2; ++f) {
    ss[f] += shfl_xor(ss[f], 16);
    ss[f] += shfl_xor(ss[f], 32);
    if constexpr (SUMX) {
      sx[f] += shfl_xor(sx[f], 16);
      sx[f] += shfl_xor(sx[f], 32);
    }
  }
  float* zp = zpart + (size_t)split * T * ZST;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tt = tbase + 16 * f + 4 * g + e;     // D row 4g+e of block f
      if (tt < T) {
#pragma unroll
        for (int n = 0; n < NT; ++n) zp[(size_t)tt * ZST + 16 * n + r] = acc[f][n][e];
      }
    }
    if (g == 0 && tv[f]) {
      zp[(size_t)(tbase + 16 * f + r) * ZST + 16 * NT] = ss[f];
      if constexpr (SUMX) zp[(size_t)(tbase + 16 * f + r) * ZST + 16 * NT + 1] = sx[f];
    }
  }
}

// ---------------------------------------------------------------------------
// Coefficients.  16 lanes per token; lane e owns logit columns e, e+16, e+32
// and entry (a, b) = (e/4, e%4) of the k x k Sinkhorn matrix, whose row sums
// are quad reductions (xor 1, 2) and column sums xor 4, 8 reductions.
// Either reduces projection partials (zpart != NULL) or reloads z and r from
// z_in (a forward's z_save).  With gram != NULL (Gram-Schmidt on, four
// components) the token's Gram record is summed over its ngram channel-block
// partials, and the post coefficients become H_post T (u~ = T U, see
// xhc_gs.h), so the write pass combines the raw components.
// ROUTE (projection partials only): logit tile 3 holds x.Wr for the router's
// candidates, and each split's record sum(x) after sum(x^2); the token's scores, its top-R choice (R argmax
// rounds over the 16 lanes on fp32 scores, equal scores to the lower
// candidate, that is the lower stream id) and the scaling of the routed
// slots' post coefficients by s = sigmoid(rho) happen here; the active list
// goes to the coefficient record (CO_IDX), route_idx and z_save's router
// record.
// ---------------------------------------------------------------------------
struct RouteArgs {
  const float* rcs;       // [RCS_BLK + 1][16]: partial column sums of W_route, then the sums
  const float* b_route;   // [N] or NULL
  int32_t* route_idx;     // [T][k] or NULL
  const int32_t* force;   // [T][k] or NULL: take these routed streams instead of choosing
                          // (the backward's recompute of a forward's records)
  RowOrder cand;          // candidate e -> stream id
  int ncand, nfix, R;
  int fixed[4];           // stream ids of the fixed slots
};

template <bool GS, bool ROUTE>
__global__ __launch_bounds__(256) void k_coef(const float* __restrict__ zpart, int SK, int ZST, int NTP,
                                              const float* __restrict__ z_in, const float* __restrict__ bias,
                                              float* __restrict__ coef, float* __restrict__ z_out, int zsv, int T,
                                              int N, int k, int nc, int P, float inv_nc_total, float eps,
                                              int iters, int unit_gates, const float* __restrict__ gram,
                                              int ngram, float gs_ceps, RouteArgs ra, HresActive ha) {
  __shared__ float zs[16][COEF_STRIDE];
  __shared__ float csum[16];
  const int e = threadIdx.x & 15, tok = threadIdx.x >> 4;
  const int t = blockIdx.x * 16 + tok;
  const bool tv = t < T;
  float r = 0.f;
  float zr = 0.f, ssum = 0.f, xsum = 0.f;   // ROUTE: raw x.Wr of candidate e, sum(x^2), sum(x)
  if constexpr (ROUTE) {
    if (threadIdx.x < 16) csum[threadIdx.x] = ra.rcs[RCS_BLK * 16 + threadIdx.x];   // W_route's column sums
  }
  float r_act = 0.f;    // hres_active: RMS of the k active rows
  if (zpart) {
    float ss = (tv && e < SK) ? zpart[((size_t)e * T + t) * ZST + NTP] : 0.f;
    // (with hres_active the splits are streams: the active ones' share)
    float sa = ((ha.mask >> e) & 1u) ? ss : 0.f;
    ss += row_xor<1>(ss);
    ss += row_xor<2>(ss);
    ss += row_xor<4>(ss);
    ss += row_xor<8>(ss);
    ssum = ss;
    r = sqrtf(ss * inv_nc_total + eps);
    if constexpr (ROUTE) {
      float sx = (tv && e < SK) ? zpart[((size_t)e * T + t) * ZST + NTP + 1] : 0.f;
      sx += row_xor<1>(sx);
      sx += row_xor<2>(sx);
      sx += row_xor<4>(sx);
      sx += row_xor<8>(sx);
      xsum = sx;
    }
    if (ha.mask) {
      sa += row_xor<1>(sa);
      sa += row_xor<2>(sa);
      sa += row_xor<4>(sa);
      sa += row_xor<8>(sa);
      r_act = sqrtf(sa * ha.inv_kc + eps);
    }
    // all partial loads issued together (SK <= 16; clamped indices, masked
    // values), summed in split order
    constexpr int NZ = ROUTE ? 4 : 3;
    float z[NZ];
#pragma unroll
    for (int n = 0; n < NZ; ++n) z[n] = 0.f;
    const int tcl = tv ? t : 0;
    // hres_active: a res column sums the active streams' splits only
    bool isres[NZ];
#pragma unroll
    for (int n = 0; n < NZ; ++n) isres[n] = ha.mask && e + 16 * n >= ha.res0 && e + 16 * n < ha.res1;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const float* zp = zpart + ((size_t)min(s, SK - 1) * T + tcl) * ZST;
      float v[NZ];
#pragma unroll
      for (int n = 0; n < NZ; ++n) v[n] = zp[min(e + 16 * n, ZST - 1)];
#pragma unroll
      for (int n = 0; n < NZ; ++n) z[n] += (s < SK && (!isres[n] || ((ha.mask >> s) & 1u))) ? v[n] : 0.f;
    }
    if constexpr (ROUTE) zr = z[3];
#pragma unroll
    for (int n = 0; n < 3; ++n) {
      const int p = e + 16 * n;
      zs[tok][p] = (tv && p < P) ? z[n] / (isres[n] ? r_act : r) + (bias ? bias[p] : 0.f) : 0.f;
    }
  } else {
    r = tv ? z_in[(size_t)t * zsv + P] : 1.f;
#pragma unroll
    for (int n = 0; n < 3; ++n) {
      const int p = e + 16 * n;
      zs[tok][p] = (tv && p < P) ? z_in[(size_t)t * zsv + p] : 0.f;
    }
  }
  __syncthreads();
  if (!tv) return;
  float* co = coef + (size_t)t * COEF_STRIDE;

  // router: scores of the candidates, top-R choice, write-back scales
  int sel[4];
  float sscale[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) { sel[a] = a < k && a < ra.nfix ? ra.fixed[a] : 0; sscale[a] = 1.f; }
  if constexpr (ROUTE) {
    const int base = (threadIdx.x & 63) & ~15;
    const float inv_nc = inv_nc_total;
    const float mu = xsum * inv_nc;
    const float var = fmaxf(ssum * inv_nc - mu * mu, 0.f);
    const float sd = sqrtf(var + eps);
    const bool cand = e < ra.ncand;
    const int sid = cand ? row_of(ra.cand, e) : 0;                    // the candidate's stream
    const float csm = cand ? csum[sid] : 0.f;
    const float ys = cand ? (zr - mu * csm) / sd : 0.f;               // rho - b_route
    const float rho = cand ? ys + (ra.b_route ? ra.b_route[sid] : 0.f) : 0.f;
    float key = (cand && rho == rho) ? rho : -INFINITY;
    int lk = cand ? e : 32 + e;                                      // equal keys: lower lane wins
    float* zo = z_out ? z_out + (size_t)t * zsv : nullptr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j >= ra.R) break;
      float bv = key;
      int bl = lk;
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        float ov;
        int ol;
        if (m == 1) { ov = row_xor<1>(bv); ol = __float_as_int(row_xor<1>(__int_as_float(bl))); }
        else if (m == 2) { ov = row_xor<2>(bv); ol = __float_as_int(row_xor<2>(__int_as_float(bl))); }
        else if (m == 4) { ov = row_xor<4>(bv); ol = __float_as_int(row_xor<4>(__int_as_float(bl))); }
        else { ov = row_xor<8>(bv); ol = __float_as_int(row_xor<8>(__int_as_float(bl))); }
        const bool take = ov > bv || (ov == bv && ol < bl);
        bv = take ? ov : bv;
        bl = take ? ol : bl;
      }
      int lw = bl & 15;                            // a candidate lane: R <= ncand
      if (ra.force) {
        // the given stream's candidate lane (the lowest matching one; lane 0
        // if the stream is no candidate, which a forward's list never holds)
        int fs = ra.force[(size_t)t * k + ra.nfix + j];
        int m = (cand && sid == fs) ? e : 16;
        m = min(m, __float_as_int(row_xor<1>(__int_as_float(m))));
        m = min(m, __float_as_int(row_xor<2>(__int_as_float(m))));
        m = min(m, __float_as_int(row_xor<4>(__int_as_float(m))));
        m = min(m, __float_as_int(row_xor<8>(__int_as_float(m))));
        lw = m < 16 ? m : 0;
      }
      const float rho_w = __shfl(rho, base + lw, 64);
      const float y_w = __shfl(ys, base + lw, 64);
      const float cs_w = __shfl(csm, base + lw, 64);
      const int a = ra.nfix + j;
      const int sw = row_of(ra.cand, lw);
      const float sg = sigmoid(rho_w);
#pragma unroll
      for (int a2 = 0; a2 < 4; ++a2)
        if (a2 == a) { sel[a2] = sw; sscale[a2] = sg; }
      if (e == lw) { key = -INFINITY; lk = 64 + e; }   // taken
      if (zo && e == 0) {
        zo[P + 3 + 3 * j] = rho_w;
        zo[P + 4 + 3 * j] = y_w;
        zo[P + 5 + 3 * j] = cs_w;
      }
    }
    if (zo && e == 0) { zo[P + 1] = mu; zo[P + 2] = sd; }
    int mine = sel[0];
#pragma unroll
    for (int a2 = 1; a2 < 4; ++a2)
      if (e == a2) mine = sel[a2];
    if (e < k) {
      co[CO_IDX + e] = __int_as_float(mine);
      if (ra.route_idx) ra.route_idx[(size_t)t * k + e] = mine;
    }
  }
  // this lane's post row a = e / 4: its write-back scale
  float my_s = sscale[0];
#pragma unroll
  for (int a2 = 1; a2 < 4; ++a2)
    if ((e >> 2) == a2) my_s = sscale[a2];

  // gates
  co[CO_PRE + e] = e < N ? (unit_gates ? 1.f : sigmoid(zs[tok][e])) : 0.f;
  if constexpr (!GS) {
    (void)gram; (void)ngram; (void)gs_ceps;
    const int a = e >> 2, m = e & 3;
    const float h = (a < k && m < nc) ? (unit_gates ? 1.f : sigmoid(zs[tok][N + a * nc + m])) : 0.f;
    co[CO_POST + e] = ROUTE ? h * my_s : h;
  } else {
    // Gram-Schmidt folded into the post coefficients (nc == 4)
    float gsum = 0.f;
    if (e < 10)
#pragma unroll 8
      for (int b = 0; b < ngram; ++b) gsum += gram[((size_t)b * T + t) * 16 + e];
    // the token's 16 lanes share one wave: every lane gathers the record
    const int base = (threadIdx.x & 63) & ~15;
    float g[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = m; n < 4; ++n) {
        g[m][n] = __shfl(gsum, base + gram_idx(m, n), 64);
        g[n][m] = g[m][n];
      }
    GsFwd f;
    gs_forward(g, gs_ceps, f);
    const int a = e >> 2, m = e & 3;
    float h = 0.f;
    if (a < k) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float hp = unit_gates ? 1.f : sigmoid(zs[tok][N + a * 4 + c]);
        h = fmaf(hp, f.T[c][m], h);
      }
    }
    co[CO_POST + e] = ROUTE ? h * my_s : h;
  }
  // Sinkhorn on the k x k res logits
  {
    const int a = e >> 2, b = e & 3;
    const bool valid = a < k && b < k;
    const float L = valid ? zs[tok][N + k * nc + a * k + b] : -INFINITY;
    float mx = fmaxf(L, row_xor<1>(L));
    mx = fmaxf(mx, row_xor<2>(mx));
    float M = valid ? expf(L - mx) : 0.f;
    for (int it = 0; it < iters; ++it) {
      float rs = M + row_xor<1>(M);
      rs += row_xor<2>(rs);
      M = valid ? M / rs : 0.f;
      float cs = M + row_xor<4>(M);
      cs += row_xor<8>(cs);
      M = valid ? M / cs : 0.f;
    }
    co[CO_RES + e] = M;
  }
  if (e < 4) co[CO_R + e] = e == 0 ? r : 0.f;      // [52, 56) may hold the active list
  if (z_out) {
#pragma unroll
    for (int n = 0; n < 3; ++n) {
      const int p = e + 16 * n;
      if (p < P) z_out[(size_t)t * zsv + p] = zs[tok][p];
    }
    if (e == 0) z_out[(size_t)t * zsv + P] = r;
    if (ha.mask && e == 1) z_out[(size_t)t * zsv + P + 1] = r_act;
  }
}

// ---------------------------------------------------------------------------
// Dense read + TFA + sparse write.  Thread = MIX_CH consecutive channels of
// one sequence segment [s0, s1), swept in order.  The last 12 rows of `out`
// live in a register window that shifts by one row per token (window[11] is
// the current position, window[11-l] the position l back).  The next token's
// rows are loaded before the current token is computed and stored: loads of
// token s+1 never alias the rows written for token s, so X_new == X (in
// place) stays safe and every load batch overlaps the previous token's work.
// FAST: N == 16 and k == 4 (all row and active-row loops compile-time);
// otherwise rows i >= N and active slots a >= k are skipped at run time.
// ROUTE: each token's active list comes from its coefficient record
// (CO_IDX, written by the router) or from the caller's lists `ids` [T][k]
// (ids outside [0, N) read as 0), by uniform scalar loads two tokens ahead
// of their use in addresses, instead of `act`.
// POST (the split forward's second call, in place): only the sparse write --
// each token's k active rows and `out` are read, h_in is neither formed nor
// written (hin is not used).
// ---------------------------------------------------------------------------
struct Active { int id[4]; };

template <typename E, int NCOMP, bool FAST, bool ROUTE, bool POST = false>
__global__ __launch_bounds__(MIX_THREADS) void k_mix(
    const void* __restrict__ X, const void* __restrict__ out, const float* __restrict__ w4,
    const float* __restrict__ w8, const float* __restrict__ w12, const float* __restrict__ coef,
    void* Xnew, void* __restrict__ hin, void* __restrict__ xact, int S, int C, int N, int k,
    Active act, int in_place, int lseg, int segs_per_seq, const int32_t* __restrict__ ids) {
  using V = Vec<E, MIX_CH>;
  constexpr int EB = E::bytes;
  const int craw = (blockIdx.x * MIX_THREADS + threadIdx.x) * MIX_CH;
  const bool cv = craw < C;
  const int c = cv ? craw : 0;                  // clamped: idle lanes read valid memory
  const uint32_t voff = (uint32_t)c * EB;       // this lane's byte offset inside a row
  const uint32_t rowb = (uint32_t)C * EB;       // bytes per row
  const uint32_t tokb = (uint32_t)N * rowb;     // bytes per token of state
  const int seg = blockIdx.y;
  const int bseq = seg / segs_per_seq;
  const int s0 = (seg - bseq * segs_per_seq) * lseg;
  const int s1 = min(s0 + lseg, S);
  const size_t tok0 = (size_t)bseq * S;
  constexpr bool FULLN = FAST;
  const int NR = FAST ? 16 : N;
  const int K = FAST ? 4 : k;
  const char* Xb = static_cast<const char*>(X);
  char* Xnb = static_cast<char*>(Xnew);

  float wk[MIX_CH][24];
  if constexpr (NCOMP == 4) {
#pragma unroll
    for (int ch = 0; ch < MIX_CH; ++ch) {
#pragma unroll
      for (int q = 0; q < 4; ++q) wk[ch][q] = w4[(size_t)(c + ch) * 4 + q];
#pragma unroll
      for (int q = 0; q < 8; ++q) wk[ch][4 + q] = w8[(size_t)(c + ch) * 8 + q];
#pragma unroll
      for (int q = 0; q < 12; ++q) wk[ch][12 + q] = w12[(size_t)(c + ch) * 12 + q];
    }
  }
  // `out` rows of this sequence, addressed per position
  const rsrc_t rout = make_rsrc(static_cast<const char*>(out) + tok0 * rowb, (uint32_t)S * rowb);
  // before the first shift, slot j+1 holds position s0-11+j (zero before the
  // sequence start)
  float win[12][MIX_CH];
#pragma unroll
  for (int ch = 0; ch < MIX_CH; ++ch) win[0][ch] = 0.f;
#pragma unroll
  for (int j = 0; j < 11; ++j) {
    const int s = s0 - 11 + j;
    V v = bload<E, MIX_CH>(rout, voff, (uint32_t)(s >= 0 ? s : 0) * rowb);
    v.to_float(win[j + 1]);
    if (NCOMP != 4 || s < 0) {
#pragma unroll
      for (int ch = 0; ch < MIX_CH; ++ch) win[j + 1][ch] = 0.f;
    }
  }

  // a token's active list
  auto token_ids = [&](int s, int (&id)[4]) {
    if constexpr (ROUTE) {
      if (ids) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int v = b < K ? ids[(tok0 + s) * K + b] : 0;
          id[b] = (unsigned)v < (unsigned)NR ? v : 0;
        }
      } else {
        const int4 v = *reinterpret_cast<const int4*>(coef + (tok0 + s) * COEF_STRIDE + CO_IDX);
        id[0] = v.x; id[1] = v.y; id[2] = v.z; id[3] = v.w;
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b) id[b] = act.id[b];
    }
  };
  // prefetch buffers: the 16 state rows, the k active rows and the out row
  // of the next token (one buffer resource per token: offsets stay small).
  // The 16 rows are the forward's last read of the state: non-temporal (the
  // active rows' second read follows at once and keeps the default).
  V xr[16], xa_r[4], ov;
  auto load_token = [&](int s, const int (&id)[4]) {
    const rsrc_t rx = make_rsrc(Xb + (tok0 + s) * tokb, tokb);
    if constexpr (!POST) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (FULLN || i < NR) xr[i] = bload<E, MIX_CH, CP_NT>(rx, voff, (uint32_t)i * rowb);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (b < K) xa_r[b] = bload<E, MIX_CH>(rx, voff, (uint32_t)id[b] * rowb);
    ov = bload<E, MIX_CH>(rout, voff, (uint32_t)s * rowb);
  };
  int id_a[4], id_b[4];            // active lists of the tokens after the current one
  token_ids(s0, id_a);
  load_token(s0, id_a);
  token_ids(s0 + 1 < s1 ? s0 + 1 : s0, id_b);
  // H_pre of the token processed next (uniform loads one token ahead: the
  // dense read needs it first; H_post and H_res are loaded with the token
  // and used after the convolutions)
  f32x4 cn[4];
  auto load_pre = [&](int s) {
    const f32x4* c4 = reinterpret_cast<const f32x4*>(coef + (tok0 + s) * COEF_STRIDE);
#pragma unroll
    for (int j = 0; j < 4; ++j) cn[j] = c4[j];
  };
  load_pre(s0);

  for (int s = s0; s < s1; ++s) {
    const size_t t = tok0 + s;
    V cx[16], cxa[4], co_out = ov;
    int cid[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) { cid[b] = id_a[b]; id_a[b] = id_b[b]; }
    if constexpr (!POST) {
#pragma unroll
      for (int i = 0; i < 16; ++i) cx[i] = xr[i];
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) cxa[b] = xa_r[b];
    load_token(s + 1 < s1 ? s + 1 : s, id_a);    // next token (the last iteration reloads, harmlessly)
    token_ids(s + 2 < s1 ? s + 2 : s1 - 1, id_b);
    // the token's coefficients: H_pre loaded one token ahead, the rest now
    // (uniform 16-byte loads)
    const f32x4* c4 = reinterpret_cast<const f32x4*>(coef + t * COEF_STRIDE);
    float cpre[16], cpost[16], cres[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 a0 = cn[j], a1 = c4[4 + j], a2 = c4[8 + j];
#pragma unroll
      for (int e = 0; e < 4; ++e) { cpre[4 * j + e] = a0[e]; cpost[4 * j + e] = a1[e]; cres[4 * j + e] = a2[e]; }
    }
    load_pre(s + 1 < s1 ? s + 1 : s);
#pragma unroll
    for (int j = 0; j < 11; ++j)
#pragma unroll
      for (int ch = 0; ch < MIX_CH; ++ch) win[j][ch] = win[j + 1][ch];
    co_out.to_float(win[11]);

    // dense read
    if constexpr (!POST) {
      float hacc[MIX_CH];
#pragma unroll
      for (int ch = 0; ch < MIX_CH; ++ch) hacc[ch] = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (FULLN || i < NR) {
          float xf[MIX_CH];
          cx[i].to_float(xf);
          const float hp = cpre[i];
#pragma unroll
          for (int ch = 0; ch < MIX_CH; ++ch) hacc[ch] = fmaf(hp, xf[ch], hacc[ch]);
        }
      }
      const rsrc_t rh = make_rsrc(static_cast<char*>(hin) + t * rowb, rowb);
      if (cv) bstore<E, MIX_CH>(V::from_float(hacc), rh, voff, 0);
    }

    float u[4][MIX_CH];
#pragma unroll
    for (int ch = 0; ch < MIX_CH; ++ch) {
      u[0][ch] = win[11][ch];
      if constexpr (NCOMP == 4) {
        float s4 = 0.f, s8 = 0.f, s12 = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) s4 = fmaf(wk[ch][q], win[8 + q][ch], s4);
#pragma unroll
        for (int q = 0; q < 8; ++q) s8 = fmaf(wk[ch][4 + q], win[4 + q][ch], s8);
#pragma unroll
        for (int q = 0; q < 12; ++q) s12 = fmaf(wk[ch][12 + q], win[q][ch], s12);
        u[1][ch] = s4; u[2][ch] = s8; u[3][ch] = s12;
      }
    }
    // The state rows (new, copied, saved) are stored non-temporal: a wave
    // writes whole lines of them, and their next reader is a later pass.
    // h_in keeps the default policy, as the sublayer reads it next.
    if (cv) {
      float xa[4][MIX_CH];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (b < K) cxa[b].to_float(xa[b]);
      const rsrc_t rxn = make_rsrc(Xnb + t * tokb, tokb);
      const rsrc_t rxs = make_rsrc(static_cast<char*>(xact) + t * (uint32_t)K * rowb, (uint32_t)K * rowb);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if (a < K) {
          float res[MIX_CH];
#pragma unroll
          for (int ch = 0; ch < MIX_CH; ++ch) {
            float v = 0.f;
#pragma unroll
            for (int b = 0; b < 4; ++b)
              if (b < K) v = fmaf(cres[a * 4 + b], xa[b][ch], v);
#pragma unroll
            for (int m = 0; m < NCOMP; ++m) v = fmaf(cpost[a * 4 + m], u[m][ch], v);
            res[ch] = v;
          }
          bstore<E, MIX_CH, CP_NT>(V::from_float(res), rxn, voff, (uint32_t)cid[a] * rowb);
          if (xact) bstore<E, MIX_CH, CP_NT>(cxa[a], rxs, voff, (uint32_t)a * rowb);
        }
      }
      if (!POST && !in_place) {                    // out of place: copy the untouched rows
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (FULLN || i < NR) {
            bool is_act = false;
#pragma unroll
            for (int b = 0; b < 4; ++b) is_act |= (b < K && i == cid[b]);
            if (!is_act) bstore<E, MIX_CH, CP_NT>(cx[i], rxn, voff, (uint32_t)i * rowb);
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
static void launch_pack_wt(const Plan& p, const void* W, void* Wf, hipStream_t st, xhc_timer* tm,
                           const void* Wr = nullptr, RowOrder cand = RowOrder{0}) {
  TimedLaunch tl(tm, KID_PACK_WT, st);
  const int nks = (p.C + 31) / 32;
  k_pack_wt<R><<<p.N * nks, 256, 0, st>>>(static_cast<const R*>(W), static_cast<R*>(Wf), p.C, p.P, p.NT, nks,
                                          static_cast<const R*>(Wr), p.N, cand, p.ncand);
}

// The router's candidates (streams that are not fixed, ascending) and the
// fixed slots' streams.
static RouteArgs route_args(const Plan& p, const int32_t* active, const float* b_route, int32_t* route_idx,
                            const int32_t* force, float* rcs) {
  RouteArgs ra{};
  ra.rcs = rcs;
  ra.b_route = b_route;
  ra.route_idx = route_idx;
  ra.force = force;
  ra.ncand = p.ncand;
  ra.nfix = p.nfix;
  ra.R = p.R;
  for (int j = 0; j < 4; ++j) ra.fixed[j] = j < p.nfix && !(p.pt && !p.R) ? active[j] : 0;
  uint64_t bits = 0;
  int n = 0;
  for (int i = 0; i < p.N && p.R; ++i) {
    bool fixed = false;
    for (int j = 0; j < p.nfix; ++j) fixed |= active[j] == i;
    if (!fixed) bits |= (uint64_t)i << (4 * n++);
  }
  ra.cand = RowOrder{bits};
  return ra;
}

template <typename E>
static void launch_proj(const Plan& p, const StreamRows& src, const void* Wf, float* zpart, hipStream_t st,
                        xhc_timer* tm) {
  TimedLaunch tl(tm, KID_PROJ, st);
  const int nb = p.proj_tiles * p.SK;
#define XHC_PROJ(NT, PU, PNS) \
  k_proj<E, NT, PU, PNS><<<nb, 64 * PROJ_WAVES, 0, st>>>(src, Wf, zpart, p.T, p.C, p.ZST, p.proj_tiles)
  if (p.SK >= 8) {
    if (p.NT == 1) XHC_PROJ(1, 1, 6); else if (p.NT == 2) XHC_PROJ(2, 1, 6);
    else if (p.NT == 3) XHC_PROJ(3, 1, 6); else XHC_PROJ(4, 1, 6);
  } else {
    if (p.NT == 1) XHC_PROJ(1, 2, 4); else if (p.NT == 2) XHC_PROJ(2, 2, 4);
    else if (p.NT == 3) XHC_PROJ(3, 2, 4); else XHC_PROJ(4, 2, 4);
  }
#undef XHC_PROJ
}

template <typename E, typename R>
static int forward_impl(const Plan& p, const Plan& pn, const xhc_fwd_args* a, const xhc_chain_args* ch, char* ws,
                        hipStream_t st, xhc_timer* tm) {
  void* Wt = ws + p.off_wt;
  float* zpart = reinterpret_cast<float*>(ws + p.off_zpart);
  float* coef = reinterpret_cast<float*>(ws + p.off_coef);
  const int NTP = p.NT * 16;
  const float* carry_in = ch ? static_cast<const float*>(ch->carry_in) : nullptr;
  const bool carry_out = ch && ch->W_next;

  float* rcs = reinterpret_cast<float*>(ws + p.off_rcs);
  const RouteArgs ra = route_args(p, a->active, a->b_route, a->route_idx, nullptr, rcs);
  if (p.pt && !p.R && a->status) {
    TimedLaunch tl(tm, KID_CHECK, st);
    launch_check_lists(p, a->route_idx, a->status, st);
  }
  // the router's column sums (for its LayerNorm mean), also when the
  // logits come carried from the previous sublayer
  if (p.R) {
    TimedLaunch tl(tm, KID_RCOLSUM, st);
    launch_route_colsum(p, a->W_route, rcs, st);
  }
  if (!carry_in) {
    launch_pack_wt<R>(p, a->W, Wt, st, tm, p.R ? a->W_route : nullptr, ra.cand);
    launch_proj<E>(p, stream_rows(p, a->X, nullptr, a->active), Wt, zpart, st, tm);
  }
  float* gram = reinterpret_cast<float*>(ws + p.off_gram);
  if (p.gs) {
    TimedLaunch tl(tm, KID_GRAM, st);
    launch_gram(p, a->out, a->w4, a->w8, a->w12, gram, st);
  }
  {
    TimedLaunch tl(tm, KID_COEF, st);
    const float* zp = carry_in ? carry_in : zpart;
    const int sk = carry_in ? p.mp_ncb : p.SK;
    const int unit = p.gate == XHC_GATE_UNIT;
#define XHC_COEF(GS, RT)                                                                                      \
  k_coef<GS, RT><<<(p.T + 15) / 16, 256, 0, st>>>(zp, sk, p.ZST, NTP, nullptr, a->bias, coef, a->z_save, p.zsv, \
                                                  p.T, p.N, p.k, p.nc, p.P, 1.0f / (float)p.NC, p.eps, p.iters,  \
                                                  unit, GS ? gram : nullptr, GS ? p.b1_cblocks : 0,              \
                                                  GS ? p.gs_ceps : 0.f, ra, hres_active(p, a->active))
    if (p.gs) {
      if (p.R) XHC_COEF(true, true); else XHC_COEF(true, false);
    } else {
      if (p.R) XHC_COEF(false, true); else XHC_COEF(false, false);
    }
#undef XHC_COEF
  }
  if (carry_out) {
    // the next sublayer's weights in the MFMA fragment order (with its
    // router's candidate columns in the fourth tile, ordered by its own
    // fixed list), then the fused write pass with its projection
    const RowOrder cand_next =
        pn.R ? route_args(pn, ch->active_next, nullptr, nullptr, nullptr, nullptr).cand : RowOrder{0};
    launch_pack_wt<R>(pn, ch->W_next, Wt, st, tm, pn.R ? ch->W_route_next : nullptr, cand_next);
    TimedLaunch tl(tm, KID_MIXPROJ, st);
    const MixArgs m{a->X, a->out, a->w4, a->w8, a->w12, a->X_new, a->h_in, a->xact_save, a->active};
    launch_mixproj(p, pn, MIX_FULL, m, coef, Wt, static_cast<float*>(ch->carry_out), st, a->route_idx);
    return hipGetLastError() == hipSuccess ? XHC_OK : XHC_ERR_HIP;
  }
  {
    TimedLaunch tl(tm, KID_MIX, st);
    Active act;
    for (int b = 0; b < 4; ++b) act.id[b] = b < p.k && !p.pt ? a->active[b] : -1;
    dim3 grid(p.mix_cblocks, p.B * p.mix_segs);
    const int in_place = a->X_new == a->X;
#define XHC_MIX(NCOMP, FULLN, RT)                                                                              \
  k_mix<E, NCOMP, FULLN, RT><<<grid, MIX_THREADS, 0, st>>>(a->X, a->out, a->w4, a->w8, a->w12, coef, a->X_new, \
                                                           a->h_in, a->xact_save, p.S, p.C, p.N, p.k, act,      \
                                                           in_place, p.mix_lseg, p.mix_segs, ids)
    const bool fast = p.N == 16 && p.k == 4;
    const int32_t* ids = p.pt && !p.R ? a->route_idx : nullptr;   // the caller's lists
    if (p.pt) {
      if (p.nc == 4) {
        if (fast) XHC_MIX(4, true, true); else XHC_MIX(4, false, true);
      } else {
        if (fast) XHC_MIX(1, true, true); else XHC_MIX(1, false, true);
      }
    } else if (p.nc == 4) {
      if (fast) XHC_MIX(4, true, false); else XHC_MIX(4, false, false);
    } else {
      if (fast) XHC_MIX(1, true, false); else XHC_MIX(1, false, false);
    }
#undef XHC_MIX
  }
  return hipGetLastError() == hipSuccess ? XHC_OK : XHC_ERR_HIP;
}

// Split forward, first call: coefficients (from the state, or from the
// previous sublayer's carried partials) and the dense read h_in; with a next
// sublayer, also its projection partials over the rows this sublayer's
// write leaves untouched.
template <typename E, typename R>
static int forward_pre_impl(const Plan& p, const Plan& pn, const xhc_pre_args* a, char* ws, hipStream_t st) {
  xhc_timer* tm = a->timer;
  void* Wt = ws + p.off_wt;
  float* zpart = reinterpret_cast<float*>(ws + p.off_zpart);
  float* coef = reinterpret_cast<float*>(ws + p.off_coef);
  float* rcs = reinterpret_cast<float*>(ws + p.off_rcs);
  const float* carry_in = static_cast<const float*>(a->carry_in);   // never with per-token lists
  const RouteArgs ra = route_args(p, a->active, a->b_route, a->route_idx, nullptr, rcs);
  if (p.pt && !p.R && a->status) {
    TimedLaunch tl(tm, KID_CHECK, st);
    launch_check_lists(p, a->route_idx, a->status, st);
  }
  if (!carry_in) {
    if (p.R) {
      TimedLaunch tl(tm, KID_RCOLSUM, st);
      launch_route_colsum(p, a->W_route, rcs, st);
    }
    launch_pack_wt<R>(p, a->W, Wt, st, tm, p.R ? a->W_route : nullptr, ra.cand);
    launch_proj<E>(p, stream_rows(p, a->X, nullptr, a->active), Wt, zpart, st, tm);
  }
  {
    TimedLaunch tl(tm, KID_COEF, st);
    const float* zp = carry_in ? carry_in : zpart;
    const int sk = carry_in ? p.mp_ncb : p.SK;
#define XHC_COEF_PRE(RT)                                                                                          k_coef<false, RT><<<(p.T + 15) / 16, 256, 0, st>>>(zp, sk, p.ZST, p.NT * 16, nullptr, a->bias, coef, a->z_save,                                                       p.zsv, p.T, p.N, p.k, p.nc, p.P, 1.0f / (float)p.NC, p.eps,                                                        p.iters, p.gate == XHC_GATE_UNIT, nullptr, 0, 0.f,                                                                 RT ? ra : RouteArgs{}, hres_active(p, a->active))
    if (p.R) XHC_COEF_PRE(true); else XHC_COEF_PRE(false);
#undef XHC_COEF_PRE
  }
  if (a->W_next) launch_pack_wt<R>(pn, a->W_next, Wt, st, tm);
  {
    TimedLaunch tl(tm, KID_MIXPROJ, st);
    // the dense read visits every row once, whatever the lists: with
    // per-token lists any row order serves
    static const int32_t kOrder[4] = {0, 1, 2, 3};
    const MixArgs m{a->X, nullptr, nullptr, nullptr, nullptr, const_cast<void*>(a->X), a->h_in, nullptr,
                    p.pt ? kOrder : a->active};
    launch_mixproj(p, pn, MIX_PRE, m, coef, a->W_next ? Wt : nullptr, static_cast<float*>(a->carry_out), st);
  }
  return hipGetLastError() == hipSuccess ? XHC_OK : XHC_ERR_HIP;
}

// Split forward, second call: the coefficients again from the first call's
// z_save, then the sparse write (in place); with a next sublayer, the new
// rows' projection partials are added to the first call's carry.
template <typename E, typename R>
static int forward_post_impl(const Plan& p, const Plan& pn, const xhc_post_args* a, char* ws, hipStream_t st) {
  xhc_timer* tm = a->timer;
  void* Wt = ws + p.off_wt;
  float* coef = reinterpret_cast<float*>(ws + p.off_coef);
  float* gram = reinterpret_cast<float*>(ws + p.off_gram);
  if (p.gs) {
    TimedLaunch tl(tm, KID_GRAM, st);
    launch_gram(p, a->out, a->w4, a->w8, a->w12, gram, st);
  }
  {
    TimedLaunch tl(tm, KID_COEF, st);
#define XHC_COEF_Z(GS)                                                                                          \
  k_coef<GS, false><<<(p.T + 15) / 16, 256, 0, st>>>(nullptr, 0, p.ZST, p.NT * 16, a->z_save, nullptr, coef,       \
                                                     nullptr, p.zsv, p.T, p.N, p.k, p.nc, p.P, 1.0f / (float)p.NC, \
                                                     p.eps, p.iters, p.gate == XHC_GATE_UNIT, GS ? gram : nullptr, \
                                                     GS ? p.b1_cblocks : 0, GS ? p.gs_ceps : 0.f, RouteArgs{},     \
                                                     HresActive{})
    if (p.gs) XHC_COEF_Z(true); else XHC_COEF_Z(false);
#undef XHC_COEF_Z
    // the router's write-back scales, from the saved scores
    if (p.R) launch_route_scale_post(p, a->z_save, coef, st);
  }
  if (p.pt) {
    // per-token lists (no carry): the sparse write of each token's own rows,
    // which it reads with `out` and nothing else
    TimedLaunch tl(tm, KID_MIX, st);
    Active act;
    for (int b = 0; b < 4; ++b) act.id[b] = -1;
    const dim3 grid(p.mix_cblocks, p.B * p.mix_segs);
#define XHC_MIX_POST(NCOMP, FULLN)                                                                              \
  k_mix<E, NCOMP, FULLN, true, true><<<grid, MIX_THREADS, 0, st>>>(a->X, a->out, a->w4, a->w8, a->w12, coef, a->X, \
                                                                   nullptr, a->xact_save, p.S, p.C, p.N, p.k, act, \
                                                                   1, p.mix_lseg, p.mix_segs, a->route_idx)
    const bool fast = p.N == 16 && p.k == 4;
    if (p.nc == 4) {
      if (fast) XHC_MIX_POST(4, true); else XHC_MIX_POST(4, false);
    } else {
      if (fast) XHC_MIX_POST(1, true); else XHC_MIX_POST(1, false);
    }
#undef XHC_MIX_POST
    return hipGetLastError() == hipSuccess ? XHC_OK : XHC_ERR_HIP;
  }
  if (a->W_next) launch_pack_wt<R>(pn, a->W_next, Wt, st, tm);
  {
    TimedLaunch tl(tm, KID_MIXPROJ, st);
    const MixArgs m{a->X, a->out, a->w4, a->w8, a->w12, a->X, nullptr, a->xact_save, a->active};
    launch_mixproj(p, pn, MIX_POST, m, coef, a->W_next ? Wt : nullptr, static_cast<float*>(a->carry_out), st);
  }
  return hipGetLastError() == hipSuccess ? XHC_OK : XHC_ERR_HIP;
}

int launch_forward_pre(const Plan& p, const Plan& pn, const xhc_pre_args* a, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  if (p.dtype == XHC_BF16) return forward_pre_impl<BF16, uint16_t>(p, pn, a, w, st);
  return forward_pre_impl<F32, float>(p, pn, a, w, st);
}

int launch_forward_post(const Plan& p, const Plan& pn, const xhc_post_args* a, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  if (p.dtype == XHC_BF16) return forward_post_impl<BF16, uint16_t>(p, pn, a, w, st);
  return forward_post_impl<F32, float>(p, pn, a, w, st);
}

int launch_forward(const Plan& p, const xhc_fwd_args* a, void* ws, hipStream_t st) {
  return launch_forward_chain(p, p, a, nullptr, ws, st);
}

int launch_forward_chain(const Plan& p, const Plan& pn, const xhc_fwd_args* a, const xhc_chain_args* c, void* ws,
                         hipStream_t st) {
  char* w = static_cast<char*>(ws);
  if (p.dtype == XHC_BF16) return forward_impl<BF16, uint16_t>(p, pn, a, c, w, st, a->timer);
  return forward_impl<F32, float>(p, pn, a, c, w, st, a->timer);
}

// Coefficient records from a forward's saved logits (no Gram-Schmidt, no
// router): the split backward's post gates.
int launch_coef_saved(const Plan& p, const float* z_save, float* coef, hipStream_t st, xhc_timer* tm) {
  TimedLaunch tl(tm, KID_COEF, st);
  k_coef<false, false><<<(p.T + 15) / 16, 256, 0, st>>>(nullptr, 0, p.ZST, p.NT * 16, z_save, nullptr, coef, nullptr,
                                                        p.zsv, p.T, p.N, p.k, p.nc, p.P, 1.0f / (float)p.NC, p.eps,
                                                        p.iters, p.gate == XHC_GATE_UNIT, nullptr, 0, 0.f,
                                                        RouteArgs{}, HresActive{});
  return hipGetLastError() == hipSuccess ? XHC_OK : XHC_ERR_HIP;
}

// Backward helper: coefficients either from a forward's z_save or, when it
// is NULL, recomputed by the projection from the pre-update state.  With a
// router the recompute also forms the router's record for the forward's
// choice (force = its route_idx), so that it equals the forward's z_save.
int launch_coef_bwd(const Plan& p, const void* X, const void* xact, const int32_t* active, const void* W,
                    const float* bias, const float* z_save, void* ws, float* coef, float* z_out,
                    hipStream_t st, xhc_timer* tm, const void* W_route, const float* b_route,
                    const int32_t* force) {
  char* w = static_cast<char*>(ws);
  float* zpart = nullptr;
  float* rcs = reinterpret_cast<float*>(w + p.off_rcs);
  const RouteArgs ra = route_args(p, active, b_route, nullptr, force, rcs);
  if (!z_save) {
    void* Wt = w + p.off_wt;
    zpart = reinterpret_cast<float*>(w + p.off_zpart);
    const StreamRows src = stream_rows(p, X, xact, active);
    if (p.R) {
      TimedLaunch tl(tm, KID_RCOLSUM, st);
      launch_route_colsum(p, W_route, rcs, st);
    }
    if (p.dtype == XHC_BF16) {
      launch_pack_wt<uint16_t>(p, W, Wt, st, tm, p.R ? W_route : nullptr, ra.cand);
      launch_proj<BF16>(p, src, Wt, zpart, st, tm);
    } else {
      launch_pack_wt<float>(p, W, Wt, st, tm, p.R ? W_route : nullptr, ra.cand);
      launch_proj<F32>(p, src, Wt, zpart, st, tm);
    }
  }
  TimedLaunch tl(tm, KID_COEF, st);
  // the backward needs z (and r, and the router's record) only: its post
  // coefficients come from z
  if (p.R && !z_save)
    k_coef<false, true><<<(p.T + 15) / 16, 256, 0, st>>>(zpart, p.SK, p.ZST, p.NT * 16, nullptr, bias, coef, z_out,
                                                         p.zsv, p.T, p.N, p.k, p.nc, p.P, 1.0f / (float)p.NC, p.eps,
                                                         p.iters, p.gate == XHC_GATE_UNIT, nullptr, 0, 0.f, ra,
                                                         HresActive{});
  else
    k_coef<false, false><<<(p.T + 15) / 16, 256, 0, st>>>(zpart, p.SK, p.ZST, p.NT * 16, z_save, bias, coef, z_out,
                                                          p.zsv, p.T, p.N, p.k, p.nc, p.P, 1.0f / (float)p.NC, p.eps,
                                                          p.iters, p.gate == XHC_GATE_UNIT, nullptr, 0, 0.f,
                                                          RouteArgs{}, hres_active(p, active));
  return hipGetLastError() == hipSuccess ? XHC_OK : XHC_ERR_HIP;
}

}  // namespace xhc

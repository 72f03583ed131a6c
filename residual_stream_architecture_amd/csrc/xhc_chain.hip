// Fused write pass of one sublayer and projection of the next one (gfx950).
//
// Source: "xHC: Expanded Hyper-Connections" retrospective (qingkeai.online),
// closing section on going further than the sparse write, which mentions a
// dense-read correction that is exactly equivalent but gives no mechanism.
// The reading implemented here: the write pass of sublayer l reads every row
// of the pre-update state X and produces the k new active rows, and the
// state after the update, X', equals X in every other row.  Sublayer l+1's
// projection partials
//     sum_c X'[t,i,c] W'[i*C + c, p]   and   sum_{i,c} X'[t,i,c]^2
// are therefore formed in the same pass, on MFMA, from rows already in
// registers: the untouched rows as read and the active rows as written
// (after rounding to the storage type).  Sublayer l+1 then starts from
// these partials and never reads X' for its projection, so a stacked
// forward reads the state once per sublayer instead of twice.
//
// Workgroup = (channel block of cpw chunks, batch of MP_TOK tokens), eight
// waves; wave w owns the batch's tokens 16w .. 16w+15 for every chunk.  A
// chunk is 32*KS channels (64 for bf16 storage, 32 for fp32): lane
// (r = lane%16, g = lane/16) holds token r and channels 32u + 8g .. +8 of
// K-step u, which is at once the MFMA operand layout and a 128-byte read of
// every token row per K-step pair.  A chunk is walked in steps of MP_RPS
// rows, the k active rows first:
//   * the step's rows of the next chunk position are loaded into registers
//     one step ahead;
//   * the W' fragments of the step's rows are copied from L2 into a
//     two-slot LDS ring by LDS-DMA (shared by the eight waves);
//   * the first step of a chunk forms the TFA components (the 11 earlier
//     positions of `out` come from the lane's 15 row neighbours by DPP
//     rotations and from the previous 16 tokens' tile) and the new rows;
//   * every step accumulates h_in (old rows), the sum of squares and the
//     projection (new state) and issues its stores.
// Each step starts with a full wait and a barrier, so loads, LDS-DMA and
// stores never need exact counts.
//
// Output: the write pass's X_new, h_in, xact_save as k_mix writes them, and
//   carry[cb][t][0 .. 16*NT)  = partial x'.W' over the block's channels
//   carry[cb][t][16*NT]       = partial sum of x'^2
// which k_coef of the next sublayer sums over the ncb channel blocks.
//
// MODE splits the pass for a sublayer whose output does not exist yet when
// its input is formed (the split forward: out = F(h_in) runs in between):
//   MP_FULL  the pass above;
//   MP_PRE   the dense read only: every row is read, h_in is written, and
//            the carry gets the untouched rows' partials (their values as
//            read are the next state's); no state is written;
//   MP_POST  the sparse write only: the k active rows are read and
//            rewritten (TFA, new rows, xact_save), and their new values'
//            partials are added to the carry the PRE pass wrote.
// proj = 0 skips the projection (no next sublayer: no carry).
//
// RTS > 0 (MP_FULL, in place, N = 16, k = 4): per-token lists, the last RTS
// of the k slots chosen per token (a router's record, CO_IDX, or the
// caller's lists `ids`), the first 4 - RTS fixed.  The first step of a chunk
// reads each token's own rows (the lane's row offset in its LDS-DMA
// address), forms and stores the new rows and adds the fixed rows' share of
// the projection; h_in gets every active row's old value there.  The walk
// then visits the rows that are not fixed (rt.cand, ascending) in steps of
// four; a lane takes the new value of a row that is routed for its token
// (held from the first step) and the value as read otherwise, and adds to
// h_in only rows that are not its token's.  With a next sublayer that routes
// (NT == 4: its router's columns form the fourth tile) the pass also sums x'
// for that router's LayerNorm mean: carry[cb][t][16*NT + 1].
#include "xhc_device.h"
#include "xhc_launch.h"

namespace xhc {

constexpr int MP_WAVES = 8;
constexpr int MP_TOK = 16 * MP_WAVES;     // tokens per workgroup
constexpr int MP_RPS = 4;                 // state rows per step
constexpr int CL_STRIDE = 52;             // floats per token of the LDS coefficient rows
constexpr int MP_FULL = MIX_FULL, MP_PRE = MIX_PRE, MP_POST = MIX_POST;

// `out` n positions back: the lane's token is r of a 16-token tile, `cur`
// holds the tile's values and `halo` those of the 16 tokens before it.
// Lanes r >= n take lane r - n of `cur` (a row shift, whose source lanes
// r < n are out of the row and keep the destination's old value); lanes
// r < n take lane r - n + 16 of `halo` (a row rotation), placed first.
template <int n, typename E>
__device__ inline V8<E> window_back(const V8<E>& cur, const V8<E>& halo) {
  constexpr int NWD = (int)sizeof(V8<E>) / 4;
  unsigned cw[NWD], hw[NWD], ow[NWD];
  __builtin_memcpy(cw, &cur, sizeof(cw));
  __builtin_memcpy(hw, &halo, sizeof(hw));
#pragma unroll
  for (int j = 0; j < NWD; ++j) {
    const int rot = __builtin_amdgcn_update_dpp(0, (int)hw[j], 0x120 + n, 0xF, 0xF, false);    // row_ror:n
    ow[j] = (unsigned)__builtin_amdgcn_update_dpp(rot, (int)cw[j], 0x110 + n, 0xF, 0xF, false); // row_shr:n
  }
  V8<E> o;
  __builtin_memcpy(&o, ow, sizeof(ow));
  return o;
}

template <typename E, int NT, int NCOMP, bool FAST, int MODE, int RTS = 0>
__global__ __launch_bounds__(64 * MP_WAVES) void k_mixproj(
    const void* __restrict__ X, const void* __restrict__ out, const float* __restrict__ w4,
    const float* __restrict__ w8, const float* __restrict__ w12, const float* __restrict__ coef,
    const void* __restrict__ Wf, void* Xnew, void* __restrict__ hin, void* __restrict__ xact,
    float* __restrict__ carry, RowOrder ro, int T, int S, int C, int N_, int k_, int in_place, int cpw,
    int nch, int nbatch, int ZST, int proj, MixRoute rt) {
  // per-token lists: the full pass; the launcher admits them at N = 16, k = 4
  static_assert(RTS == 0 || (MODE == MP_FULL && RTS <= 4), "per-token lists: the full pass");
  const int N = FAST ? 16 : N_;
  const int k = FAST ? 4 : k_;
  constexpr int NFIX = 4 - RTS;              // with per-token lists: the fixed slots
  constexpr int EB = E::bytes;
  constexpr int KS = EB == 2 ? 2 : 1;        // MFMA K-steps of 32 channels per chunk
  constexpr int CW = 32 * KS;                // channels per chunk
  constexpr int FB = 512 * EB;               // bytes of one W' fragment
  constexpr int SLOTB = KS * NT * FB;        // W' bytes of one row and chunk
  constexpr int PPR = SLOTB / 1024;          // 1 KiB copies per row
  constexpr int WSLOT = MP_RPS * SLOTB;      // W' bytes of one step
  static_assert(SLOTB % 1024 == 0, "W' step slot");
  // the spreading of the active rows' work over two steps (below) holds
  // their K-step-1 fragments from a chunk's first step to its third
  constexpr bool SPLIT_OK = RTS == 0 && NT <= 3;
  // the W' ring, then (only in a pass that spreads the active rows' work)
  // the active rows' held K-step-1 fragments: a pass with a fourth logit
  // tile has no room for them in LDS
  constexpr int HELD = SPLIT_OK ? MP_RPS * 3 * 1024 : 0;
  __shared__ __attribute__((aligned(16))) unsigned char wbuf[2 * WSLOT + HELD];
  unsigned char (*const wst)[WSLOT] = reinterpret_cast<unsigned char (*)[WSLOT]>(wbuf);
  unsigned char* const wa1 = wbuf + 2 * WSLOT;
  __shared__ __attribute__((aligned(16))) float cwl[24][64];
  __shared__ __attribute__((aligned(16))) float cl[MP_TOK][CL_STRIDE];
  __shared__ __attribute__((aligned(16))) unsigned char xbuf[MP_WAVES][MP_RPS * 1024 * KS * (EB / 2)];

  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  const int cb = lb / nbatch, bt = lb - cb * nbatch;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int tb = bt * MP_TOK, t0 = tb + 16 * wave, t = t0 + r;
  const int spos = (t < T ? t : 0) % S;                 // position in the sequence
  // steps per chunk (the POST pass visits the k active rows only: one step;
  // with per-token lists the active rows, then the rows that are not fixed)
  const int nq = RTS ? 1 + (rt.ncand + MP_RPS - 1) / MP_RPS : MODE == MP_POST ? 1 : (N + MP_RPS - 1) / MP_RPS;
  // bf16 chunks hold two K-steps; with four steps per chunk the active rows'
  // second K-step (TFA, new rows, their projection) moves to the third step,
  // so that the arithmetic of the first step is split over two steps
  const bool split = SPLIT_OK && MODE == MP_FULL && KS == 2 && nq == 4;
  // with per-token lists: the token's routed rows (slots NFIX ..), read once
  int rid[4] = {0, 0, 0, 0};
  if constexpr (RTS > 0) {
    const int tt = t < T ? t : T - 1;
#pragma unroll
    for (int a = NFIX; a < 4; ++a) {
      const int v = rt.ids ? rt.ids[(size_t)tt * 4 + a] : __float_as_int(coef[(size_t)tt * COEF_STRIDE + CO_IDX + a]);
      rid[a] = (unsigned)v < 16u ? v : 0;
    }
  }
  const int c0 = cb * cpw, c1 = min(c0 + cpw, nch);
  const int nsteps = (c1 - c0) * nq;
  const int nks = (C + 31) >> 5;                        // K-steps of the packed W'
  const uint32_t rowb = (uint32_t)C * EB, tokb = (uint32_t)N * rowb;
  const int tc = min(t0, T);
  const int ntile = min(max(T - t0, 0), 16);
  // `out` of the tile and of the 16 tokens before it in one resource; the
  // first tile (t0 = 0) has no halo and reads its own rows there, which the
  // position mask discards
  const int th = max(t0 - 16, 0);
  const uint32_t cur_soff = (uint32_t)(t0 - th) * ((uint32_t)C * EB);
  const rsrc_t rx = make_rsrc_u(static_cast<const char*>(X) + (size_t)tc * tokb, clamp_bytes(ntile, tokb));
  const rsrc_t rxn = make_rsrc_u(static_cast<char*>(Xnew) + (size_t)tc * tokb, clamp_bytes(ntile, tokb));
  const rsrc_t rout = make_rsrc_u(static_cast<const char*>(out) + (size_t)min(th, T) * rowb,
                                clamp_bytes(min(max(T - th, 0), 32), rowb));
  const rsrc_t rh = make_rsrc_u(static_cast<char*>(hin) + (size_t)tc * rowb, clamp_bytes(ntile, rowb));
  const uint32_t xsb = (uint32_t)k * rowb;              // bytes per token of xact
  const rsrc_t rxs = make_rsrc_u(xact ? static_cast<char*>(xact) + (size_t)tc * xsb : Xnew,
                               xact ? clamp_bytes(ntile, xsb) : 0u);

  // lane byte offset of (chunk c, K-step u) in a row of `stride` bytes per
  // token; channels past C get an offset the buffer range check drops
  auto lane_off = [&](int c, int u, uint32_t stride) -> uint32_t {
    const int ch = c * CW + 32 * u + 8 * g;
    return ch < C ? (uint32_t)r * stride + (uint32_t)ch * EB : 0x80000000u;
  };

  // coefficients of the batch's tokens -> cl[token][pre 16 | post 16 | res 16 | r, pad]
  // (13 pieces of 16 bytes per token: the padded row stride spreads the 16
  // tokens a wave reads over the LDS banks)
  {
    constexpr int PIECES = CL_STRIDE / 4;
    const int ntok = min(max(T - tb, 0), MP_TOK);
    const rsrc_t rco = make_rsrc_u(coef + (size_t)min(tb, T) * COEF_STRIDE, clamp_bytes(ntok, COEF_STRIDE * 4));
#pragma unroll
    for (int j = 0; j < (MP_TOK * PIECES + 64 * MP_WAVES - 1) / (64 * MP_WAVES); ++j) {
      const int id = j * 64 * MP_WAVES + tid;            // 16-byte piece: token id/PIECES, part id%PIECES
      const int tk = id / PIECES, part = id - tk * PIECES;
      if (j * 64 * MP_WAVES + wave * 64 < MP_TOK * PIECES)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rco, (lds_void_t*)(reinterpret_cast<unsigned char*>(&cl[0][0]) + (j * 64 * MP_WAVES + wave * 64) * 16),
            16, (uint32_t)(tk * COEF_STRIDE + part * 4) * 4, 0, 0, 0);
    }
  }

  // conv weights of chunk c: thread-strided over the chunk's [w4 | w8 | w12]
  // source ranges (contiguous in memory), stored transposed as cwl[tap][ch]
  float cwr[3];
  auto conv_src = [&](int c, int f, int& tap, int& cc) -> const float* {
    if (f < 4 * CW) { cc = f >> 2; tap = f & 3; return w4 + (size_t)c * CW * 4 + f; }
    if (f < 12 * CW) { const int f2 = f - 4 * CW; cc = f2 >> 3; tap = 4 + (f2 & 7); return w8 + (size_t)c * CW * 8 + f2; }
    const int f3 = f - 12 * CW;
    cc = f3 / 12; tap = 12 + (f3 - cc * 12);
    return w12 + (size_t)c * CW * 12 + f3;
  };
  auto load_conv = [&](int c) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int f = tid + i * 64 * MP_WAVES;
      float v = 0.f;
      if (f < 24 * CW) {
        int tap, cc;
        const float* src = conv_src(c, f, tap, cc);
        if (c * CW + cc < C) v = *src;
      }
      cwr[i] = v;
    }
  };
  auto store_conv = [&](int c) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int f = tid + i * 64 * MP_WAVES;
      if (f < 24 * CW) {
        int tap, cc;
        (void)conv_src(c, f, tap, cc);
        cwl[tap][cc] = cwr[i];
      }
    }
  };

  // with per-token lists: the state row of step q's slot j, and whether the
  // step projects it -- the first step the fixed rows only (the routed ones
  // differ per token), the walk the rows that are not fixed
  auto step_row = [&](int q, int j, bool& projected) -> int {
    if (q == 0) {
      projected = j < NFIX;
      return row_of(ro, j < NFIX ? j : 0);
    }
    const int sl = (q - 1) * MP_RPS + j;
    projected = sl < rt.ncand;
    return row_of(rt.cand, sl < rt.ncand ? sl : rt.ncand - 1);
  };

  // W' fragments of step s's rows -> wst[s & 1][slot j][u][n]
  auto w_dma = [&](int s) {
    const int cq = s / nq, q = s - cq * nq, c = c0 + cq;
    const int ksb = c * KS;
    const int valid_bytes = min(nks - ksb, KS) * NT * FB;
#pragma unroll
    for (int i = 0; i < (MP_RPS * PPR + MP_WAVES - 1) / MP_WAVES; ++i) {
      const int pc = wave + MP_WAVES * i;
      if (pc < MP_RPS * PPR) {
        const int j = pc / PPR, o = pc - j * PPR;
        bool wanted;
        int wrow;
        if constexpr (RTS > 0) {
          wrow = step_row(q, j, wanted);
        } else {
          const int slot = q * MP_RPS + j;
          // PRE projects the untouched rows only, POST the active ones only
          wanted = slot < N && (MODE == MP_FULL || (MODE == MP_PRE ? slot >= k : slot < k));
          wrow = row_of(ro, slot);
        }
        if (proj && wanted && o * 1024 < valid_bytes) {
          const unsigned char* src = static_cast<const unsigned char*>(Wf) +
                                     ((size_t)wrow * nks + ksb) * NT * FB + o * 1024 + lane * 16;
          if (split && q == 0 && j < k && o >= PPR / 2)   // K-step 1 of an active row
            __builtin_amdgcn_global_load_lds((const gbl_void_t*)src,
                                             (lds_void_t*)&wa1[j * (PPR / 2) * 1024 + (o - PPR / 2) * 1024], 16, 0, 0);
          else
            __builtin_amdgcn_global_load_lds((const gbl_void_t*)src, (lds_void_t*)&wst[s & 1][j * SLOTB + o * 1024],
                                             16, 0, 0);
        }
      }
    }
  };

  // register state
  V8<E> xc[MP_RPS][KS];                       // rows of the current step
  V8<E> oc[KS], oh[KS];                       // out and its halo of the chunk (loaded after the
                                              // previous chunk's first step consumed them)
  // the next step's rows go to the wave's LDS buffer by LDS-DMA (16 bytes
  // per lane and copy, lane-ordered), so that prefetching costs no
  // registers; the step reads them back into registers at its start
  constexpr int PP = EB / 2;                  // 16-byte pieces per lane and V8
  auto dma_rows = [&](int c, int q) {
#pragma unroll
    for (int j = 0; j < MP_RPS; ++j) {
      if (MODE == MP_POST && j >= k) continue;       // untouched rows: not read by the POST pass
      // with per-token lists the walk's last step may hold fewer rows than
      // slots: the empty slots are neither loaded nor read
      if (RTS > 0 && q > 0 && (q - 1) * MP_RPS + j >= rt.ncand) continue;
      uint32_t soff = (uint32_t)row_of(ro, q * MP_RPS + j) * rowb;    // rows past N repeat a valid row
      if constexpr (RTS > 0) {
        bool unused;
        soff = (uint32_t)step_row(q, j, unused) * rowb;
      }
      // with per-token lists the first step's routed slots read the
      // lane's own row: its offset goes into the lane's address
      uint32_t vrow = 0;
      if constexpr (RTS > 0) {
        if (q == 0 && j >= NFIX) {
          soff = 0;
          vrow = (uint32_t)rid[j] * rowb;
        }
      }
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        const uint32_t vo = lane_off(c, u, tokb) + vrow;
#pragma unroll
        for (int pp = 0; pp < PP; ++pp)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)&xbuf[wave][((j * KS + u) * PP + pp) * 1024], 16,
                                                   (int)(vo + pp * 16), (int)soff, 0, 0);
      }
    }
  };
  auto read_rows = [&]() {
#pragma unroll
    for (int j = 0; j < MP_RPS; ++j)
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        unsigned w[4 * PP];
#pragma unroll
        for (int pp = 0; pp < PP; ++pp) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(&xbuf[wave][((j * KS + u) * PP + pp) * 1024 + lane * 16]);
          w[4 * pp] = v[0]; w[4 * pp + 1] = v[1]; w[4 * pp + 2] = v[2]; w[4 * pp + 3] = v[3];
        }
        __builtin_memcpy(&xc[j][u], w, sizeof(w));
      }
    // the buffer is refilled right after: every read must have completed
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
  };
  auto load_out = [&](int c) {
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      oc[u] = bload<E, 8>(rout, lane_off(c, u, rowb), cur_soff);
      oh[u] = bload<E, 8>(rout, lane_off(c, u, rowb), 0);
    }
  };

  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  float sx = 0.f;                             // sum of x' (NT == 4: for the next router's mean)
  float hacc[KS][8];
#pragma unroll
  for (int u = 0; u < KS; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) hacc[u][e] = 0.f;
  const float* co = &cl[16 * wave + r][0];
  // with per-token lists: the new values of the token's routed rows (slots
  // NFIX ..), from a chunk's first step to the walk that projects them
  V8<E> nvr[4][KS];

  // one row of the step: h_in from the old values, sum of squares and the
  // projection from `xv` (the row of the new state), K-step u
  auto row_work = [&](const unsigned char* wfr, int u, int c, float hp, const V8<E>& xold, const V8<E>& xv,
                      bool project) {
    if constexpr (MODE != MP_POST) {
#pragma unroll
      for (int e = 0; e < 8; ++e) hacc[u][e] = fmaf(hp, xold.f(e), hacc[u][e]);
    }
    if (!project) return;
    if constexpr (EB == 2) {
      // bf16 pairs: the products are exact in fp32
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x2 p2 = __builtin_bit_cast(bf16x2, xv.w[d]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, ss, false);
        if constexpr (NT == 4) {
          const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
          sx = __builtin_amdgcn_fdot2_f32_bf16(p2, one2, sx, false);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = xv.f(e);
        ss = fmaf(y, y, ss);
        if constexpr (NT == 4) sx += y;
      }
    }
    if (proj && c * KS + u < nks) {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const V8<E> wv = *reinterpret_cast<const V8<E>*>(wfr + n * FB + lane * 8 * EB);
        acc[n] = mma32(wv, xv, acc[n]);
      }
    }
  };

  // K-step u of chunk c for the active rows: TFA components, the new rows
  // (stored, and projected with the fragments at wact + row j * wstride),
  // h_in and sum of squares.  xs[b] holds active row b's K-step u.
  auto active_u = [&](int c, int u, const V8<E>* xs, const unsigned char* wact, int wstride) {
    unsigned nvw[4][sizeof(V8<E>) / 4];       // packed new rows: [a][dword] (bf16 pairs or fp32 bits)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float u0[4], u1[4], u2[4], u3[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) u0[e] = oc[u].f(4 * h + e);
      if constexpr (NCOMP == 4) {
        const float* wl = &cwl[0][32 * u + 8 * g + 4 * h];
        auto tap4 = [&](int tap) { return *reinterpret_cast<const f32x4*>(wl + tap * 64); };
        {
          const f32x4 wa = tap4(3), wb = tap4(4 + 7), wc = tap4(12 + 11);
#pragma unroll
          for (int e = 0; e < 4; ++e) { u1[e] = wa[e] * u0[e]; u2[e] = wb[e] * u0[e]; u3[e] = wc[e] * u0[e]; }
        }
        // U_m = sum_{n < K_m} w_m[c, K_m - 1 - n] * out[t - n]
        static_for<1, 12>([&](auto NI) {
          constexpr int n = decltype(NI)::value;
          const V8<E> ob = window_back<n, E>(oc[u], oh[u]);
          float of[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) of[e] = spos < n ? 0.f : ob.f(4 * h + e);
          if constexpr (n < 4) {
            const f32x4 w = tap4(3 - n);
#pragma unroll
            for (int e = 0; e < 4; ++e) u1[e] = fmaf(w[e], of[e], u1[e]);
          }
          if constexpr (n < 8) {
            const f32x4 w = tap4(4 + 7 - n);
#pragma unroll
            for (int e = 0; e < 4; ++e) u2[e] = fmaf(w[e], of[e], u2[e]);
          }
          {
            const f32x4 w = tap4(12 + 11 - n);
#pragma unroll
            for (int e = 0; e < 4; ++e) u3[e] = fmaf(w[e], of[e], u3[e]);
          }
        });
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if (a < k) {
          const f32x4 res = *reinterpret_cast<const f32x4*>(co + 32 + 4 * a);
          const f32x4 post = *reinterpret_cast<const f32x4*>(co + 16 + 4 * a);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float y = 0.f;
#pragma unroll
            for (int b = 0; b < 4; ++b)
              if (b < k) y = fmaf(res[b], xs[b].f(4 * h + e), y);
            y = fmaf(post[0], u0[e], y);
            if constexpr (NCOMP == 4) {
              y = fmaf(post[1], u1[e], y);
              y = fmaf(post[2], u2[e], y);
              y = fmaf(post[3], u3[e], y);
            }
            v[e] = y;
          }
          const Vec<E, 4> hv = Vec<E, 4>::from_float(v);
          __builtin_memcpy(&nvw[a][h * (int)sizeof(Vec<E, 4>) / 4], &hv, sizeof(hv));
        }
      }
    }
    // new and saved rows are stored non-temporal, as in the mix kernel
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if (a < k) {
        V8<E> nv;
        __builtin_memcpy(&nv, &nvw[a][0], sizeof(nv));
        if (RTS > 0 && a >= NFIX) {
          // a row of the token's own: stored at the lane's row, its old value
          // into h_in with the token's coefficient, its new value held for
          // the walk, which projects it
          bstore<E, 8, CP_NT>(nv, rxn, lane_off(c, u, tokb) + (uint32_t)rid[a] * rowb, 0);
          if (xact) bstore<E, 8, CP_NT>(xs[a], rxs, lane_off(c, u, xsb), (uint32_t)a * rowb);
          const float hp = co[rid[a]];
#pragma unroll
          for (int e = 0; e < 8; ++e) hacc[u][e] = fmaf(hp, xs[a].f(e), hacc[u][e]);
          nvr[a][u] = nv;
        } else {
          const int row = row_of(ro, a);
          bstore<E, 8, CP_NT>(nv, rxn, lane_off(c, u, tokb), (uint32_t)row * rowb);
          if (xact) bstore<E, 8, CP_NT>(xs[a], rxs, lane_off(c, u, xsb), (uint32_t)a * rowb);
          row_work(wact + a * wstride, u, c, co[row], xs[a], nv, true);
        }
      }
    }
  };
  V8<E> xa1[4];                               // active rows' K-step 1, first to third step

  // step (chunk cq, quarter q): rows 4q .. 4q+4 of the row order.  FIRST:
  // q == 0, which also forms the new active rows (both K-steps, or K-step 0
  // when split, K-step 1 then following in the third step).
  auto step = [&](auto FI, int cq, int q) {
    constexpr bool FIRST = decltype(FI)::value;
    auto& x = xc;
    const int c = c0 + cq;
    const int s = cq * nq + q;
    wait_vmcnt<0>();
    if constexpr (FIRST && NCOMP == 4 && MODE != MP_PRE) {
      if (nq == 1) __syncthreads();     // one step per chunk: every wave is done with the last conv weights
      store_conv(c);
    }
    __syncthreads();            // W' of step s, conv weights and coefficients visible; step s-1 consumed
    read_rows();
    // the next step's copies
    if (q + 1 < nq) {
      w_dma(s + 1);
      dma_rows(c, q + 1);
    } else if (cq + 1 < c1 - c0) {
      w_dma(s + 1);
      dma_rows(c + 1, 0);
      if constexpr (NCOMP == 4 && MODE != MP_PRE) load_conv(c + 1);
    }
    const unsigned char* wsl = wst[s & 1];

    if constexpr (FIRST && MODE != MP_PRE) {
      if (split) {
        V8<E> xs0[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) { xs0[b] = x[b][0]; xa1[b] = x[b][KS - 1]; }
        active_u(c, 0, xs0, wsl, SLOTB);
      } else {
#pragma unroll
        for (int u = 0; u < KS; ++u) {
          V8<E> xs[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) xs[b] = x[b][u];
          active_u(c, u, xs, wsl + u * NT * FB, SLOTB);
        }
        if (cq + 1 < c1 - c0) load_out(c + 1);      // this chunk's `out` has been consumed
      }
    } else {
      if (split && q == 2) {
        active_u(c, KS - 1, xa1, wa1, NT * FB);
        if (cq + 1 < c1 - c0) load_out(c + 1);
      }
    }
    // the walk with per-token lists: the rows that are not fixed; the
    // token's routed rows take their held new values, and their old ones
    // are already in h_in
    if constexpr (RTS > 0 && !FIRST) {
#pragma unroll
      for (int j = 0; j < MP_RPS; ++j) {
        const int sl = (q - 1) * MP_RPS + j;
        if (sl < rt.ncand) {
          const int row = row_of(rt.cand, sl);
          bool mine = false;
#pragma unroll
          for (int a = NFIX; a < 4; ++a) mine |= rid[a] == row;
          const float hp = mine ? 0.f : co[row];
#pragma unroll
          for (int u = 0; u < KS; ++u) {
            V8<E> xv = x[j][u];
#pragma unroll
            for (int a = NFIX; a < 4; ++a) {
              if (rid[a] == row) {
                xv = nvr[a][u];
              }
            }
            row_work(wsl + j * SLOTB + u * NT * FB, u, c, hp, x[j][u], xv, true);
          }
        }
      }
    }
    // the step's other rows (untouched by the update); the PRE pass reads the
    // active rows here too, for h_in only
#pragma unroll
    for (int j = 0; j < MP_RPS; ++j) {
      const int slot = q * MP_RPS + j;
      const bool untouched = !FIRST || j >= k;
      if (RTS == 0 && MODE != MP_POST && slot < N && (untouched || MODE == MP_PRE)) {
        const int row = row_of(ro, slot);
        const float hp = co[row];
#pragma unroll
        for (int u = 0; u < KS; ++u) {
          row_work(wsl + j * SLOTB + u * NT * FB, u, c, hp, x[j][u], x[j][u], untouched);
          if (MODE == MP_FULL && !in_place) bstore<E, 8, CP_NT>(x[j][u], rxn, lane_off(c, u, tokb), (uint32_t)row * rowb);
        }
      }
    }
    if (MODE != MP_POST && q + 1 == nq) {
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        bstore<E, 8>(V8<E>::from_float(hacc[u]), rh, lane_off(c, u, rowb), 0);
#pragma unroll
        for (int e = 0; e < 8; ++e) hacc[u][e] = 0.f;
      }
    }
  };

  if constexpr (NCOMP == 4 && MODE != MP_PRE) load_conv(c0);
  if (c1 > c0) {
    w_dma(0);
    dma_rows(c0, 0);
    if constexpr (MODE != MP_PRE) load_out(c0);
  }
  for (int cq = 0; cq < c1 - c0; ++cq) {
    step(std::true_type{}, cq, 0);
    for (int q = 1; q < nq; ++q) step(std::false_type{}, cq, q);
  }
  wait_vmcnt<0>();

  ss += shfl_xor(ss, 16);
  ss += shfl_xor(ss, 32);
  if constexpr (NT == 4) {
    sx += shfl_xor(sx, 16);
    sx += shfl_xor(sx, 32);
  }
  if (proj && t < T) {
    float* zp = carry + ((size_t)cb * T + t) * ZST;
    if constexpr (MODE == MP_POST) {
      // the PRE pass's partials (untouched rows) plus the new rows'
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        f32x4* dst = reinterpret_cast<f32x4*>(zp + 16 * n + 4 * g);
        *dst = *dst + acc[n];
      }
      if (g == 0) zp[16 * NT] += ss;
      if (NT == 4 && g == 0) zp[16 * NT + 1] += sx;
    } else {
#pragma unroll
      for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(zp + 16 * n + 4 * g) = acc[n];
      if (g == 0) zp[16 * NT] = ss;
      if (NT == 4 && g == 0) zp[16 * NT + 1] = sx;
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
// pn: the next sublayer's plan; its tile count and partial-record stride
// shape the projection and the carry.  mode: MP_FULL, MP_PRE or MP_POST;
// Wf == NULL: no projection (and no carry).
template <typename E>
static void launch_mixproj_e(const Plan& p, const Plan& pn, int mode, const MixArgs& m, const float* coef,
                             const void* Wf, float* carry, hipStream_t st, const int32_t* ids) {
  RowOrder ro{0};
  MixRoute rt{};
  // with per-token lists the host list holds the fixed slots only (none for
  // the caller's lists)
  const bool per_token = p.pt && mode == MP_FULL;   // the split passes visit rows alike for every token
  const int nfix = per_token ? (p.R ? p.nfix : 0) : p.k;
  {
    bool used[16] = {false};
    int order[16], n = 0;
    for (int b = 0; b < nfix; ++b) { order[n++] = m.active[b]; used[m.active[b]] = true; }
    uint64_t cbits = 0;
    for (int i = 0; i < p.N; ++i)
      if (!used[i]) {
        cbits |= (uint64_t)i << (4 * rt.ncand++);
        order[n++] = i;
      }
    for (; n < 16; ++n) order[n] = order[0];
    for (int i = 0; i < 16; ++i) ro.bits |= (uint64_t)order[i] << (4 * i);
    rt.cand = RowOrder{cbits};
    rt.ids = per_token && !p.R ? ids : nullptr;
  }
  const int in_place = m.X_new == m.X;
  const int proj = Wf != nullptr;
  const int NT = proj ? pn.NT : 1;
  const dim3 grid(p.mp_ncb * p.mp_nbatch);
#define XHC_MP_R(NTV, NC, MODE, RTS)                                                                              \
  k_mixproj<E, NTV, NC, false, MODE, RTS><<<grid, 64 * MP_WAVES, 0, st>>>(                                        \
      m.X, m.out, m.w4, m.w8, m.w12, coef, Wf, m.X_new, m.h_in, m.xact_save, carry, ro, p.T, p.S, p.C, p.N, p.k,   \
      in_place, p.mp_cpw, p.mp_nch, p.mp_nbatch, pn.ZST, proj, rt)
#define XHC_MP(NTV, NC, MODE) XHC_MP_R(NTV, NC, MODE, 0)
#define XHC_MP_NT(NC, MODE)                                                                                       \
  do {                                                                                                           \
    if (NT == 3) XHC_MP(3, NC, MODE); else if (NT == 2) XHC_MP(2, NC, MODE); else XHC_MP(1, NC, MODE);           \
  } while (0)
  // a fourth logit tile (the next sublayer's router) in the full pass only:
  // the split passes are not chained with per-token lists
  if (per_token) {
    // per-token lists (the full pass, in place, N = 16, k = 4, so the next
    // sublayer has at least three logit tiles): two or four slots per token
    const int rts = 4 - nfix;
#define XHC_MP_RT(NC)                                                                                             \
  do {                                                                                                           \
    if (rts == 2) {                                                                                              \
      if (NT == 4) XHC_MP_R(4, NC, MP_FULL, 2); else XHC_MP_R(3, NC, MP_FULL, 2);                               \
    } else {                                                                                                     \
      if (NT == 4) XHC_MP_R(4, NC, MP_FULL, 4); else XHC_MP_R(3, NC, MP_FULL, 4);                               \
    }                                                                                                            \
  } while (0)
    if (p.nc == 4) XHC_MP_RT(4); else XHC_MP_RT(1);
#undef XHC_MP_RT
  } else if (mode == MP_PRE) {
    XHC_MP_NT(1, MP_PRE);                  // no write-back: the component count does not matter
  } else if (mode == MP_POST) {
    if (p.nc == 4) XHC_MP_NT(4, MP_POST); else XHC_MP_NT(1, MP_POST);
  } else if (NT == 4) {
    if (p.nc == 4) XHC_MP(4, 4, MP_FULL); else XHC_MP(4, 1, MP_FULL);
  } else {
    if (p.nc == 4) XHC_MP_NT(4, MP_FULL); else XHC_MP_NT(1, MP_FULL);
  }
#undef XHC_MP_NT
#undef XHC_MP
#undef XHC_MP_R
}

void launch_mixproj(const Plan& p, const Plan& pn, int mode, const MixArgs& m, const float* coef, const void* Wf,
                    float* carry, hipStream_t st, const int32_t* ids) {
  if (p.dtype == XHC_BF16) launch_mixproj_e<BF16>(p, pn, mode, m, coef, Wf, carry, st, ids);
  else launch_mixproj_e<F32>(p, pn, mode, m, coef, Wf, carry, st, ids);
}

}  // namespace xhc

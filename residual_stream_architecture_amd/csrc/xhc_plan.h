// Host-side execution plan of one xHC call: derived sizes, launch shapes and
// the workspace layout.  Pure C++ (no HIP), so that workspace sizing and
// argument validation run without a GPU.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "xhc.h"

namespace xhc {

// Per-token coefficient record written by the coefficient kernels (floats):
//   [0, 16)   H_pre[i]
//   [16, 32)  H_post[a*4 + m]
//   [32, 48)  H_res[a*4 + b]
//   48        r (RMS of the flattened state)
//   [52, 56)  with a router: the token's active list (stream ids as int bits)
constexpr int COEF_STRIDE = 64;
constexpr int CO_PRE = 0, CO_POST = 16, CO_RES = 32, CO_R = 48, CO_IDX = 52;

// Per-token backward dot records (floats):
//   B1x, per channel block of BX_CB:   [0, 16)  dH_pre[i]      = <dh_in, X_i>
//                                      [16, 32) dH_res[a*4+b]  = <G_a, X_{i_b}>
//   B1, per channel block of B1:       [32, 48) <G_a, U_m> (dH_post[a*4+m]
//                                      without Gram-Schmidt)
//                                      [0, 10)  Gram record <U_m, U_n>, m <= n
//                                      (with Gram-Schmidt)
constexpr int DOT_STRIDE = 48;
constexpr int BX_OUT = 32;

constexpr int PROJ_WAVES = 8;     // waves per projection workgroup
constexpr int PROJ_TOK = 32 * PROJ_WAVES;   // tokens per projection workgroup (32 per wave)
constexpr int MIX_CH = 2;         // channels per thread in the mix kernel
constexpr int MIX_THREADS = 256;
constexpr int MIX_TARGET_WAVES = 10240;  // grid size: several rounds of short token segments
constexpr int B1_CH = 2;          // channels per lane in B1's TFA part
constexpr int B1_WAVE_CH = 128;   // channels per B1 wave (64 lanes x 2)
constexpr int B1_WAVES = 4;       // waves per B1 workgroup (consecutive chunks)
constexpr int BX_WAVES = 8;       // waves per B1x workgroup
constexpr int BX_WCH = 64;        // channels per B1x wave (two K=32 steps)
constexpr int BX_CB = BX_WAVES * BX_WCH;
constexpr int BX_TOK = 64;        // tokens per B1x workgroup
constexpr int BX_GRP = 8;         // tokens per B1x cross-wave reduction
constexpr int B2_WAVE_CH = 32;    // channels per B2 wave (one state row)
constexpr int B2_CB = 64;         // channels per B2 workgroup: whole 128-byte lines of a bf16 row
constexpr int B2_WAVES = 8;       // 4 rows x 2 channel halves
constexpr int B2_TT = 16;         // tokens per B2 tile (one MFMA K / N extent)
constexpr int B2_SUB = 2;         // tiles per B2 iteration (loaded together, one iteration ahead)
constexpr int B2_TARGET_WG = 2048;  // B2 grid: four rounds of 2 workgroups per CU (later rounds balance the load)

// Per-tile backward record (B2_TT tokens), written by the coefficient
// backward kernel and copied verbatim into LDS by B2, so its layout is the
// order in which B2's lanes read it (lane = g*16 + r):
//   [REC_DZR0, ..)    dz/r logits 0..31, B fragments of the projection's
//                     K=32 MFMA: [half][g 4][t 16] x 8 elements, p = 8g + e
//   [REC_DZR1, ..)    dz/r logits 32..47, B fragments of its K=16 MFMA:
//                     [half][g 4][t 16] x 4 elements, p = 32 + 4g + e
//   [REC_DZRT, ..)    dz/r as the dW MFMA's B fragments:
//                     [half][pt 3][g 4][r 16] x 4 elements, logit 16pt + r, token 4g + e
//   [REC_CO, +2304)   coefficients [field 36][t 16] floats: H_pre[16], H_res[16], gamma,
//                     gamma_act (the active rows' extra term with hres_active, else 0)
// half = bf16 hi and lo parts (bf16 storage) or one fp32 part (fp32 storage);
// each region has the same size in both storages.
constexpr int REC_BYTES = 9216;
constexpr int REC_USED = 8448;   // bytes of a record that carry data (the rest pads to 1 KiB)
constexpr int REC_DZR0 = 0, REC_DZR1 = 2048, REC_DZRT = 3072, REC_CO = 6144;
constexpr int RF_PRE = 0, RF_RES = 16, RF_GAMMA = 32, REC_NF = 36;
constexpr int rec_dzr0_half(int esz) { return 4 * 16 * 8 * esz; }
constexpr int rec_dzr1_half(int esz) { return 4 * 16 * 4 * esz; }
constexpr int rec_dzrt_half(int esz) { return 3 * 4 * 16 * 4 * esz; }

// The same record with a router (routed backward): the projection's K is 64
// (logits 0..47, then the router's 16 stream columns), so
//   [REC_DZR0, ..)    dz/r logits 0..31 as above
//   [RR_DZR1, ..)     logits 32..63 as a second K=32 step, p = 32 + 8g + e
//   [RR_DZRT, ..)     four dW B-fragment tiles (logits 0..63)
//   [RR_CO, ..)       fields [RRF_NF][t 16]: H_pre[16], gamma, the LayerNorm
//                     term that every element of the token's dX receives
// B2 copies REC_R_USED bytes of it; records are REC_R_BYTES apart.
constexpr int RR_DZR1 = 2048, RR_DZRT = 4096, RR_CO = 8192;
constexpr int RRF_PRE = 0, RRF_GAMMA = 16, RRF_CONST = 17, RRF_NF = 18;
constexpr int REC_R_USED = RR_CO + RRF_NF * B2_TT * 4;
constexpr int REC_R_BYTES = 10240;
static_assert(REC_R_USED <= REC_R_BYTES, "routed record");

constexpr int NT_MAX = 4;   // logit tiles of 16: P = N + k*nc + k*k <= 48, plus the router's tile
constexpr int RCS_BLK = 256; // partial column sums of W_route (forward router), then the sums
constexpr int DZ_R = 80;    // floats per token of the routed backward's dz record:
                            // dz [0,48), drho [48,64), mean*drho/sd [64,80)

// The res logits of the active-row form (hres_active): which logit columns
// are res columns and which streams are active.
struct HresActive {
  unsigned mask;      // bit i: stream i is active (0: the form is off)
  int res0, res1;     // res logit columns [res0, res1)
  float inv_kc;       // 1 / (k*C)
};

struct Plan {
  int B, S, C, N, k, nc, P, NT, T, iters, dtype, gate;
  float eps;
  bool gs;            // Gram-Schmidt over the four components (nc == 4)
  float gs_ceps;      // C * gs_eps
  bool hact;          // H_res generated from the k active rows (res logits normed by their RMS)
  int R;              // routed slots (0: fixed active list)
  bool pt;            // per-token active lists (the router's, or given by the caller)
  int nfix;           // fixed slots, k - R
  int ncand;          // router candidates, N - nfix (<= 16)
  int zsv;            // floats per token of z_save
  int dzs;            // floats per token of the backward's dz record
  int dwr;            // floats per row of the backward's dW partials
  int rec_bytes;      // bytes per B2 tile record
  int64_t NC;
  int esz;            // bytes per storage element
  // forward
  int SK;             // projection K-splits (one per stream)
  int ZST;            // floats per (split, token) partial record
  int proj_tiles;     // token tiles of PROJ_TOK
  int mix_cblocks;    // channel blocks of MIX_THREADS*MIX_CH
  int mix_lseg;       // tokens per mix segment
  int mix_segs;       // segments per sequence
  // backward
  int b1_cblocks;     // channel blocks of B1_WAVES*B1_WAVE_CH
  int b1_lseg;        // tokens per B1 segment (multiple of 12)
  int b1_segs;        // segments per sequence
  int bx_cblocks;     // channel blocks of BX_CB
  int bx_tiles;       // token tiles of BX_TOK
  int b2_rowgroups;   // 1 active group + ceil((N-k)/4) inactive groups
  int b2_cblocks;     // channel blocks of B2_CB
  int b2_ts;          // token splits
  int b2_tok_per_split;
  int64_t Tpad;       // T rounded up to B2_TT
  // fused write + next-sublayer projection (chained forward)
  int mp_nch;         // channel chunks (64 channels for bf16 storage, 32 for fp32)
  int mp_cpw;         // chunks per workgroup
  int mp_ncb;         // channel blocks = projection partials per token (<= 16)
  int mp_nbatch;      // token batches of 128
  size_t carry_bytes; // [mp_ncb][T][ZST] floats
  // workspace layout (byte offsets; every region 256-byte aligned)
  size_t off_wt, off_zpart, off_coef, off_gram, off_rcs, fwd_bytes;
  size_t off_zbuf, off_wp, off_dpart, off_dpa, off_dwpart, off_dz, off_rec, off_dwpart2, off_gss;
  size_t state_bytes;     // bwd_state of the split backward: dot partials [b1_cblocks][T][DOT_STRIDE]
  size_t off_hres, off_pass, off_rred, bwd_bytes;
};

// Fills `p` from `d`; returns XHC_OK or an XHC_ERR_* code for an
// unsupported description.
int make_plan(const xhc_desc* d, Plan* p);
// make_plan, then the forward's argument checks (what xhc_validate does for
// XHC_PHASE_FWD).
int prepare_forward(const xhc_desc* d, const xhc_fwd_args* a, Plan* p);

}  // namespace xhc

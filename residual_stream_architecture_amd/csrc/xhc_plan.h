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
//   49        gamma = (dz . (z - bias)) / (N*C*r^2), backward only
constexpr int COEF_STRIDE = 64;
constexpr int CO_PRE = 0, CO_POST = 16, CO_RES = 32, CO_R = 48, CO_GAMMA = 49;

// Per-token backward dot record (floats, per channel block of B1):
//   [0, 16)   dH_pre[i]      = <dh_in, X_i>
//   [16, 32)  dH_res[a*4+b]  = <G_a, X_{i_b}>
//   [32, 48)  dH_post[a*4+m] = <G_a, U_m>
constexpr int DOT_STRIDE = 48;

constexpr int PROJ_TOK = 128;     // tokens per projection workgroup (4 waves x 32)
constexpr int MIX_CH = 2;         // channels per thread in the mix kernel
constexpr int MIX_THREADS = 256;
constexpr int MIX_TARGET_WAVES = 2560;   // grid size aimed at ~one resident round
constexpr int B1_CH = 2;          // channels per lane in B1's TFA part
constexpr int B1_WAVE_CH = 128;   // channels per B1 wave (64 lanes x 2)
constexpr int B1_WAVES = 4;       // waves per B1 workgroup (consecutive chunks)
constexpr int B2_CB = 32;         // channels per B2 wave row
constexpr int B2_TT = 16;         // tokens per B2 tile
constexpr int B2_TARGET_WG = 1536;  // B2 grid aimed at two rounds of 3 workgroups per CU

struct Plan {
  int B, S, C, N, k, nc, P, NT, T, iters, dtype, gate;
  float eps;
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
  int b2_rowgroups;   // 1 active group + ceil((N-k)/4) inactive groups
  int b2_cblocks;     // channel blocks of B2_CB
  int b2_ts;          // token splits
  int b2_tok_per_split;
  int64_t Tpad;       // T rounded up to B2_TT
  // workspace layout (byte offsets; every region 256-byte aligned)
  size_t off_wt, off_zpart, off_coef, fwd_bytes;
  size_t off_zbuf, off_wp, off_dpart, off_dwpart, off_dz, off_dzr, off_dzrt, off_dwpart2, bwd_bytes;
};

// Fills `p` from `d`; returns XHC_OK or an XHC_ERR_* code for an
// unsupported description.
int make_plan(const xhc_desc* d, Plan* p);

}  // namespace xhc

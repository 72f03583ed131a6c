// Bandwidth probes for the benchmark (libxhc_probe.so, not part of libxhc):
// plain kernels that move bytes in the access patterns of the xHC kernels, so
// that each kernel's achieved bandwidth can be set against what the same
// pattern reaches on the same chip.  They compute nothing of the method.
//
//   xhc_probe_stream(a, b, d, bytes, nread, nwrite)
//       contiguous streaming over buffers of `bytes`: nread in {1, 2} reads,
//       nwrite in {0, 1} writes (d = a ^ b), each workgroup walking its own
//       contiguous slice with 16-byte accesses
//   xhc_probe_rows(a, b, d, T, row_bytes, run_bytes, nread, nwrite, splits)
//       the buffers are T rows of row_bytes (one token's state: N*C*2 bytes);
//       workgroup (column block, token split) owns run_bytes of every row in
//       its split of the tokens and walks the tokens -- the pattern of the
//       backward's assembly kernel (two reads, one write) and of the
//       projection (one read) with run_bytes per workgroup and row
//   xhc_probe_frag(a, T, rows, row_bytes, mode)
//       T tokens of `rows` rows of row_bytes (the state, [T][N][C]); each
//       workgroup of 8 waves owns 1 KiB of every row of a 64-token tile, each
//       wave 128 bytes of it, read one token at a time with two 16-byte loads
//       per lane.  mode 0 lays the loads out as MFMA A fragments (lane
//       (r = lane % 16, g = lane / 16) reads row r at 16 g and 64 + 16 g: one
//       instruction touches 16 rows x 64 bytes, half of each 128-byte line);
//       mode 1 reads the same bytes with every instruction covering 8 rows x
//       128 bytes (whole lines).  The pattern of the backward's state dots
//       and, with tokens for rows, of the projection.
//
// Workgroups are mapped to logical blocks XCD by XCD (as in libxhc), so that
// the blocks running on one XCD cover neighbouring columns of the same
// tokens.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline int xcd_block(int bid, int n) {
  if (n & 7) return bid;
  return (bid & 7) * (n >> 3) + (bid >> 3);
}

constexpr int THREADS = 256;
constexpr int UNROLL = 4;

// ACC folds what was read into one value that is stored only if it equals a
// value no input holds, so that the loads are not optimised away.
template <int NR, int NW>
__global__ __launch_bounds__(THREADS) void k_stream(const u32x4* __restrict__ a, const u32x4* __restrict__ b,
                                                    u32x4* __restrict__ d, int64_t n16, int64_t per_block,
                                                    unsigned* __restrict__ sink) {
  const int lb = xcd_block(blockIdx.x, gridDim.x);
  const int64_t beg = (int64_t)lb * per_block;
  const int64_t end = beg + per_block < n16 ? beg + per_block : n16;
  unsigned acc = 0;
  for (int64_t i = beg + threadIdx.x; i < end; i += (int64_t)THREADS * UNROLL) {
    u32x4 va[UNROLL], vb[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t j = i + (int64_t)u * THREADS;
      if (j < end) {
        va[u] = __builtin_nontemporal_load(a + j);
        if (NR == 2) vb[u] = __builtin_nontemporal_load(b + j);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t j = i + (int64_t)u * THREADS;
      if (j < end) {
        u32x4 v = va[u];
        if (NR == 2) v ^= vb[u];
        if (NW) d[j] = v;
        else acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
    }
  }
  if (!NW && acc == 0x9e3779b9u) sink[0] = acc;
}

// RUN bytes of each row per workgroup; THREADS*16/RUN rows per iteration.
template <int RUN, int NR, int NW>
__global__ __launch_bounds__(THREADS) void k_rows(const u32x4* __restrict__ a, const u32x4* __restrict__ b,
                                                  u32x4* __restrict__ d, int T, int row16, int ncol,
                                                  int tok_per_split, unsigned* __restrict__ sink) {
  constexpr int LPR = RUN / 16;            // lanes per row
  constexpr int RPI = THREADS / LPR;       // rows per iteration
  const int lb = xcd_block(blockIdx.x, gridDim.x);
  const int col = lb % ncol;
  const int ts = lb / ncol;
  const int t0 = ts * tok_per_split;
  const int t1 = t0 + tok_per_split < T ? t0 + tok_per_split : T;
  const int r = threadIdx.x / LPR, e = threadIdx.x % LPR;
  unsigned acc = 0;
  for (int t = t0 + r; t < t1; t += RPI * UNROLL) {
    u32x4 va[UNROLL], vb[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int tk = t + u * RPI;
      if (tk < t1) {
        const int64_t j = (int64_t)tk * row16 + (int64_t)col * LPR + e;
        va[u] = a[j];
        if (NR == 2) vb[u] = b[j];
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int tk = t + u * RPI;
      if (tk < t1) {
        const int64_t j = (int64_t)tk * row16 + (int64_t)col * LPR + e;
        u32x4 v = va[u];
        if (NR == 2) v ^= vb[u];
        if (NW) d[j] = v;
        else acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
    }
  }
  if (!NW && acc == 0x9e3779b9u) sink[0] = acc;
}

template <int NR, int NW>
int launch_rows_run(int run, const u32x4* a, const u32x4* b, u32x4* d, int T, int row16, int ncol, int tps,
                    int nblk, unsigned* sink, hipStream_t st) {
  switch (run) {
    case 128: k_rows<128, NR, NW><<<nblk, THREADS, 0, st>>>(a, b, d, T, row16, ncol, tps, sink); return 0;
    case 256: k_rows<256, NR, NW><<<nblk, THREADS, 0, st>>>(a, b, d, T, row16, ncol, tps, sink); return 0;
    case 512: k_rows<512, NR, NW><<<nblk, THREADS, 0, st>>>(a, b, d, T, row16, ncol, tps, sink); return 0;
    case 1024: k_rows<1024, NR, NW><<<nblk, THREADS, 0, st>>>(a, b, d, T, row16, ncol, tps, sink); return 0;
    default: return -1;
  }
}

constexpr int FRAG_WAVES = 8;
constexpr int FRAG_TOK = 64;
constexpr int FRAG_RING = 4;

template <int MODE>
__global__ __launch_bounds__(64 * FRAG_WAVES) void k_frag(const unsigned char* __restrict__ a, int T, int rows,
                                                         int row_bytes, int ncb, unsigned* __restrict__ sink) {
  const int lb = xcd_block(blockIdx.x, gridDim.x);
  const int cb = lb % ncb;
  const int tile = lb / ncb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = tile * FRAG_TOK;
  const int tn = T - t0 < FRAG_TOK ? T - t0 : FRAG_TOK;
  const int64_t tokb = (int64_t)rows * row_bytes;
  const int base = cb * 1024 + wave * 128;
  int off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int row, col;
    if (MODE == 0) { row = lane & 15; col = 64 * i + 16 * (lane >> 4); }
    else { row = 8 * i + (lane >> 3); col = 16 * (lane & 7); }
    off[i] = (row < rows ? row : 0) * row_bytes + base + col;
  }
  unsigned acc = 0;
  u32x4 v[FRAG_RING][2];
  auto load = [&](int tt, int q) {
    const int tc = tt < tn ? tt : tn - 1;
    const unsigned char* p = a + (int64_t)(t0 + tc) * tokb;
#pragma unroll
    for (int i = 0; i < 2; ++i) v[q][i] = *reinterpret_cast<const u32x4*>(p + off[i]);
  };
#pragma unroll
  for (int q = 0; q < FRAG_RING - 1; ++q) load(q, q);
  for (int tt = 0; tt < tn; tt += FRAG_RING) {
#pragma unroll
    for (int u = 0; u < FRAG_RING; ++u) {
      load(tt + u + FRAG_RING - 1, (u + FRAG_RING - 1) % FRAG_RING);
      if (tt + u < tn)
#pragma unroll
        for (int i = 0; i < 2; ++i) acc ^= v[u][i][0] ^ v[u][i][1] ^ v[u][i][2] ^ v[u][i][3];
    }
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

extern "C" {

// Returns 0, -1 for arguments outside the supported set (nothing launched),
// -2 for a launch failure.  `sink` is a device word the read-only forms may
// write (never in practice); `blocks` is the grid size of the streaming form.
int xhc_probe_stream(const void* a, const void* b, void* d, int64_t bytes, int nread, int nwrite, int blocks,
                     unsigned* sink, hipStream_t st) {
  if (!a || bytes <= 0 || (bytes & 15) || blocks < 1 || !sink) return -1;
  if (nread < 1 || nread > 2 || nwrite < 0 || nwrite > 1) return -1;
  if ((nread == 2 && !b) || (nwrite && !d)) return -1;
  const int64_t n16 = bytes / 16;
  const int64_t per = (n16 + blocks - 1) / blocks;
  const u32x4* pa = static_cast<const u32x4*>(a);
  const u32x4* pb = static_cast<const u32x4*>(b);
  u32x4* pd = static_cast<u32x4*>(d);
  if (nread == 1 && !nwrite) k_stream<1, 0><<<blocks, THREADS, 0, st>>>(pa, pb, pd, n16, per, sink);
  else if (nread == 1) k_stream<1, 1><<<blocks, THREADS, 0, st>>>(pa, pb, pd, n16, per, sink);
  else if (!nwrite) k_stream<2, 0><<<blocks, THREADS, 0, st>>>(pa, pb, pd, n16, per, sink);
  else k_stream<2, 1><<<blocks, THREADS, 0, st>>>(pa, pb, pd, n16, per, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Buffers of T * row_bytes bytes; run_bytes in {128, 256, 512, 1024} divides
// row_bytes; splits >= 1 token splits (grid = row_bytes / run_bytes * splits).
int xhc_probe_rows(const void* a, const void* b, void* d, int T, int row_bytes, int run_bytes, int nread,
                   int nwrite, int splits, unsigned* sink, hipStream_t st) {
  if (!a || T < 1 || row_bytes < 16 || (row_bytes & 15) || splits < 1 || !sink) return -1;
  if (run_bytes < 128 || run_bytes > 1024 || (run_bytes & (run_bytes - 1)) || row_bytes % run_bytes) return -1;
  if (nread < 1 || nread > 2 || nwrite < 0 || nwrite > 1) return -1;
  if ((nread == 2 && !b) || (nwrite && !d)) return -1;
  const int ncol = row_bytes / run_bytes;
  const int tps = (T + splits - 1) / splits;
  const int64_t nblk = (int64_t)ncol * splits;
  if (nblk > (1 << 30)) return -1;
  const u32x4* pa = static_cast<const u32x4*>(a);
  const u32x4* pb = static_cast<const u32x4*>(b);
  u32x4* pd = static_cast<u32x4*>(d);
  const int row16 = row_bytes / 16;
  int rc;
  if (nread == 1 && !nwrite) rc = launch_rows_run<1, 0>(run_bytes, pa, pb, pd, T, row16, ncol, tps, (int)nblk, sink, st);
  else if (nread == 1) rc = launch_rows_run<1, 1>(run_bytes, pa, pb, pd, T, row16, ncol, tps, (int)nblk, sink, st);
  else if (!nwrite) rc = launch_rows_run<2, 0>(run_bytes, pa, pb, pd, T, row16, ncol, tps, (int)nblk, sink, st);
  else rc = launch_rows_run<2, 1>(run_bytes, pa, pb, pd, T, row16, ncol, tps, (int)nblk, sink, st);
  if (rc) return rc;
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// T tokens of `rows` (<= 16) rows of row_bytes (a multiple of 1024) each;
// grid = row_bytes / 1024 column blocks x ceil(T / 64) token tiles.
int xhc_probe_frag(const void* a, int T, int rows, int row_bytes, int mode, unsigned* sink, hipStream_t st) {
  if (!a || T < 1 || rows < 1 || rows > 16 || row_bytes < 1024 || (row_bytes % 1024) || !sink) return -1;
  if (mode != 0 && mode != 1) return -1;
  const int ncb = row_bytes / 1024;
  const int64_t nblk = (int64_t)ncb * ((T + FRAG_TOK - 1) / FRAG_TOK);
  if (nblk > (1 << 30)) return -1;
  const unsigned char* pa = static_cast<const unsigned char*>(a);
  if (mode == 0) k_frag<0><<<(int)nblk, 64 * FRAG_WAVES, 0, st>>>(pa, T, rows, row_bytes, ncb, sink);
  else k_frag<1><<<(int)nblk, 64 * FRAG_WAVES, 0, st>>>(pa, T, rows, row_bytes, ncb, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"

// Device-side helpers shared by the xHC kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace xhc {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Storage element types.
struct BF16 { static constexpr int bytes = 2; };
struct F32 { static constexpr int bytes = 4; };

// ---------------------------------------------------------------------------
// W consecutive elements held by one lane, loaded and stored with one vector
// access per 16 bytes.  V8 is also one lane's share of an MFMA K=32 step.
// ---------------------------------------------------------------------------
template <typename E, int W> struct Vec;

template <int W> struct Vec<BF16, W> {
  static constexpr int NW = W / 2;          // 32-bit words
  unsigned w[NW];                           // element 2j in the low half of w[j]
  __device__ static Vec zero() {
    Vec v;
#pragma unroll
    for (int j = 0; j < NW; ++j) v.w[j] = 0u;
    return v;
  }
  __device__ static Vec load(const void* base, size_t elem) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + elem;
    Vec v;
    if constexpr (W == 8) {
      u32x4 r = *reinterpret_cast<const u32x4*>(p);
      v.w[0] = r[0]; v.w[1] = r[1]; v.w[2] = r[2]; v.w[3] = r[3];
    } else if constexpr (W == 4) {
      u32x2 r = *reinterpret_cast<const u32x2*>(p);
      v.w[0] = r[0]; v.w[1] = r[1];
    } else {
      v.w[0] = *reinterpret_cast<const unsigned*>(p);
    }
    return v;
  }
  // a whole vector of 8, read non-temporal (the data's last use in a pass)
  __device__ static Vec load_nt(const void* base, size_t elem) {
    static_assert(W == 8, "non-temporal loads of 16 bytes");
    const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint16_t*>(base) + elem));
    Vec v;
    v.w[0] = r[0]; v.w[1] = r[1]; v.w[2] = r[2]; v.w[3] = r[3];
    return v;
  }
  __device__ void store(void* base, size_t elem) const {
    uint16_t* p = reinterpret_cast<uint16_t*>(base) + elem;
    if constexpr (W == 8) {
      *reinterpret_cast<u32x4*>(p) = u32x4{w[0], w[1], w[2], w[3]};
    } else if constexpr (W == 4) {
      *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
    } else {
      *reinterpret_cast<unsigned*>(p) = w[0];
    }
  }
  __device__ float f(int j) const {
    unsigned x = w[j >> 1];
    return __uint_as_float((j & 1) ? (x & 0xffff0000u) : (x << 16));
  }
  __device__ void to_float(float* o) const {
#pragma unroll
    for (int j = 0; j < W; ++j) o[j] = f(j);
  }
  __device__ static Vec from_float(const float* x) {
    Vec v;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      bf16x2 p = {(__bf16)x[2 * j], (__bf16)x[2 * j + 1]};   // RNE (v_cvt_pk_bf16_f32)
      v.w[j] = __builtin_bit_cast(unsigned, p);
    }
    return v;
  }
};

template <int W> struct Vec<F32, W> {
  float x[W];
  __device__ static Vec zero() {
    Vec v;
#pragma unroll
    for (int j = 0; j < W; ++j) v.x[j] = 0.f;
    return v;
  }
  __device__ static Vec load(const void* base, size_t elem) {
    const float* p = reinterpret_cast<const float*>(base) + elem;
    Vec v;
#pragma unroll
    for (int q = 0; q < W; q += 4) {
      if constexpr (W >= 4) {
        f32x4 r = *reinterpret_cast<const f32x4*>(p + q);
        v.x[q] = r[0]; v.x[q + 1] = r[1]; v.x[q + 2] = r[2]; v.x[q + 3] = r[3];
      }
    }
    if constexpr (W == 2) {
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      f32x2 r = *reinterpret_cast<const f32x2*>(p);
      v.x[0] = r[0]; v.x[1] = r[1];
    }
    return v;
  }
  __device__ static Vec load_nt(const void* base, size_t elem) {
    static_assert(W % 4 == 0, "non-temporal loads of 16 bytes");
    const float* p = reinterpret_cast<const float*>(base) + elem;
    Vec v;
#pragma unroll
    for (int q = 0; q < W; q += 4) {
      const f32x4 r = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + q));
      v.x[q] = r[0]; v.x[q + 1] = r[1]; v.x[q + 2] = r[2]; v.x[q + 3] = r[3];
    }
    return v;
  }
  __device__ void store(void* base, size_t elem) const {
    float* p = reinterpret_cast<float*>(base) + elem;
    if constexpr (W >= 4) {
#pragma unroll
      for (int q = 0; q < W; q += 4)
        *reinterpret_cast<f32x4*>(p + q) = f32x4{x[q], x[q + 1], x[q + 2], x[q + 3]};
    } else {
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      *reinterpret_cast<f32x2*>(p) = f32x2{x[0], x[1]};
    }
  }
  __device__ float f(int j) const { return x[j]; }
  __device__ void to_float(float* o) const {
#pragma unroll
    for (int j = 0; j < W; ++j) o[j] = x[j];
  }
  __device__ static Vec from_float(const float* y) {
    Vec v;
#pragma unroll
    for (int j = 0; j < W; ++j) v.x[j] = y[j];
    return v;
  }
};

template <typename E> using V8 = Vec<E, 8>;

// ---------------------------------------------------------------------------
// Raw buffer access: a 128-bit resource (base, byte size) in SGPRs, a per-lane
// byte offset in a VGPR and a uniform byte offset in an SGPR.  Reads past the
// resource's size return zero; writes past it are dropped.
// ---------------------------------------------------------------------------
// LDS and global address-space pointers for the LDS-DMA loads (the LDS
// destination must be an address-space-3 pointer for the compiler to see
// the write)
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int n>
__device__ inline void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for data the waves exchange through LDS.  It waits for
// this wave's own LDS accesses (lgkmcnt) and nothing else, then meets the
// other waves.  __syncthreads() also waits for every global load this wave
// has in flight: its fence counts an LDS-DMA copy as an LDS write, and
// copies and loads share one counter, so a prefetch issued before it would
// land before the barrier instead of behind the work that follows.  Copies
// that the other side of the barrier reads must be waited for explicitly
// (wait_vmcnt) before calling this.  The memory clobber keeps the compiler
// from moving memory accesses across the barrier.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0); vmcnt and expcnt left alone (gfx9 encoding)
  asm volatile("s_barrier" ::: "memory");
}

// Bitwise OR of two vectors, one of them zero: picks the other without a
// per-lane branch (two loads of which one reads nothing, then the OR).
template <int W>
__device__ inline Vec<BF16, W> vor(const Vec<BF16, W>& a, const Vec<BF16, W>& b) {
  Vec<BF16, W> v;
#pragma unroll
  for (int j = 0; j < W / 2; ++j) v.w[j] = a.w[j] | b.w[j];
  return v;
}
template <int W>
__device__ inline Vec<F32, W> vor(const Vec<F32, W>& a, const Vec<F32, W>& b) {
  Vec<F32, W> v;
#pragma unroll
  for (int j = 0; j < W; ++j) v.x[j] = __uint_as_float(__float_as_uint(a.x[j]) | __float_as_uint(b.x[j]));
  return v;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
// rows * row_bytes as a buffer size, saturated below 4 GiB
__device__ inline uint32_t clamp_bytes(int rows, uint32_t row_bytes) {
  const uint64_t b = (uint64_t)(uint32_t)rows * row_bytes;
  return b > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)b;
}

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// make_rsrc with the base address and size read from the first lane: the
// compiler keeps the resource in scalar registers even where it cannot prove
// the operands uniform (a resource in vector registers turns every access
// into a loop over the distinct values).  The operands must be uniform.
__device__ inline rsrc_t make_rsrc_u(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint32_t n = (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes);
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), n);
}

// Cache policy of a buffer access: CP_NT marks the line non-temporal (the
// store streams to memory instead of sitting dirty in the caches).  It pays
// where each instruction writes whole 128-byte lines that no later kernel of
// the pass reads soon; a line written in halves by two waves is slower.
constexpr int CP_DEFAULT = 0;
constexpr int CP_NT = 2;

template <typename E, int W, int CP = CP_DEFAULT>
__device__ inline Vec<E, W> bload(rsrc_t r, uint32_t voff, uint32_t soff) {
  constexpr int B = W * E::bytes;
  Vec<E, W> v;
  if constexpr (B == 4) {
    const unsigned x = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, CP);
    __builtin_memcpy(&v, &x, 4);
  } else if constexpr (B == 8) {
    const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, CP);
    __builtin_memcpy(&v, &x, 8);
  } else if constexpr (B == 16) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CP);
    __builtin_memcpy(&v, &x, 16);
  } else {
    static_assert(B == 32, "vector width");
    const u32x4 x0 = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CP);
    const u32x4 x1 = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, soff, CP);
    __builtin_memcpy(&v, &x0, 16);
    __builtin_memcpy(reinterpret_cast<char*>(&v) + 16, &x1, 16);
  }
  return v;
}

template <typename E, int W, int CP = CP_DEFAULT>
__device__ inline void bstore(const Vec<E, W>& v, rsrc_t r, uint32_t voff, uint32_t soff) {
  constexpr int B = W * E::bytes;
  if constexpr (B == 4) {
    unsigned x;
    __builtin_memcpy(&x, &v, 4);
    __builtin_amdgcn_raw_buffer_store_b32(x, r, voff, soff, CP);
  } else if constexpr (B == 8) {
    u32x2 x;
    __builtin_memcpy(&x, &v, 8);
    __builtin_amdgcn_raw_buffer_store_b64(x, r, voff, soff, CP);
  } else if constexpr (B == 16) {
    u32x4 x;
    __builtin_memcpy(&x, &v, 16);
    __builtin_amdgcn_raw_buffer_store_b128(x, r, voff, soff, CP);
  } else {
    static_assert(B == 32, "vector width");
    u32x4 x0, x1;
    __builtin_memcpy(&x0, &v, 16);
    __builtin_memcpy(&x1, reinterpret_cast<const char*>(&v) + 16, 16);
    __builtin_amdgcn_raw_buffer_store_b128(x0, r, voff, soff, CP);
    __builtin_amdgcn_raw_buffer_store_b128(x1, r, voff + 16, soff, CP);
  }
}

// One K=32 step of a 16x16 fp32-accumulating MFMA tile.  Lane l holds row
// (A) or column (B) l%16 and the 8 K-elements of group l/16; the K order
// inside a step is free as long as A and B use the same one.
__device__ inline f32x4 mma32(const V8<BF16>& a, const V8<BF16>& b, f32x4 c) {
  u32x4 ra = {a.w[0], a.w[1], a.w[2], a.w[3]};
  u32x4 rb = {b.w[0], b.w[1], b.w[2], b.w[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ra),
                                                 __builtin_bit_cast(bf16x8, rb), c, 0, 0, 0);
}
__device__ inline f32x4 mma32(const V8<F32>& a, const V8<F32>& b, f32x4 c) {
  // eight 16x16x4 steps, step s taking element s of every lane's group
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f(s), b.f(s), c, 0, 0, 0);
  return c;
}

// One K=16 step of a 16x16 MFMA: lane l holds row/column l%16 and the 4
// K-elements of group l/16 (bf16: 16x16x16; fp32: four 16x16x4 steps).
__device__ inline f32x4 mma16(const Vec<BF16, 4>& a, const Vec<BF16, 4>& b, f32x4 c) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  u32x2 ra = {a.w[0], a.w[1]}, rb = {b.w[0], b.w[1]};
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, ra), __builtin_bit_cast(s16x4, rb), c,
                                                   0, 0, 0);
}
__device__ inline f32x4 mma16(const Vec<F32, 4>& a, const Vec<F32, 4>& b, f32x4 c) {
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f(s), b.f(s), c, 0, 0, 0);
  return c;
}

// Split an fp32 value into bf16 hi + lo (hi = RNE(x), lo = RNE(x - hi)):
// hi + lo carries ~16 significant bits, enough for fp32-accurate products.
__device__ inline void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

__device__ inline float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

__device__ inline float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Cross-lane steps on the VALU (gfx950), for wave-wide reductions:
// swap32(x, y) / swap16(x, y) return x + y' where the permlane swap moves
// y's values of the lower half (lanes 0..31, or rows 0 and 2) to the upper
// half and x's values of the upper half to the lower half.  With x = the
// values a lane keeps when its bit (5, resp. 4) is 0 and y = those it keeps
// when the bit is 1, the result is the lane's kept value summed with its
// partner's (lane ^ 32, resp. lane ^ 16): one step of a halving exchange.
__device__ inline float halve32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float halve16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// DPP lane moves within rows of 16: value of lane (l ^ 15), of lane (l ^ 7),
// of lane (l ^ 2) and of lane (l ^ 1)
__device__ inline float dpp_xor15(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
}
__device__ inline float dpp_xor7(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
}
__device__ inline float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ inline float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
// value of lane (l ^ 8) and of lane (l ^ 4) within rows of 16 (rotations by
// 8, and by 4 or 12 depending on lane bit 2)
__device__ inline float dpp_xor8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}
__device__ inline float dpp_xor4(float v) {
  const float a = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
  const float b = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x12C, 0xF, 0xF, false));
  return (__lane_id() & 4) ? a : b;
}
// exact xor-partner exchange within 16-lane rows, m in {1, 2, 4, 8}
template <int m>
__device__ inline float row_xor(float v) {
  static_assert(m == 1 || m == 2 || m == 4 || m == 8, "row xor mask");
  if constexpr (m == 1) return dpp_xor1(v);
  else if constexpr (m == 2) return dpp_xor2(v);
  else if constexpr (m == 4) return dpp_xor4(v);
  else return dpp_xor8(v);
}

// compile-time loop: f(std::integral_constant<int, I>) for I in [I0, I1)
template <int I0, int I1, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < I1) {
    f(std::integral_constant<int, I0>{});
    static_for<I0 + 1, I1>(f);
  }
}

// XCD-aware remap of the linear workgroup id.  Workgroups are dispatched to
// the 8 XCDs round-robin (id % 8); this returns a logical id such that each
// XCD receives one contiguous range of logical ids, so neighbouring tiles
// (which share operands) sit behind the same L2.  Requires nblocks % 8 == 0;
// otherwise the id is returned unchanged.
__device__ inline int xcd_logical_block(int bid, int nblocks) {
  if (nblocks & 7) return bid;
  return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

}  // namespace xhc

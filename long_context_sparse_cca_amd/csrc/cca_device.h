// Device-side helpers shared by the CCA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cca {

constexpr int kWave = 64;

// bfloat16 is stored as its 16-bit pattern; arithmetic happens in float32.
struct bf16_t {
  uint16_t bits;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even float32 -> bfloat16 bits (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// IEEE binary16 is stored as its 16-bit pattern; arithmetic happens in float32.
struct f16_t {
  uint16_t bits;
};

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// Round-to-nearest-even float32 -> binary16 bits (overflow gives infinity).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
}

// Element traits: loads of 16-byte chunks and conversion to float.
template <typename T> struct Elem;

template <> struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;  // elements per 16-byte chunk
  __device__ __forceinline__ static void chunk_to_f32(const uint4& c, float* f) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static float load1(const bf16_t* p) { return bf16_bits_to_f32(p->bits); }
  __device__ __forceinline__ static void store1(bf16_t* p, float v) { p->bits = f32_to_bf16_bits(v); }
  // 16-bit types: one element from its bits, two from a 32-bit word, two packed into one
  __device__ __forceinline__ static float bits_to_f32(uint32_t h) { return bf16_bits_to_f32(h); }
  __device__ __forceinline__ static void pair_to_f32(uint32_t w, float* f) {
    f[0] = __uint_as_float(w << 16);
    f[1] = __uint_as_float(w & 0xffff0000u);
  }
  __device__ __forceinline__ static uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
  static constexpr uint16_t kNaNBits = 0x7fc0;
};

template <> struct Elem<f16_t> {
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;
  __device__ __forceinline__ static void chunk_to_f32(const uint4& c, float* f) {
    const f16x8_t h = __builtin_bit_cast(f16x8_t, c);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
  }
  __device__ __forceinline__ static float load1(const f16_t* p) { return f16_bits_to_f32(p->bits); }
  __device__ __forceinline__ static void store1(f16_t* p, float v) { p->bits = f32_to_f16_bits(v); }
  __device__ __forceinline__ static float bits_to_f32(uint32_t h) { return f16_bits_to_f32(h); }
  __device__ __forceinline__ static void pair_to_f32(uint32_t w, float* f) {
    const f16x2_t h = __builtin_bit_cast(f16x2_t, w);
    f[0] = (float)h[0];
    f[1] = (float)h[1];
  }
  __device__ __forceinline__ static uint32_t pack2(float lo, float hi) { return pack_f16x2(lo, hi); }
  static constexpr uint16_t kNaNBits = 0x7e00;
};

template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  static constexpr int kPerChunk = 4;
  __device__ __forceinline__ static void chunk_to_f32(const uint4& c, float* f) {
    f[0] = __uint_as_float(c.x);
    f[1] = __uint_as_float(c.y);
    f[2] = __uint_as_float(c.z);
    f[3] = __uint_as_float(c.w);
  }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
  __device__ __forceinline__ static void store1(float* p, float v) { *p = v; }
};

// Matrix-core traits of the 16-bit element types: the 32x32x16 and 16x16x32 MFMAs on
// 16-byte operand registers, the rounding of two float32 values into one operand word, and
// the two-term dot product with float32 accumulation.  Tile fills and LDS transpose reads
// move 16-bit elements without looking at them, so they need nothing type-specific.
template <typename T> struct Mma16;
template <> struct Mma16<bf16_t> {
  typedef __bf16 x2 __attribute__((ext_vector_type(2)));
  __device__ __forceinline__ static f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4_t mfma16(const uint4& a, const uint4& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  }
  __device__ __forceinline__ static x2 round2(float a, float b) { return x2{(__bf16)a, (__bf16)b}; }
  __device__ __forceinline__ static float dot2(x2 a, x2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
};
template <> struct Mma16<f16_t> {
  typedef _Float16 x2 __attribute__((ext_vector_type(2)));
  __device__ __forceinline__ static f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  }
  __device__ __forceinline__ static f32x4_t mfma16(const uint4& a, const uint4& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  }
  __device__ __forceinline__ static x2 round2(float a, float b) { return x2{(_Float16)a, (_Float16)b}; }
  __device__ __forceinline__ static float dot2(x2 a, x2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// 16-byte load of data that one launch reads once (the K/V rows a decode step or a pooling
// pass streams): the nontemporal hint keeps such rows from displacing reused lines in the
// caches, and on this part it lifts a long read stream from about 6.0 to about 6.5 TB/s.
// A working set near or below the 256 MB last-level cache is better read the ordinary way:
// repeated decode steps over it then partly hit that cache (measured: a 238 MB serving step
// takes 58 us with ordinary loads, 65 us with streaming ones).  kStreamBytes (1.5x that
// cache) is the switch-over, applied to an upper bound of the step's K/V bytes.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}
template <bool STREAM>
__device__ __forceinline__ uint4 ld16_kv(const void* p) {
  if constexpr (STREAM) return ld16_stream(p);
  else return ld16(p);
}
constexpr int64_t kStreamBytes = (int64_t)384 << 20;

// Butterfly reductions over the lanes of a wave that differ in the bits of `mask_bits`.
__device__ __forceinline__ float wave_max_xor(float v, int lo_bit, int hi_bit) {
  for (int b = lo_bit; b < hi_bit; b <<= 1) v = fmaxf(v, __shfl_xor(v, b, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum_xor(float v, int lo_bit, int hi_bit) {
  for (int b = lo_bit; b < hi_bit; b <<= 1) v += __shfl_xor(v, b, kWave);
  return v;
}

// Sum over aligned groups of N consecutive lanes (N in {1, 2, 4, 8, 16}) with DPP
// row operations (no LDS traffic): two quad permutes, then the half-row and the
// row mirror.  Every lane of a group ends with the bitwise-same total (each step
// adds two equal partial sums in either order, and float addition commutes).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float lane_group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1..16 lanes");
  if constexpr (N >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp_mov<0x140>(x); // row_mirror
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Orders the LDS accesses of the lanes of one wave around this point (for LDS
// scratch that a single wave owns): the LDS operations of a wave complete in
// order, so a compiler-level fence plus a wave barrier suffice.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr float kLog2e = 1.4426950408889634f;
// Finite stand-in for -infinity as the initial running max: keeps
// exp2(m_old - m_new) finite when a row has seen only masked keys.
constexpr float kNegBig = -1.0e30f;

// Workgroup -> (slice, query tile).  Consecutive workgroups are dealt round-robin
// to the 8 XCDs; when the grid divides evenly, XCD x gets a contiguous range of
// slices and, inside a slice, the query tiles from the heaviest (last) down, so
// that the co-resident workgroups of one XCD sweep the same core K/V in its L2.
__device__ __forceinline__ void map_block(int nblocks, int ntiles, int& bh, int& tile) {
  const int bid = blockIdx.x;
  int li = bid;
  if ((nblocks & 7) == 0) li = (bid & 7) * (nblocks >> 3) + (bid >> 3);
  bh = li / ntiles;
  tile = ntiles - 1 - (li - bh * ntiles);
}

// Query slice (b*Hq + h) of virtual slice v for attention over a cache of sequences of
// different lengths: map_block hands each XCD a contiguous range of slices, so the
// slices are taken in the order (key/value head, sequence, query head of that key/value
// head).  Every XCD then gets every sequence (balanced work), and the nq query heads
// that read one key/value slice stay adjacent (they share its tiles in L2).  The
// sequences come in the order `order` gives (longest first), so that each XCD hands out
// its heaviest workgroups first and the light ones fill the tail.
__device__ __forceinline__ int kv_major_slice(int v, int BH, int Hq, int nq, const int32_t* order) {
  const int B = BH / Hq;
  const int per_kv = B * nq;
  const int hkv = v / per_kv;
  const int rem = v - hkv * per_kv;
  const int i = rem / nq;
  return order[i] * Hq + hkv * nq + (rem - i * nq);
}

}  // namespace cca

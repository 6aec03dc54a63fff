// Device-side helpers shared by the gfx950 kernels of the drafting hot path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// bfloat16 values live in memory as raw 16-bit words.
typedef uint16_t bf16_t;

// Eight consecutive storage elements as raw bits: 16 bytes for bf16, 32 for fp32.
struct Raw8 {
  u32x4 lo, hi;
};

template <typename S>
__device__ __forceinline__ void load_raw8(Raw8& r, const S* p);
template <>
__device__ __forceinline__ void load_raw8<bf16_t>(Raw8& r, const bf16_t* p) {
  r.lo = *reinterpret_cast<const u32x4*>(p);
}
template <>
__device__ __forceinline__ void load_raw8<float>(Raw8& r, const float* p) {
  r.lo = reinterpret_cast<const u32x4*>(p)[0];
  r.hi = reinterpret_cast<const u32x4*>(p)[1];
}

// Streaming (non-temporal) variant for data read exactly once per step (weights, logits).
template <typename S>
__device__ __forceinline__ void load_raw8_nt(Raw8& r, const S* p);
template <>
__device__ __forceinline__ void load_raw8_nt<bf16_t>(Raw8& r, const bf16_t* p) {
  r.lo = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
template <>
__device__ __forceinline__ void load_raw8_nt<float>(Raw8& r, const float* p) {
  r.lo = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  r.hi = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
}

// 8-bit KV entries (int8 values; their run scales are loaded separately):
// eight consecutive values in the low 8 bytes of a Raw8.
template <>
__device__ __forceinline__ void load_raw8<int8_t>(Raw8& r, const int8_t* p) {
  const u32x2 t = *reinterpret_cast<const u32x2*>(p);
  r.lo = u32x4{t[0], t[1], 0u, 0u};
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 round-to-nearest-even (hardware conversion on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

__device__ __forceinline__ bf16x8 f32x8_to_bf16x8(f32x4 a, f32x4 b) {
  bf16x8 r;
  r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
  r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
  return r;
}

// A pair of fp32 values as a bf16 hi/lo pair (x = hi + lo + O(2^-17 |x|)):
// one packed conversion for the two hi values, whose fp32 values are the
// packed word's halves (a shift and a mask), then one for the two remainders.
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x0, x1}, bf16x2_t));
  const float r0 = x0 - __uint_as_float(hi << 16), r1 = x1 - __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{r0, r1}, bf16x2_t));
}

// Element (m, k) of an [M, K] bf16 activation stored in matrix-core fragment
// blocks (K % 32 == 0): the 16 x 32 block (rows 16a.., columns 32s..) is 1 KB
// at ((a * K/32 + s) * 64) * 8 elements, lane l of it holding row 16a + (l & 15),
// columns 32s + 8(l >> 4) .. + 7 -- the order of the tiled weight copy, so a
// 16-row k-step of activations is one contiguous kilobyte.
__device__ __forceinline__ size_t frag_block_index(int m, int k, int K) {
  return ((size_t)(m >> 4) * (size_t)(K >> 5) + (size_t)(k >> 5)) * 512 + (size_t)(((m & 15) | (k & 24) << 1) << 3) +
         (size_t)(k & 7);
}

// Raw storage bits -> bf16x8 MFMA operand.
template <typename S>
__device__ __forceinline__ bf16x8 raw_to_bf16x8(const Raw8& r);
template <>
__device__ __forceinline__ bf16x8 raw_to_bf16x8<bf16_t>(const Raw8& r) {
  return __builtin_bit_cast(bf16x8, r.lo);
}
template <>
__device__ __forceinline__ bf16x8 raw_to_bf16x8<float>(const Raw8& r) {
  return f32x8_to_bf16x8(__builtin_bit_cast(f32x4, r.lo), __builtin_bit_cast(f32x4, r.hi));
}

// Raw storage bits -> 8 floats.
template <typename S>
__device__ __forceinline__ void raw_to_f32x8(const Raw8& r, float* out);
template <>
__device__ __forceinline__ void raw_to_f32x8<bf16_t>(const Raw8& r, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(r.lo[i] << 16);
    out[2 * i + 1] = __uint_as_float(r.lo[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void raw_to_f32x8<float>(const Raw8& r, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[i] = __uint_as_float(r.lo[i]);
    out[4 + i] = __uint_as_float(r.hi[i]);
  }
}

template <>
__device__ __forceinline__ void raw_to_f32x8<int8_t>(const Raw8& r, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[i] = (float)((int32_t)(r.lo[0] << (24 - 8 * i)) >> 24);
    out[4 + i] = (float)((int32_t)(r.lo[1] << (24 - 8 * i)) >> 24);
  }
}

template <typename S>
__device__ __forceinline__ float load_f32(const S* p);
template <>
__device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p) { return bf16_bits_to_f32(*p); }

template <typename S>
__device__ __forceinline__ void store_from_f32(S* p, float v);
template <>
__device__ __forceinline__ void store_from_f32<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_from_f32<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16_bits(v); }

// 16x16x32 bf16 matrix-core product, fp32 accumulate.
// Operand lanes: A row (lane & 15), B column (lane & 15), 8 k-values per lane
// whose k-slot depends on (lane >> 4); A and B loaded with the same slot map
// contract the same k.  Result: lane holds column (lane & 15), rows
// 4 * (lane >> 4) + [0, 4).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- argmax key
// Monotone packing of (value, index) into one u64: higher value wins, exact
// ties go to the lower index, NaN ranks below every number (so it is never
// chosen unless the whole row is NaN, in which case index 0 wins), -0 == +0.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
  uint32_t hi;
  if (v != v) {
    hi = 0u;
  } else {
    uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
    hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(0xffffffffu - idx);
}
__device__ __forceinline__ int32_t argmax_key_index(uint64_t key) {
  return static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(key));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m);
  uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}
// v of lane (lane ^ 1) / (lane ^ 2): DPP quad permutes, register to register
// (a general shuffle goes through the LDS pipe, ~100 cycles a round).
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt vmcnt(0): every vector memory access of the wave has completed.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------- LDS-DMA
// global_load_lds_dwordx4 (gfx950) writes lane l's 16 bytes at the
// wave-uniform LDS address + 16 * l; the loads count in vmcnt like any other
// and complete in issue order.  Waits for them are explicit: the compiler
// treats a register load followed by LDS-DMA loads as possibly completing out
// of order and waits for all of them before using the register, and a
// workgroup fence waits for every LDS-DMA load in flight.
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void lds_dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds_dst, 16, 0, 0);
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt untouched).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0): this wave's LDS writes are done.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier without a memory fence (the compiler keeps memory
// accesses on their side of it; the waits before it are explicit).
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float silu_f32(float x) {
  return x / (1.0f + fast_exp2(-x * 1.4426950408889634f));
}

}  // namespace dfl

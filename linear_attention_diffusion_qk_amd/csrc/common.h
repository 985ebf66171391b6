// Shared device helpers for the gfx950 kernels of libsanala.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

namespace sanala {

constexpr int kPartStride = kHeadDim * kHeadDim + kHeadDim;  // 1056 floats: S row-major [d][e], then z[d]

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
// The value of f after rounding to bf16, as fp32.
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(f32_to_bf16_bits(f) << 16); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }
__device__ __forceinline__ f32x4 as_f32x4(u32x4 w) { return __builtin_bit_cast(f32x4, w); }

// acc + a.lo*b.lo + a.hi*b.hi for two packed bf16 pairs (v_dot2_f32_bf16; products exact in fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

// ReLU of two packed bf16 values: a bf16 with its sign bit set is a negative 16-bit integer, so a
// packed signed 16-bit max with 0 zeroes exactly the negative values (and -0).
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(i16x2, w), (i16x2){0, 0}));
}

// Two fp32 values to packed bf16 with the hardware converter (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// IEEE binary16 counterparts (v_dot2_f32_f16, v_cvt_f32_f16, v_cvt_f16_f32 with round to nearest even).
__device__ __forceinline__ f16x8 as_f16x8(u32x4 w) { return __builtin_bit_cast(f16x8, w); }
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }
__device__ __forceinline__ uint32_t cvt_pk_f16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
}

// The 16-bit storage type at compile time: F16 = IEEE binary16, else bf16.  Both keep the sign in the
// top bit of each half, so the integer-max ReLU and the sign-mask XOR serve both.
template <bool F16>
__device__ __forceinline__ float h_lo(uint32_t w) { return F16 ? f16_lo(w) : bf16_lo(w); }
template <bool F16>
__device__ __forceinline__ float h_hi(uint32_t w) { return F16 ? f16_hi(w) : bf16_hi(w); }
template <bool F16>
__device__ __forceinline__ uint32_t cvt_pk_h(float lo, float hi) { return F16 ? cvt_pk_f16(lo, hi) : cvt_pk_bf16(lo, hi); }
template <bool F16>
__device__ __forceinline__ float dot2_h(uint32_t a, uint32_t b, float acc) {
  return F16 ? dot2_f16(a, b, acc) : dot2_bf16(a, b, acc);
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Raw buffer resource over [base, base + bytes) (gfx9 descriptor word 3 for untyped 32-bit access).
// A buffer store whose byte offset is not below `bytes` is discarded by the hardware range check, so
// masked lanes can take kOutOfRange instead of a branch around the store.
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void buffer_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
// Non-temporal forms for outputs this library never reads back: streamed to memory instead of being
// kept in the caches, where their write-back would otherwise land on the next kernel's time.
__device__ __forceinline__ void buffer_store16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 2 /* nt */);
}
__device__ __forceinline__ void store16_nt(void* p, u32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p)); }
// A load whose range check fails returns zeros without a memory access.
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// Device-scope forms (cache policy sc1): the store is written through to the level every XCD reads,
// and the load is served from it, so data one block stores another block on any XCD can load once the
// store has completed, without a fence that writes back or invalidates a whole L2.
constexpr int kScDevice = 16;
__device__ __forceinline__ void buffer_store16_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kScDevice);
}
__device__ __forceinline__ u32x4 buffer_load16_dev(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kScDevice);
}
__device__ __forceinline__ f32x4 loadf4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Sum over the 4 lanes {l, l^16, l^32, l^48} (the four 16-lane groups of a wave64).
__device__ __forceinline__ float sum_over_lane_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

}  // namespace sanala

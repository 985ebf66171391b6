// Operand images of the reduced KV state shared by the 16-bit state kernels and the output kernels.
#pragma once

#include "common.h"

namespace sanala {

constexpr int kOpPerHead = 2 * 64 * 8;  // S' operand per head: 2 e-blocks x 64 lanes x 8 bf16
constexpr int kZopPerHead = 2 * kHeadDim;  // z' per head: 32 bf16 hi, then 32 bf16 lo
constexpr int kSgnPerHead = 16;            // query sign masks per head: 4 lane groups x 4 words

// Position of S'[d][e] inside a head's operand block.  Lane l = m + 16*kg of e-block eb holds
// S'[8*kg + j][e] (j = 0..7) with e = 8*(m/4) + 4*eb + m%4; with that column order the MFMA result
// lane (t, kg) receives output channels 8kg..8kg+7 of token t.
__device__ __forceinline__ int sop_index(int d, int e) {
  const int m = 4 * (e >> 3) + (e & 3), eb = (e >> 2) & 1, kg = d >> 3, j = d & 7;
  return eb * 512 + (m + 16 * kg) * 8 + j;
}

// Sign masks (0x8000 per negative gain) of query dims 8kg + 2u, 8kg + 2u + 1 of head h.
template <bool NORM>
__device__ __forceinline__ uint32_t sign_word(const float* __restrict__ gq, int h, int kg, int u) {
  if (!NORM) return 0u;
  const int d0 = h * kHeadDim + 8 * kg + 2 * u;
  return (gq[d0] < 0.f ? 0x8000u : 0u) | (gq[d0 + 1] < 0.f ? 0x80000000u : 0u);
}

// Writes one reduced state element (i < 1024: S~[i/32][i%32]; else z~[i-1024]) of head h of sample
// row bh as the output kernel's operands, scaled by G_d = |gq_d| |gk_d| (1 without the norm).
template <bool NORM>
__device__ __forceinline__ void emit_state(int64_t bh, int h, int i, float s, const float* __restrict__ gq,
                                           const float* __restrict__ gk, uint16_t* __restrict__ Sop,
                                           uint16_t* __restrict__ zop) {
  const int d = i < kHeadDim * kHeadDim ? i / kHeadDim : i - kHeadDim * kHeadDim;
  if (NORM) s *= fabsf(gq[h * kHeadDim + d]) * fabsf(gk[h * kHeadDim + d]);
  if (i < kHeadDim * kHeadDim) {
    Sop[bh * kOpPerHead + sop_index(d, i % kHeadDim)] = (uint16_t)f32_to_bf16_bits(s);
  } else {
    const uint32_t hi = f32_to_bf16_bits(s);
    zop[bh * kZopPerHead + d] = (uint16_t)hi;
    zop[bh * kZopPerHead + kHeadDim + d] = (uint16_t)f32_to_bf16_bits(s - __uint_as_float(hi << 16));
  }
}

}  // namespace sanala

// Row statistics kernel shared by the fp32 and bf16 paths.
#pragma once

#include "common.h"

namespace sanala {

// r[row] = 1 / sqrt(mean_c x[row, c]^2 + eps) over all C channels of a token row (the QK-Norm
// scale), one wave per row, 16-byte loads (16-bit T: bf16, or binary16 with F16).  Rows are `ld` elements apart.
// With x1 given, the launch covers 2 * rows rows: the second half are the rows of x1 (stride ld1)
// and their scales go to r1 (K and Q in one launch).  NT: rows of up to 64 * MAXU units are read with
// non-temporal loads.
template <typename T, bool F16 = false, bool NT = false>
__global__ __launch_bounds__(256) void rowstats_kernel(const T* __restrict__ x, int64_t ld, int64_t rows, int C,
                                                       float eps, float* __restrict__ r,
                                                       const T* __restrict__ x1 = nullptr, int64_t ld1 = 0,
                                                       float* __restrict__ r1 = nullptr) {
  int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= (x1 ? 2 * rows : rows)) return;
  if (row >= rows) {  // uniform per wave
    x = x1;
    ld = ld1;
    r = r1;
    row -= rows;
  }
  const char* p = reinterpret_cast<const char*>(x + row * ld);
  const int nvec = C * (int)sizeof(T) / 16;
  float ss = 0.f;
  constexpr int MAXU = 8;  // rows of up to 512 units: every load issued before the sums
  if (nvec <= 64 * MAXU) {
    u32x4 w[MAXU];
#pragma unroll
    for (int j = 0; j < MAXU; ++j) {
      const int i = lane + 64 * j;
      if constexpr (NT)
        w[j] = i < nvec ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 16 * (int64_t)i))
                        : u32x4{0u, 0u, 0u, 0u};
      else
        w[j] = i < nvec ? load16(p + 16 * (int64_t)i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < MAXU; ++j) {
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int u = 0; u < 4; ++u) ss = dot2_h<F16>(w[j][u], w[j][u], ss);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float a = __uint_as_float(w[j][u]);
          ss = fmaf(a, a, ss);
        }
      }
    }
  } else {
    for (int i = lane; i < nvec; i += 64) {
      const u32x4 w = load16(p + 16 * (int64_t)i);
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int u = 0; u < 4; ++u) ss = dot2_h<F16>(w[u], w[u], ss);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float a = __uint_as_float(w[u]);
          ss = fmaf(a, a, ss);
        }
      }
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) r[row] = 1.0f / sqrtf(ss / (float)C + eps);
}

}  // namespace sanala

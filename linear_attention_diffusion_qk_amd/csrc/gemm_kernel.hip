// QKV projection qkv[M, 3C] = x[M, C] @ W[C, 3C] on gfx950 MFMA (bf16 in, fp32 accumulate, bf16 out).
//
// The projection that the Sana notes (section 7, on-device deployment) fuse with ReLU(K)^T V; here it
// is a separate dense contraction ahead of the attention kernels.
//
// Block tile 256 x 192, K tile 64, 512 threads = 8 waves as 4 (M) x 2 (N); each wave owns a 64 x 96
// sub-tile = 2 x 3 tiles of v_mfma_f32_32x32x16_bf16.  Both operands are staged through LDS with a
// double buffer: x rows go in as they are (k contiguous), W goes in transposed ([n][k]) because the
// MFMA wants 8 consecutive k per lane for both operands.  Rows past M and columns past 3C are masked.
#include "common.h"

namespace sanala {

namespace {
constexpr int BM = 256, BN = 192, BK = 64;
constexpr int PA = BK + 8;  // LDS pitch (bf16) of the x tile rows
constexpr int PB = BK + 8;  // LDS pitch (bf16) of the transposed W tile rows
constexpr int kThreads = 512;
}  // namespace

__global__ __launch_bounds__(kThreads) void qkv_gemm_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ w,
                                                            uint16_t* __restrict__ y, int64_t M, int K, int NO) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * PA];
  __shared__ __attribute__((aligned(16))) uint16_t Bt[2][BN * PB];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 3, wn = wave >> 2;
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;
  const int li = lane & 31, lg = lane >> 5;

  // global -> register staging
  u32x4 ra[4], rb[3];
  auto load_tile = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int i = tid + it * kThreads;  // 2048 vectors: row = i / 8, 8 vectors per row
      const int row = i >> 3, kc = i & 7;
      const int64_t m = m0 + row;
      ra[it] = (m < M && k0 + kc * 8 < K) ? load16(x + m * K + k0 + kc * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const int i = tid + it * kThreads;  // 1536 vectors: k = i % 64, column octet nc = i / 64
      const int kk = i & 63, nc = i >> 6;
      const int n = n0 + nc * 8;
      rb[it] = (n < NO && k0 + kk < K) ? load16(w + (int64_t)(k0 + kk) * NO + n) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int i = tid + it * kThreads;
      const int row = i >> 3, kc = i & 7;
      store16(&As[buf][row * PA + kc * 8], ra[it]);
    }
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const int i = tid + it * kThreads;
      const int kk = i & 63, nc = i >> 6;
      uint16_t* dst = &Bt[buf][(nc * 8) * PB + kk];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        dst[(2 * u) * PB] = (uint16_t)(rb[it][u] & 0xffffu);
        dst[(2 * u + 1) * PB] = (uint16_t)(rb[it][u] >> 16);
      }
    }
  };

  f32x16 acc[2][3];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 3; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int KT = (K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_tile(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 av[2], bv[3];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        av[a] = as_bf16x8(load16(&As[buf][(wm * 64 + a * 32 + li) * PA + ks * 16 + lg * 8]));
#pragma unroll
      for (int b = 0; b < 3; ++b)
        bv[b] = as_bf16x8(load16(&Bt[buf][(wn * 96 + b * 32 + li) * PB + ks * 16 + lg * 8]));
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    if (kt + 1 < KT) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const int n = n0 + wn * 96 + b * 32 + li;
      if (n >= NO) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + a * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
        if (m < M) y[m * NO + n] = (uint16_t)f32_to_bf16_bits(acc[a][b][r]);
      }
    }
  }
}

hipError_t launch_qkv_gemm(const uint16_t* x, const uint16_t* w, uint16_t* qkv, int64_t M, int C, hipStream_t stream) {
  const int NO = 3 * C;
  if (C % 8 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((M + BM - 1) / BM), (NO + BN - 1) / BN);
  SANA_LAUNCH("qkv_gemm", qkv_gemm_kernel<<<grid, kThreads, 0, stream>>>(x, w, qkv, M, C, NO));
  return hipGetLastError();
}

}  // namespace sanala

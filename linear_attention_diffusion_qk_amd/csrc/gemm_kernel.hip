// QKV projection qkv[M, 3C] = x[M, C] @ W[C, 3C] on gfx950 MFMA (bf16 in, fp32 accumulate, bf16 out).
//
// The projection that the Sana notes (section 7, on-device deployment) fuse with ReLU(K)^T V; here it
// is a separate dense contraction ahead of the attention kernels.
//
// Block tile 256 (rows of x) x 192 (columns of W), K step 32, 4 waves as 2 x 2, wave tile 128 x 96.
// Tiles of x and W go from global memory straight to LDS (global_load_lds_dwordx4) through a ring of
// 4 stage buffers, so up to three K steps are in flight while one is multiplied; the buffers are
// separate LDS objects read through a restrict-qualified pointer, which lets the compiler see that
// reading one stage does not wait for the loads into the others.  Both LDS images are XOR-swizzled in
// 16-byte units so that the operand reads are free of bank conflicts:
//   x tile [256][32] (64-byte rows): unit kc of row m sits at unit kc ^ (((m >> 1) ^ (m >> 2)) & 3);
//   W tile [32][192] (384-byte rows): unit nc of row k sits at unit nc ^ (2 * (k & 3)).
// The product is formed transposed, Y^T = W^T x^T, on v_mfma_f32_32x32x16_bf16: the W operand (8
// consecutive k of one column per lane) comes from two ds_read_b64_tr_b16 transposing reads of the
// row-major W tile, the x operand from one ds_read_b128 of an x row.  Each lane then holds 4
// consecutive output columns of one row per accumulator quad and writes them as one 8-byte store.
// With at least 8 row panels, block ids congruent mod 8 (one XCD) cover a slab of row panels, and the
// 32 CUs of an XCD work on 8 row panels x 4 column panels at a time, so their slices stay in its L2.
#include "common.h"

#include <algorithm>
#include <type_traits>

namespace sanala {

namespace {
constexpr int BM = 256, BN = 192, BK = 32, STAGES = 4;
constexpr int kThreads = 256;
constexpr int A_ROW = BK * 2;                   // 64 bytes per x tile row
constexpr int B_ROW = BN * 2;                   // 384 bytes per W tile row
constexpr int A_BYTES = BM * A_ROW;             // 16 KB
constexpr int B_BYTES = BK * B_ROW;             // 12 KB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;  // 28 KB
constexpr int A_DMA = A_BYTES / 1024 / 4;       // 1-KB wave instructions per wave per stage: 4
constexpr int B_DMA = B_BYTES / 1024 / 4;       // 3
constexpr int DMA_PER_STAGE = A_DMA + B_DMA;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;

// s_waitcnt with only vmcnt <= n (n < 64); expcnt and lgkmcnt are not waited on.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16-byte unit kc of x row m sits at unit kc ^ xswz(m): for a fixed kc, any 8 consecutive rows use 8
// different 16-byte slots of a 128-byte bank line and any 16 consecutive rows 16 different slots of 256 bytes.
__device__ __forceinline__ int xswz(int m) { return ((m >> 1) ^ (m >> 2)) & 3; }
__device__ __forceinline__ int x_addr(int m, int kc) { return m * A_ROW + 16 * (kc ^ xswz(m)); }
__device__ __forceinline__ int w_addr(int k, int n) {  // byte offset of W tile element (k, n)
  return k * B_ROW + 16 * ((n >> 3) ^ (2 * (k & 3))) + 2 * (n & 7);
}

__shared__ __attribute__((aligned(1024))) char g_stage0[STAGE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_stage1[STAGE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_stage2[STAGE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_stage3[STAGE_BYTES];

template <int S>
__device__ __forceinline__ char* stage_buf() {
  static_assert(S >= 0 && S < STAGES, "stage index");
  return S == 0 ? g_stage0 : S == 1 ? g_stage1 : S == 2 ? g_stage2 : g_stage3;
}

// Lane roles in the operand reads of one wave.
struct Roles {
  int xrow;    // x row of mt = 0 (+ 32 mt)
  int xhalf;   // 16-byte k unit 2s + xhalf
  int wn_col;  // W column of nt = 0 read by this lane's transposing read (+ 32 nt)
  int wk;      // W row of sub-step 0, low half (+ 16 s, + 4 for the high half)
};

// Operands of one K step (two 16-wide sub-steps) of one wave.
struct Ops {
  bf16x8 xa[BK / 16][4];
  bf16x8 wb[BK / 16][3];
};

// Reads a K step's operands from a stage buffer.  The roles are taken by value: read through a
// reference they would be memory accesses of their own, and the compiler could then no longer keep the
// stage reads apart from the loads still landing in the other buffers.
__device__ __forceinline__ void read_ops(const char* __restrict__ As, Roles ro, Ops& op) {
  const char* __restrict__ Bs = As + A_BYTES;
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      op.xa[s][mt] = as_bf16x8(*reinterpret_cast<const u32x4*>(As + x_addr(ro.xrow + 32 * mt, 2 * s + ro.xhalf)));
#pragma unroll
    for (int nt = 0; nt < 3; ++nt) {
      const int n = ro.wn_col + 32 * nt;
      const int k = 16 * s + ro.wk;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(Bs + w_addr(k, n)));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(Bs + w_addr(k + 4, n)));
      const v4s both[2] = {lo, hi};
      op.wb[s][nt] = *reinterpret_cast<const bf16x8*>(both);
    }
  }
}

__device__ __forceinline__ void mma(const Ops& op, int s, f32x16 (&acc)[3][4]) {
#pragma unroll
  for (int nt = 0; nt < 3; ++nt)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      acc[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op.wb[s][nt], op.xa[s][mt], acc[nt][mt], 0, 0, 0);
}
}  // namespace

__global__ __launch_bounds__(kThreads) void qkv_gemm_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ w,
                                                            uint16_t* __restrict__ y, int M, int K, int NO,
                                                            int mblocks, int nblocks, int slab,
                                                            float* __restrict__ k_ssq, int k_parts) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  int mb, nb;
  if (slab > 0) {  // XCD-aware order (see the header)
    const int xcd = (int)(blockIdx.x & 7u), local = (int)(blockIdx.x >> 3);
    mb = xcd * slab + local % slab;
    nb = local / slab;
  } else {
    mb = (int)blockIdx.x / nblocks;
    nb = (int)blockIdx.x % nblocks;
  }
  if (mb >= mblocks || nb >= nblocks) return;
  const int m0 = mb * BM, n0 = nb * BN;

  // Per-lane sources of this wave's DMA instructions (the K step is added per stage).  A instruction
  // i covers rows 16i..16i+15 of the x image, B instruction i bytes [1024i, 1024i + 1024) of the W
  // image.  Rows past M and columns past NO read clamped addresses; their products are never stored.
  const uint16_t* a_src[A_DMA];
  const uint16_t* b_src[B_DMA];
#pragma unroll
  for (int a = 0; a < A_DMA; ++a) {
    const int r = 16 * (wave * A_DMA + a) + (lane >> 2);
    const int kc = (lane & 3) ^ xswz(r);
    a_src[a] = x + (int64_t)min(m0 + r, M - 1) * K + 8 * kc;
  }
#pragma unroll
  for (int b = 0; b < B_DMA; ++b) {
    const int off = 1024 * (wave * B_DMA + b) + 16 * lane;
    const int k = off / B_ROW, c = (off % B_ROW) / 16;
    const int nc = c ^ (2 * (k & 3));
    b_src[b] = w + (int64_t)k * NO + min(n0 + 8 * nc, NO - 8);
  }
  const int KT = K / BK;
  // Every step issues the same 7 instructions per wave (past the last K step they re-read it into a
  // buffer that is not read again), so the number of outstanding loads is the same at every wait.
  auto issue = [&](char* base, int t) {
    const int k0 = min(t, KT - 1) * BK;
#pragma unroll
    for (int a = 0; a < A_DMA; ++a)
      __builtin_amdgcn_global_load_lds(a_src[a] + k0, (lds_ptr_t)(base + 1024 * (wave * A_DMA + a)), 16, 0, 0);
#pragma unroll
    for (int b = 0; b < B_DMA; ++b)
      __builtin_amdgcn_global_load_lds(b_src[b] + (int64_t)k0 * NO,
                                       (lds_ptr_t)(base + A_BYTES + 1024 * (wave * B_DMA + b)), 16, 0, 0);
  };

  f32x16 acc[3][4];
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const Roles ro{128 * wm + (lane & 31), lane >> 5, 96 * wn + 16 * ((lane >> 4) & 1) + 4 * (lane & 3),
                 8 * (lane >> 5) + ((lane >> 2) & 3)};

  // Step t (t % STAGES == S) multiplies operands read during step t - 1.  Between its two sub-steps it
  // waits until stage t + 1 has landed in every wave (stage t + 2 may still be in flight), refills the
  // buffer of stage t - 1 (its operands were read two steps ago) with stage t + 3, and reads stage
  // t + 1's operands into the other register set, so their latency overlaps the second sub-step.
  auto step = [&](auto S_const, int t, Ops& cur, Ops& nxt) {
    constexpr int S = decltype(S_const)::value;
    mma(cur, 0, acc);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<DMA_PER_STAGE>();
    __builtin_amdgcn_s_barrier();
    issue(stage_buf<(S + STAGES - 1) % STAGES>(), t + STAGES - 1);
    read_ops(stage_buf<(S + 1) % STAGES>(), ro, nxt);
    __builtin_amdgcn_sched_barrier(0);
    mma(cur, 1, acc);
  };
  const std::integral_constant<int, 0> S0{};
  const std::integral_constant<int, 1> S1{};
  const std::integral_constant<int, 2> S2{};
  const std::integral_constant<int, 3> S3{};

  Ops ops0, ops1;
  issue(stage_buf<0>(), 0);
  issue(stage_buf<1>(), 1);
  issue(stage_buf<2>(), 2);
  wait_vm<2 * DMA_PER_STAGE>();
  __builtin_amdgcn_s_barrier();
  read_ops(stage_buf<0>(), ro, ops0);
  int t = 0;
  for (; t + 3 < KT; t += STAGES) {
    step(S0, t, ops0, ops1);
    step(S1, t + 1, ops1, ops0);
    step(S2, t + 2, ops0, ops1);
    step(S3, t + 3, ops1, ops0);
  }
  if (t < KT) step(S0, t, ops0, ops1);
  if (t + 1 < KT) step(S1, t + 1, ops1, ops0);
  if (t + 2 < KT) step(S2, t + 2, ops0, ops1);
  wait_vm<0>();  // no load into LDS outlives the block
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the last (unused) operand reads have returned

  // Stores, and (k_ssq) per-row sums of squares of the stored bf16 values that fall in the K block
  // [K, 2K) (K = C here).  A 32-column tile lies wholly inside or outside that block (C is a multiple of
  // 32), and v_dot2_f32_bf16 squares the packed pairs being stored; the lane sum (tiles, then
  // quads in order) is combined with the other column half of the wave (lanes l, l + 32) and then with
  // the other wave of the same rows through LDS, always in that order.
  const int nb_k0 = K / BN;
  const bool row_ssq = k_ssq && nb >= nb_k0 && nb <= (2 * K - 1) / BN;
  float ss[4] = {0.f, 0.f, 0.f, 0.f};
  // acc[nt][mt] lane l, register 4q + i: row m = 32 mt + l % 32, column n = 32 nt + 8q + 4(l / 32) + i.
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int m = m0 + 128 * wm + 32 * mt + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int nt = 0; nt < 3; ++nt) {
      const int ntile = n0 + 96 * wn + 32 * nt;
      const bool in_k = row_ssq && ntile >= K && ntile < 2 * K;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = ntile + 8 * q + 4 * (lane >> 5);
        const f32x16& a = acc[nt][mt];
        const uint32_t p0 = cvt_pk_bf16(a[4 * q], a[4 * q + 1]);
        const uint32_t p1 = cvt_pk_bf16(a[4 * q + 2], a[4 * q + 3]);
        if (n < NO) {
          uint32_t* dst = reinterpret_cast<uint32_t*>(y + (int64_t)m * NO + n);
          dst[0] = p0;
          dst[1] = p1;
        }
        if (in_k) ss[mt] = dot2_bf16(p1, p1, dot2_bf16(p0, p0, ss[mt]));
      }
    }
  }
  if (row_ssq) {
    __syncthreads();  // the stage buffers are free
    float* red = reinterpret_cast<float*>(g_stage0);  // [2 column halves of the block][256 rows]
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const float t = ss[mt] + __shfl_xor(ss[mt], 32);
      if (lane < 32) red[wn * BM + 128 * wm + 32 * mt + lane] = t;
    }
    __syncthreads();
    const int m = m0 + tid;
    if (m < M) k_ssq[(int64_t)m * k_parts + (nb - nb_k0)] = red[tid] + red[BM + tid];
  }
}

int qkv_gemm_k_parts(int C) { return (2 * C - 1) / BN - C / BN + 1; }

hipError_t launch_qkv_gemm(const uint16_t* x, const uint16_t* w, uint16_t* qkv, int64_t M, int C, hipStream_t stream,
                           float* k_ssq) {
  const int NO = 3 * C;
  if (C % BK != 0 || M > (1LL << 30)) return hipErrorInvalidValue;
  const int mblocks = (int)((M + BM - 1) / BM), nblocks = (NO + BN - 1) / BN;
  const int slab = mblocks >= 8 ? (mblocks + 7) / 8 : 0;
  const int64_t blocks = slab > 0 ? (int64_t)8 * slab * nblocks : (int64_t)mblocks * nblocks;
  SANA_LAUNCH("qkv_gemm", qkv_gemm_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(
                              x, w, qkv, (int)M, C, NO, mblocks, nblocks, slab, k_ssq, qkv_gemm_k_parts(C)));
  return hipGetLastError();
}

}  // namespace sanala

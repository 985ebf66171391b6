// QKV projection qkv[M, 3C] = x[M, C] @ W[C, 3C] on gfx950 MFMA (bf16 in, fp32 accumulate, bf16 out),
// and its W8A8 form (int8 x and W with per-row and per-column fp32 scales, int32 accumulate, bf16 out).
//
// The projection that the Sana notes (section 7, on-device deployment) fuse with ReLU(K)^T V; here it
// is a separate dense contraction ahead of the attention kernels.  The same notes deploy the model with
// 8-bit weights and activations while keeping the linear attention in full precision.
//
// Block tile 256 (rows of x) x 192 (columns of W), K step 32, 4 waves as 2 x 2, wave tile 128 x 96.
// x arrives K-blocked, [K/32][M][32] (relayout_k32_kernel writes it from row-major x; the Mix-FFN's
// conv kernel writes its output so directly): the 16 rows x 64 bytes that one global->LDS instruction
// stages are then one contiguous 1 KB run instead of 16 pieces of rows 2K bytes apart, which both
// moves tiles faster and keeps the MFMA issue stream from stalling behind the loads.
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
//
// W8A8 (I8): the K step is 64 int8 (the same 64 bytes per x row), W is given transposed, Wt[3C, C]
// (K contiguous per output column), and its tile [192][64 bytes] is staged and read exactly like the x
// tile; v_mfma_i32_32x32x32_i8 takes 16 consecutive k per lane from both operands.  The epilogue
// converts the exact int32 sums to fp32 and scales them by s_x[m] then s_w[n].
#include "common.h"

#include <algorithm>
#include <cstdlib>
#include <type_traits>

namespace sanala {

namespace {
constexpr int BM = 256, BK = 32, STAGES = 4;  // BK in bf16 elements (64 int8 with I8)
constexpr int kThreads = 256;
constexpr int A_ROW = BK * 2;                   // 64 bytes per x tile row
constexpr int A_BYTES = BM * A_ROW;             // 16 KB
constexpr int A_DMA = A_BYTES / 1024 / 4;       // 1-KB wave instructions per wave per stage: 4

// Block width BN = 64 NT: each wave's tile is 128 rows x NT 32-column tiles (NT = 3: 256 x 192 blocks,
// NT = 4: 256 x 256).  The int8 form uses NT = 3.
template <int NT>
struct Geo {
  static_assert(NT == 3 || NT == 4, "block width");
  static constexpr int BN = 64 * NT;
  static constexpr int B_ROW = BN * 2;              // bytes per W tile row (bf16); I8: 192 rows of 64 bytes
  static constexpr int B_BYTES = BK * B_ROW;        // 12 or 16 KB
  static constexpr int B_DMA = B_BYTES / 1024 / 4;  // 3 or 4
  static constexpr int DMA_PER_STAGE = A_DMA + B_DMA;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int OUT_PITCH = NT == 4 ? BN * 2 : BN * 2 + 16;  // row pitch of the epilogue's LDS image
};
constexpr int kStageBytes = Geo<4>::STAGE_BYTES;  // 32 KB per stage buffer
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
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
// Byte offset of W tile element (k, n).  With 512-byte rows (NT = 4) odd rows also flip unit bit 3,
// which puts them 128 bytes along in the bank space as the 384-byte rows of NT = 3 are by themselves.
template <int NT>
__device__ __forceinline__ int w_swz(int k) { return (2 * (k & 3)) ^ (NT == 4 ? 8 * (k & 1) : 0); }
template <int NT>
__device__ __forceinline__ int w_addr(int k, int n) {
  return k * Geo<NT>::B_ROW + 16 * ((n >> 3) ^ w_swz<NT>(k)) + 2 * (n & 7);
}

__shared__ __attribute__((aligned(1024))) char g_stage0[kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_stage1[kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_stage2[kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_stage3[kStageBytes];

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
  int wrow;    // I8: Wt row (output column) of nt = 0 (+ 32 nt)
};

// Operands of one K step (two 16-wide sub-steps) of one wave.
template <int NT>
struct Ops {
  bf16x8 xa[BK / 16][4];
  bf16x8 wb[BK / 16][NT];
};

// Reads a K step's operands from a stage buffer.  The roles are taken by value: read through a
// reference they would be memory accesses of their own, and the compiler could then no longer keep the
// stage reads apart from the loads still landing in the other buffers.
template <bool I8, int NT>
__device__ __forceinline__ void read_ops(const char* __restrict__ As, Roles ro, Ops<NT>& op) {
  const char* __restrict__ Bs = As + A_BYTES;
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      op.xa[s][mt] = as_bf16x8(*reinterpret_cast<const u32x4*>(As + x_addr(ro.xrow + 32 * mt, 2 * s + ro.xhalf)));
    if (I8) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        op.wb[s][nt] = as_bf16x8(*reinterpret_cast<const u32x4*>(Bs + x_addr(ro.wrow + 32 * nt, 2 * s + ro.xhalf)));
      continue;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = ro.wn_col + 32 * nt;
      const int k = 16 * s + ro.wk;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(Bs + w_addr<NT>(k, n)));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(Bs + w_addr<NT>(k + 4, n)));
      const v4s both[2] = {lo, hi};
      op.wb[s][nt] = *reinterpret_cast<const bf16x8*>(both);
    }
  }
}

// Instruction schedule of one K step: after each of its first NV MFMAs the wave issues one
// global->LDS load (7 per step), then after each following MFMA three LDS operand reads while any
// remain (14 or 20 per step), so the MFMA pipe is never left idle while the wave issues memory
// instructions.  The loads come first: a global->LDS load is a write to LDS, and the compiler makes it
// wait for every LDS read still outstanding, which after this step's reads would stall the wave.
template <int I, int NM, int NDS, int NV>
__device__ __forceinline__ void interleave_step() {
  if constexpr (I < NM) {
    constexpr int kDsPer = 3;
    constexpr int ds0 = NDS - (I - NV) * kDsPer, ds = I < NV || ds0 < 0 ? 0 : (ds0 > kDsPer ? kDsPer : ds0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if constexpr (I < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global->LDS load
    if constexpr (ds > 0) __builtin_amdgcn_sched_group_barrier(0x100, ds, 0);  // LDS reads
    interleave_step<I + 1, NM, NDS, NV>();
  }
}

template <int NT, typename Acc>
__device__ __forceinline__ void mma(const Ops<NT>& op, int s, Acc (&acc)[NT][4]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if constexpr (std::is_same_v<Acc, i32x16>)
        acc[nt][mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, op.wb[s][nt]),
                                                            __builtin_bit_cast(i32x4, op.xa[s][mt]), acc[nt][mt], 0, 0, 0);
      else
        acc[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op.wb[s][nt], op.xa[s][mt], acc[nt][mt], 0, 0, 0);
    }
}

// Epilogue image (see the kernel): the piece swizzle of row r, and 16-byte unit c of row r.
template <int NT>
__device__ __forceinline__ int img_swz(int r) {
  return NT == 4 ? ((r & 3) << 3) | ((r >> 2) & 7) : 0;
}
template <int NT>
__device__ __forceinline__ u32x4 img_load16(char* const (&obuf)[4], int r, int c) {
  const char* const row = obuf[r >> 6] + (r & 63) * Geo<NT>::OUT_PITCH;
  if constexpr (NT == 4) {
    const int sw = img_swz<NT>(r);
    const u32x4 v = load16(row + 16 * (c ^ (sw >> 1)));
    return (sw & 1) ? u32x4{v[2], v[3], v[0], v[1]} : v;
  } else {
    return load16(row + 16 * c);
  }
}
}  // namespace

// x: K-blocked, [K/32][M][32] bf16 (I8: [K/64][M][64] int8), 64 bytes per row and K step; w: bf16 [K, NO]
// row-major (I8: int8 Wt, K-blocked: [K/64][NO][64]); s_x [M] and s_w [NO]: I8 only.  y: [M][NO]
// row-major, or with Y_BLK [NO/32][M][32] (NO a multiple of 32), the layout the Mix-FFN's conv reads.
template <bool I8, bool Y_BLK, int NT>
__global__ __launch_bounds__(kThreads) void qkv_gemm_kernel(const void* __restrict__ x, const void* __restrict__ w,
                                                            const float* __restrict__ s_x,
                                                            const float* __restrict__ s_w,
                                                            uint16_t* __restrict__ y, int M, int K, int NO,
                                                            int mblocks, int nblocks, int slab,
                                                            float* __restrict__ k_ssq, int k_parts) {
  static_assert(!I8 || NT == 3, "the int8 form uses 256 x 192 blocks");
  using Acc = std::conditional_t<I8, i32x16, f32x16>;
  constexpr int kElem = I8 ? 1 : 2;  // bytes per x / W element
  const char* const xb = static_cast<const char*>(x);
  const char* const wbp = static_cast<const char*>(w);
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
  const int m0 = mb * BM, n0 = nb * Geo<NT>::BN;

  // Sources of this wave's DMA instructions: a scalar base per K step (block origin + step) plus a
  // per-lane 32-bit offset fixed for the whole loop, so a step spends one vector add per load on
  // addresses.  A instruction i covers rows 16i..16i+15 of the x image, B instruction i bytes
  // [1024i, 1024i + 1024) of the W image (I8: rows 16i..16i+15 of the Wt image, placed like x).  Rows
  // past M and columns past NO read clamped addresses; their products are never stored.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // wave index in an SGPR (LDS destinations)
  // b_off has the largest size for every NT (the first Geo<NT>::B_DMA entries are used): an array whose
  // size depends on NT, captured by the lambdas below, leaves the kernel without a host launch stub.
  uint32_t a_off[A_DMA], b_off[Geo<4>::B_DMA];
#pragma unroll
  for (int a = 0; a < A_DMA; ++a) {
    const int r = 16 * (wave * A_DMA + a) + (lane >> 2);
    const int kc = (lane & 3) ^ xswz(r);
    // x arrives K-blocked (64-byte slabs, slab t holding row m at byte (t*M + m)*64), so the 16 rows of
    // one instruction are one contiguous 1 KB run.
    a_off[a] = (uint32_t)(min(m0 + r, M - 1) - m0) * A_ROW + 16u * kc;
  }
#pragma unroll
  for (int b = 0; b < Geo<NT>::B_DMA; ++b) {
    if (I8) {
      const int r = 16 * (wave * Geo<NT>::B_DMA + b) + (lane >> 2);
      const int kc = (lane & 3) ^ xswz(r);
      b_off[b] = (uint32_t)(min(n0 + r, NO - 1) - n0) * A_ROW + 16u * kc;
    } else {
      const int off = 1024 * (wave * Geo<NT>::B_DMA + b) + 16 * lane;
      const int k = off / Geo<NT>::B_ROW, c = (off % Geo<NT>::B_ROW) / 16;
      const int nc = c ^ w_swz<NT>(k);
      b_off[b] = ((uint32_t)k * NO + (uint32_t)(min(n0 + 8 * nc, NO - 8) - n0)) * 2u;
    }
  }
  const int KT = K * kElem / A_ROW;
  // Every step issues the same 7 instructions per wave (past the last K step they re-read it into a
  // buffer that is not read again), so the number of outstanding loads is the same at every wait.
  auto issue = [&](char* base, int t) {
    const int64_t tt = min(t, KT - 1);
    const char* const a_base = xb + (tt * M + m0) * A_ROW;
    const char* const b_base = I8 ? wbp + (tt * NO + n0) * A_ROW : wbp + (tt * BK * NO + n0) * 2;
#pragma unroll
    for (int a = 0; a < A_DMA; ++a)
      __builtin_amdgcn_global_load_lds(a_base + a_off[a], (lds_ptr_t)(base + 1024 * (wave_s * A_DMA + a)), 16, 0, 0);
#pragma unroll
    for (int b = 0; b < Geo<NT>::B_DMA; ++b)
      __builtin_amdgcn_global_load_lds(b_base + b_off[b], (lds_ptr_t)(base + A_BYTES + 1024 * (wave_s * Geo<NT>::B_DMA + b)), 16,
                                       0, 0);
  };

  Acc acc[NT][4];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  const Roles ro{128 * wm + (lane & 31), lane >> 5, Geo<NT>::BN / 2 * wn + 16 * ((lane >> 4) & 1) + 4 * (lane & 3),
                 8 * (lane >> 5) + ((lane >> 2) & 3), 96 * wn + (lane & 31)};

  // Step t (t % STAGES == S) multiplies operands read during step t - 1.  It first waits until stage
  // t + 1 has landed in every wave (stage t + 2 may still be in flight; the MFMAs of step t - 1 are still
  // executing), then, interleaved with its 24 MFMAs, refills the buffer of stage t - 1 (its operands
  // were read two steps ago) with stage t + 3 and reads stage t + 1's operands into the other register
  // set.
  auto step = [&](auto S_const, int t, Ops<NT>& cur, Ops<NT>& nxt) {
    constexpr int S = decltype(S_const)::value;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this step's operands, read during the last step
    wait_vm<Geo<NT>::DMA_PER_STAGE>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(stage_buf<(S + STAGES - 1) % STAGES>(), t + STAGES - 1);
    read_ops<I8, NT>(stage_buf<(S + 1) % STAGES>(), ro, nxt);
    mma<NT>(cur, 0, acc);
    mma<NT>(cur, 1, acc);
    interleave_step<0, 8 * NT, I8 ? 14 : 8 + 4 * NT, Geo<NT>::DMA_PER_STAGE>();
    __builtin_amdgcn_sched_barrier(0);
  };
  const std::integral_constant<int, 0> S0{};
  const std::integral_constant<int, 1> S1{};
  const std::integral_constant<int, 2> S2{};
  const std::integral_constant<int, 3> S3{};

  Ops<NT> ops0, ops1;
  issue(stage_buf<0>(), 0);
  issue(stage_buf<1>(), 1);
  issue(stage_buf<2>(), 2);
  wait_vm<2 * Geo<NT>::DMA_PER_STAGE>();
  __builtin_amdgcn_s_barrier();
  read_ops<I8, NT>(stage_buf<0>(), ro, ops0);
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

  // The output tile goes through LDS so that its global stores are whole runs: each wave first writes
  // its accumulators as bf16 (I8: after the scaling by s_x[m] and s_w[n]) into a [256][BN] image held
  // in the stage buffers (rows 64g..64g+63 in buffer g), then the block stores the image 16 bytes per
  // lane: whole row runs for row-major y, 1 KB runs (16 rows x 64 bytes of one 32-column chunk) for the
  // chunk-major layout.  NT = 3: 400-byte row pitch.  NT = 4: the 512-byte rows fill the buffers, so
  // instead of padding, 8-byte piece g of row r sits at piece g ^ swz(r), swz a permutation of the
  // 32 rows a wave writes at once (those writes then hit 32 different bank pairs, and the 4 rows x 4
  // pieces of 16 bytes that 16 lanes read for the chunk-major layout 16 different bank quads).  With
  // k_ssq, the per-row sums of squares of the stored
  // bf16 values that fall in the K block [K, 2K) (K = C here) are formed on the way: a 32-column tile
  // lies wholly inside or outside that block (C is a multiple of 32), and v_dot2_f32_bf16 squares the
  // packed pairs; the lane sum (tiles, then quads in order) is combined with the other column half of
  // the wave (lanes l, l + 32) and then with the other wave of the same rows through LDS, always in that
  // order.
  char* const obuf[4] = {stage_buf<0>(), stage_buf<1>(), stage_buf<2>(), stage_buf<3>()};
  __syncthreads();  // every wave has read its last operands: the stage buffers are free
  const int nb_k0 = K / Geo<NT>::BN;
  const bool row_ssq = k_ssq && nb >= nb_k0 && nb <= (2 * K - 1) / Geo<NT>::BN;
  float ss[4] = {0.f, 0.f, 0.f, 0.f};
  // acc[nt][mt] lane l, register 4q + i: row m = 32 mt + l % 32, column n = 32 nt + 8q + 4(l / 32) + i.
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int rl = 128 * wm + 32 * mt + (lane & 31);  // row within the tile
    const int m = m0 + rl;
    const float sxm = I8 ? s_x[min(m, M - 1)] : 1.f;
    char* const orow = obuf[rl >> 6] + (rl & 63) * Geo<NT>::OUT_PITCH;
    const int rsw = img_swz<NT>(rl);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int cl0 = Geo<NT>::BN / 2 * wn + 32 * nt;
      const bool in_k = row_ssq && m < M && n0 + cl0 >= K && n0 + cl0 < 2 * K;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cl = cl0 + 8 * q + 4 * (lane >> 5);
        float v4[4];
        if constexpr (I8) {
          const int n = n0 + cl;
          const f32x4 sw = n < NO ? loadf4(s_w + n) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < 4; ++i) v4[i] = ((float)acc[nt][mt][4 * q + i] * sxm) * sw[i];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) v4[i] = acc[nt][mt][4 * q + i];
        }
        const uint32_t p0 = cvt_pk_bf16(v4[0], v4[1]);
        const uint32_t p1 = cvt_pk_bf16(v4[2], v4[3]);
        *reinterpret_cast<uint2*>(orow + 8 * ((cl >> 2) ^ rsw)) = make_uint2(p0, p1);
        if (in_k) ss[mt] = dot2_bf16(p1, p1, dot2_bf16(p0, p0, ss[mt]));
      }
    }
  }
  __syncthreads();
  const int rows = min(BM, M - m0), cols = min(Geo<NT>::BN, NO - n0);  // cols: a multiple of 8
  if constexpr (Y_BLK) {
    // Chunk j of the tile: rows x 64 bytes, consecutive in y.  Non-temporal: the Mix-FFN's expanded
    // activations (367 MB on the 2K grid) exceed the Infinity Cache and are read once, by the conv
    // (Mix-FFN call 1208.0 -> 1203.9 us on MI355X, bitwise-equal output).
    for (int i = tid; i < (Geo<NT>::BN / 32) * BM * 4; i += kThreads) {
      const int j = i / (BM * 4), r = (i / 4) % BM, w = i & 3;
      if (r < rows && 32 * j < cols)
        store16_nt(y + ((((int64_t)(n0 >> 5) + j) * M + m0 + r) << 5) + 8 * w, img_load16<NT>(obuf, r, 4 * j + w));
    }
  } else {
    for (int i = tid; i < BM * (Geo<NT>::BN / 8); i += kThreads) {
      const int r = i / (Geo<NT>::BN / 8), c = i % (Geo<NT>::BN / 8);
      if (r < rows && 8 * c < cols)
        store16(y + (int64_t)(m0 + r) * NO + n0 + 8 * c, img_load16<NT>(obuf, r, c));
    }
  }
  if (row_ssq) {
    __syncthreads();  // the image has been stored: stage buffer 0 is free
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

// The per-lane DMA offsets are 32-bit: at most 255 rows x K x 2 bytes (x) and 32 x NO x 2 bytes (W).
constexpr int kMaxK = 1 << 20, kMaxNO = 1 << 24;

// Block width per shape.  A 256-column block costs about 4% less per output column than a 192-column
// one (2K shapes on MI355X: QKV projection 427.5 against 432 us, Mix-FFN expansion 675 against 713 us),
// but the two widths fill the CUs in different numbers of rounds (the Mix-FFN projection, 2240 columns:
// 576 blocks of 256, 2.25 rounds, 382 us, against 768 of 192, 3 full rounds, 335 us).  The width with
// the smaller ceil(blocks / CUs) x width, the 256 one weighted by 0.96, is taken; SANA_GEMM_WIDE=0 or 1
// forces 192 or 256.
bool gemm_wide(int64_t M, int NO) {
  const char* e = std::getenv("SANA_GEMM_WIDE");
  if (e && (e[0] == '0' || e[0] == '1') && e[1] == 0) return e[0] == '1';
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const int64_t mblocks = (M + BM - 1) / BM;
  const int64_t mpad = mblocks >= 8 ? (mblocks + 7) / 8 * 8 : mblocks;  // the XCD-ordered grid's rows
  auto cost = [&](int bn, double per_col) {
    const int64_t blocks = mpad * ((NO + bn - 1) / bn);
    return (double)((blocks + cus - 1) / cus) * bn * per_col;
  };
  return cost(Geo<4>::BN, 0.96) < cost(Geo<3>::BN, 1.0);
}

int qkv_gemm_k_parts(int C, bool wide) {
  const int BN = wide ? Geo<4>::BN : Geo<3>::BN;
  return (2 * C - 1) / BN - C / BN + 1;
}

// Per-row symmetric int8 quantisation of bf16 x [M, C] (the dynamic activation half of W8A8): with
// a = max_c |x[m, c]|, q = clamp(rne(x * (127 / a)), -127, 127) and s_x[m] = a / 127, every step in
// fp32 with correctly rounded division (a = 0 gives q = 0 and s_x = 0).  One wave per row, 16-byte
// loads; rows of up to 64 * kQuantRegUnits units stay in registers between the two passes, longer
// rows are read a second time.
constexpr int kQuantRegUnits = 8;

__device__ __forceinline__ float bf16_abs_max(u32x4 w, float m) {
#pragma unroll
  for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  return m;
}

__device__ __forceinline__ uint2 quant_unit(u32x4 w, float inv) {
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
    const float qf = fminf(fmaxf(rintf(v * inv), -127.f), 127.f);
    packed[i >> 2] |= ((uint32_t)(int)qf & 0xffu) << (8 * (i & 3));
  }
  return make_uint2(packed[0], packed[1]);
}

// BLOCKED: codes stored K-blocked for the int8 GEMM, [C/64][M][64] (the 8 codes of unit u of row m at
// byte ((8u / 64) * M + m) * 64 + 8u % 64); else row-major [M][C].
template <bool BLOCKED>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t M, int C,
                                                         int8_t* __restrict__ xq, float* __restrict__ s_x) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const uint16_t* xr = x + row * C;
  const int units = C / 8;  // 16-byte units of the row
  auto dst = [&](int u) -> uint2* {
    return reinterpret_cast<uint2*>(BLOCKED ? xq + ((int64_t)(u >> 3) * M + row) * 64 + 8 * (u & 7)
                                            : xq + row * C + 8 * u);
  };
  float amax = 0.f;
  if (units <= 64 * kQuantRegUnits) {
    u32x4 w[kQuantRegUnits];
#pragma unroll
    for (int j = 0; j < kQuantRegUnits; ++j) {
      const int u = lane + 64 * j;
      w[j] = u < units ? load16(xr + 8 * u) : u32x4{0u, 0u, 0u, 0u};
      amax = bf16_abs_max(w[j], amax);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float inv = amax > 0.f ? 127.f / amax : 0.f;
#pragma unroll
    for (int j = 0; j < kQuantRegUnits; ++j) {
      const int u = lane + 64 * j;
      if (u < units) *dst(u) = quant_unit(w[j], inv);
    }
  } else {
    for (int u = lane; u < units; u += 64) amax = bf16_abs_max(load16(xr + 8 * u), amax);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float inv = amax > 0.f ? 127.f / amax : 0.f;
    for (int u = lane; u < units; u += 64) *dst(u) = quant_unit(load16(xr + 8 * u), inv);
  }
  if (lane == 0) s_x[row] = amax / 127.f;
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t M, int C, int8_t* xq, float* s_x, hipStream_t stream,
                             bool k_blocked) {
  if (C % 8 != 0 || (k_blocked && C % 64 != 0)) return hipErrorInvalidValue;
  if (k_blocked)
    launch_kernel("quant_rows", quant_rows_kernel<true>, (unsigned)((M + 3) / 4), 256, 0, stream, x, M, C, xq, s_x);
  else
    launch_kernel("quant_rows", quant_rows_kernel<false>, (unsigned)((M + 3) / 4), 256, 0, stream, x, M, C, xq, s_x);
  return hipGetLastError();
}

// x [M][K] bf16 row-major -> xb [K/32][M][32] (the GEMM's x layout; K a multiple of 32).  Wave w of
// block (bx, by) moves rows 64 bx + 16 w + l/4 (lane l) of the 32-column groups [8 by, 8 by + 8): the
// 16-byte unit l % 4 of each group.  Its eight loads are issued before its stores, and each store
// instruction writes one contiguous 1 KB run (16 rows x 64 bytes).
__global__ __launch_bounds__(256) void relayout_k32_kernel(const uint16_t* __restrict__ x, int64_t M, int K,
                                                           uint16_t* __restrict__ xb) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 64 + 16 * wave + (lane >> 2);
  const int G = K / 32, g0 = (int)blockIdx.y * 8;
  if (m >= M) return;
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (g0 + i < G) v[i] = load16(x + m * K + (g0 + i) * 32 + 8 * (lane & 3));
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (g0 + i < G) store16(xb + ((int64_t)(g0 + i) * M + m) * 32 + 8 * (lane & 3), v[i]);
}

hipError_t launch_relayout_k32(const uint16_t* x, int64_t M, int K, uint16_t* xb, hipStream_t stream) {
  if (K % 32 != 0 || M > (1LL << 30) || K / 256 >= 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((M + 63) / 64), (unsigned)((K / 32 + 7) / 8));
  launch_kernel("relayout_x", relayout_k32_kernel, grid, 256, 0, stream, x, M, K, xb);
  return hipGetLastError();
}

// One thread per 16-byte unit u of row n: src[n][16u..16u+15] -> dst[u/4][n][16(u%4)..].
__global__ __launch_bounds__(256) void pack_k64_kernel(const int8_t* __restrict__ src, int64_t rows, int C,
                                                       int8_t* __restrict__ dst) {
  const int upr = C / 16;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * upr) return;
  const int64_t n = i / upr;
  const int u = (int)(i - n * upr);
  *reinterpret_cast<u32x4*>(dst + ((int64_t)(u >> 2) * rows + n) * 64 + 16 * (u & 3)) =
      *reinterpret_cast<const u32x4*>(src + n * C + 16 * u);
}

hipError_t launch_pack_k64(const int8_t* src, int64_t rows, int C, int8_t* dst, hipStream_t stream) {
  if (C % 64 != 0) return hipErrorInvalidValue;
  const int64_t units = rows * (C / 16);
  launch_kernel("pack_k64", pack_k64_kernel, (unsigned)((units + 255) / 256), 256, 0, stream, src, rows, C, dst);
  return hipGetLastError();
}

namespace {
typedef void (*GemmKernel)(const void*, const void*, const float*, const float*, uint16_t*, int, int, int, int, int,
                           int, float*, int);

// The kernel is named by the (non-template) caller, which makes the compiler emit its launch stub.
void launch_gemm(GemmKernel kernel, int bn, const char* label, const void* x, const void* w, const float* s_x,
                 const float* s_w, uint16_t* y, int64_t M, int K, int NO, hipStream_t stream, float* k_ssq,
                 int k_parts) {
  const int mblocks = (int)((M + BM - 1) / BM), nblocks = (NO + bn - 1) / bn;
  const int slab = mblocks >= 8 ? (mblocks + 7) / 8 : 0;
  const int64_t blocks = slab > 0 ? (int64_t)8 * slab * nblocks : (int64_t)mblocks * nblocks;
  launch_kernel(label, kernel, (unsigned)blocks, kThreads, 0, stream, x, w, s_x, s_w, y, (int)M, K, NO, mblocks,
                nblocks, slab, k_ssq, k_parts);
}
}  // namespace

hipError_t launch_qkv_gemm(const uint16_t* xb, const uint16_t* w, uint16_t* qkv, int64_t M, int C,
                           hipStream_t stream, float* k_ssq) {
  const int NO = 3 * C;
  if (C % BK != 0 || M > (1LL << 30) || C > kMaxK) return hipErrorInvalidValue;
  const bool wide = gemm_wide(M, NO);
  launch_gemm(wide ? qkv_gemm_kernel<false, false, 4> : qkv_gemm_kernel<false, false, 3>,
              wide ? Geo<4>::BN : Geo<3>::BN, "qkv_gemm", xb, w, nullptr, nullptr, qkv, M, C, NO, stream, k_ssq,
              qkv_gemm_k_parts(C, wide));
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const uint16_t* xb, const uint16_t* w, uint16_t* y, int64_t M, int K, int NO,
                            hipStream_t stream, const char* label, bool y_blocked) {
  if (K % BK != 0 || NO % 8 != 0 || M > (1LL << 30) || K > kMaxK || NO > kMaxNO) return hipErrorInvalidValue;
  if (y_blocked && NO % 32 != 0) return hipErrorInvalidValue;
  const bool wide = gemm_wide(M, NO);
  const GemmKernel kernel = y_blocked ? (wide ? qkv_gemm_kernel<false, true, 4> : qkv_gemm_kernel<false, true, 3>)
                                      : (wide ? qkv_gemm_kernel<false, false, 4> : qkv_gemm_kernel<false, false, 3>);
  launch_gemm(kernel, wide ? Geo<4>::BN : Geo<3>::BN, label, xb, w, nullptr, nullptr, y, M, K, NO, stream, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_qkv_gemm_i8(const int8_t* xq, const int8_t* wt, const float* s_x, const float* s_w, uint16_t* qkv,
                              int64_t M, int C, hipStream_t stream, float* k_ssq) {
  const int NO = 3 * C;
  if (C % (2 * BK) != 0 || M > (1LL << 30) || C > kMaxK) return hipErrorInvalidValue;
  launch_gemm(qkv_gemm_kernel<true, false, 3>, Geo<3>::BN, "qkv_gemm_i8", xq, wt, s_x, s_w, qkv, M, C, NO, stream,
              k_ssq, qkv_gemm_k_parts(C, false));
  return hipGetLastError();
}

}  // namespace sanala

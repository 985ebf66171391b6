// bf16-storage path of the linear attention on gfx950 (fp32 accumulation, bf16 MFMA operands).
//
// "Sana: Efficient High-Resolution Image Synthesis with Linear Diffusion Transformers" (paper notes),
// section 2.1, Eq. (1), per head, in the precompute-then-apply order the notes give after Eq. (1);
// phi(x) = ReLU(x * r * g), r = 1/sqrt(mean_c x_c^2 + eps) over all channels of a token ("SANA 1.5:
// Efficient Scaling of Training-Time and Inference-Time Compute in Linear Diffusion Transformer"
// (research notes), model architecture, QK Norm).
//
// Algebra used to keep per-element work small (exact up to rounding):
//   r > 0, so ReLU(x * r * g) = r * |g| * ReLU(s * x) with s = sign(g); ReLU(s * x) of a bf16 x is
//   exact in bf16 (a sign flip and a packed integer max).  Hence, with G_d = |gq_d| * |gk_d|,
//     S[d][e] * |gq_d| = G_d * sum_j r_k,j ReLU(sk_d k_j,d) v_j,e         (S' below)
//     z[d] * |gq_d|    = G_d * sum_j r_k,j ReLU(sk_d k_j,d)                (z' below)
//     O_i[e] = r_q,i a / (r_q,i b + eps) = a / (b + eps / r_q,i),
//   a = sum_d ReLU(sq_d q_i,d) S'[d][e],  b = sum_d ReLU(sq_d q_i,d) z'[d].
//   The query side therefore needs no fp32 multiply per element, and r_q enters once per token.
//
// Launches on one stream:
//   rowstats  r_k for every K row (one wave per 2240-channel row)
//   kv_state  per (b, head pair, token chunk): S~ = sum_j (r_k,j ReLU(sk k_j)) v_j^T and
//             z~ = sum_j r_k,j ReLU(sk k_j) on v_mfma_f32_32x32x16_bf16 (phi(K) rounded to bf16 once,
//             fp32 accumulation; z~ from a second MFMA against a ones operand)
//   kv_reduce sums the chunk partials in chunk order (deterministic, no float atomics) and writes
//             S' as bf16 A operands of v_mfma_f32_16x16x32_bf16 and z' as a bf16 hi + lo pair
//             (skipped when one chunk covers the sequence: kv_state then writes them itself)
//   out       persistent blocks hold S', z' and the query sign masks of the current sample in LDS
//             and stream 16-token tiles of Q (two tiles' loads in flight): r_q from the Q rows
//             held in registers (v_dot2_f32_bf16), a on MFMA, b by v_dot2_f32_bf16.
#include "rowstats.h"
#include "state_ops.h"

#include <algorithm>

namespace sanala {

// ---------------------------------------------------------------------------------------------
// KV state of one chunk.  The block (4 waves) forms the state of heads 2p, 2p+1 over tokens
// [c*Tc, min(N, c*Tc+Tc)) of sample b, staged through LDS in 64-token sub-blocks; the next
// sub-block's global loads are in flight while the current one is multiplied.  Wave w: head 2p + (w & 1),
// token half (w >> 1) of each sub-block.  MFMA 32x32x16: A[d][t] = bf16(r_t ReLU(s_d k_t,d)) (lane
// d + 32g holds tokens 8g..8g+7 of the 16-token step), B[t][e] = v_t,e; accumulator lane l, register
// r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32.  A second MFMA against an all-ones B gives z~ in
// every column.  On return (after a barrier) fin holds, per head, S~[d][e] then z~[d] (kPartStride
// floats), the two token halves added in a fixed order.
// ---------------------------------------------------------------------------------------------
constexpr int kStateSB = 64;     // tokens per sub-block
constexpr int kStatePitch = 72;  // bf16 per staged row (64 used)

template <bool NORM, bool F16, bool NTV = false>
__device__ __forceinline__ void chunk_state(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t ld,
                                            const float* __restrict__ r_k, const float* __restrict__ gk, int N, int H,
                                            int b, int p, int c, int Tc, uint16_t* Ks, uint16_t* Vs, float* rs,
                                            float* fin) {
  constexpr int SB = kStateSB, PITCH = kStatePitch;
  const int h0 = 2 * p;
  const int nh = min(2, H - h0);
  const int n_begin = c * Tc;
  const int n_end = min(N, n_begin + Tc);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int hh = w & 1, th = w >> 1;
  const int d = lane & 31, grp = lane >> 5;
  const int hcol = min(h0 + hh, H - 1) * kHeadDim + d;
  const uint32_t sgn = (NORM && gk[hcol] < 0.f) ? 0x80008000u : 0u;  // flips both tokens of a pair
  const int64_t row0 = (int64_t)b * N;
  constexpr uint32_t kOne2 = F16 ? 0x3c003c00u : 0x3f803f80u;  // two 1.0 values
  const u32x4 ones = {kOne2, kOne2, kOne2, kOne2};

  u32x4 pk[2], pv[2];
  float pr = 1.f;
  auto gload = [&](int n0) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int i = tid + it * 256;
      const int row = i >> 3, cu = i & 7;  // cu: 16-byte unit of the 128-byte head pair
      const int n = n0 + row;
      pk[it] = u32x4{0u, 0u, 0u, 0u};
      pv[it] = u32x4{0u, 0u, 0u, 0u};
      if (n < n_end && (cu >> 2) < nh) {
        const int64_t off = (row0 + n) * ld + h0 * kHeadDim + cu * 8;
        if constexpr (NTV)
          pk[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off));
        else
          pk[it] = load16(k + off);
        if constexpr (NTV)
          pv[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off));
        else
          pv[it] = load16(v + off);
      }
    }
    if (tid < SB) pr = (NORM && n0 + tid < n_end) ? r_k[row0 + n0 + tid] : 1.0f;  // rows past the end are zero
  };

  f32x16 acc, accz;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc[r] = 0.f;
    accz[r] = 0.f;
  }

  if (n_begin < n_end) gload(n_begin);
  for (int n0 = n_begin; n0 < n_end; n0 += SB) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int i = tid + it * 256;
      const int row = i >> 3, cu = i & 7;
      store16(&Ks[row * PITCH + cu * 8], pk[it]);
      store16(&Vs[row * PITCH + cu * 8], pv[it]);
    }
    if (tid < SB) rs[tid] = pr;
    __syncthreads();
    if (n0 + SB < n_end) gload(n0 + SB);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int tb = 32 * th + 16 * s + 8 * grp;  // this lane's tokens tb .. tb+7
      const int col = hh * kHeadDim + d;
      uint32_t aw[4], bw[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t0 = tb + 2 * u;
        const uint32_t kp = (uint32_t)Ks[t0 * PITCH + col] | ((uint32_t)Ks[(t0 + 1) * PITCH + col] << 16);
        bw[u] = (uint32_t)Vs[t0 * PITCH + col] | ((uint32_t)Vs[(t0 + 1) * PITCH + col] << 16);
        aw[u] = relu_bf16x2(kp ^ sgn);
      }
      if (NORM) {
        const f32x4 r0 = *reinterpret_cast<const f32x4*>(&rs[tb]);
        const f32x4 r1 = *reinterpret_cast<const f32x4*>(&rs[tb + 4]);
        const float rr[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          aw[u] = cvt_pk_h<F16>(h_lo<F16>(aw[u]) * rr[2 * u], h_hi<F16>(aw[u]) * rr[2 * u + 1]);
      }
      const u32x4 A = {aw[0], aw[1], aw[2], aw[3]};
      const u32x4 Bv = {bw[0], bw[1], bw[2], bw[3]};
      if constexpr (F16) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(A), as_f16x8(Bv), acc, 0, 0, 0);
        accz = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(A), as_f16x8(ones), accz, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(A), as_bf16x8(Bv), acc, 0, 0, 0);
        accz = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(A), as_bf16x8(ones), accz, 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // Combine the two token halves of each head in a fixed order (wave hh + 2 hands over to wave hh).
  float* fh = fin + hh * kPartStride;
  if (th == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * grp + (r & 3);
      fh[row * kHeadDim + d] = acc[r];
      if (d == 0) fh[kHeadDim * kHeadDim + row] = accz[r];
    }
  }
  __syncthreads();
  if (th == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * grp + (r & 3);
      fh[row * kHeadDim + d] = acc[r] + fh[row * kHeadDim + d];
      if (d == 0) fh[kHeadDim * kHeadDim + row] = accz[r] + fh[kHeadDim * kHeadDim + row];
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------------------------
// Chunk rendezvous (a split sequence whose state blocks are all resident at once).  Block (c, p, b)
// stores its chunk partial with device-scope stores, waits for them to complete and sets its flag to
// the call's tag; it then waits, up to a time limit, for the flags of the pair's other chunks, and sums
// slice c of the pair's state over all chunks in chunk order (one round of loads), writing that slice
// of the output kernel's operands.  So the NC blocks of a pair share the reduction that would otherwise
// be a launch of its own.  A chunk whose flag has not appeared by the limit (its block not resident
// yet, say) is formed by the waiting block itself with the same code, so the bits do not depend on the
// route and no wait can hang.  The flags carry the call's tag (never 0), so they need no clearing.
// No fence is used: an agent-scope fence writes back and invalidates the whole L2 of the XCD, which
// made the state pass six times slower on MI355X while other blocks streamed K and V through that L2.
// ---------------------------------------------------------------------------------------------
constexpr int kMaxRendezvousChunks = 16;

// Stores the block's partial of heads h0 .. h0+nh-1 (fin: kPartStride floats per head) as chunk c of
// NC, device-scope 16-byte stores; then, once every thread's stores have completed, sets the flag.
__device__ __forceinline__ void publish_partial(float* __restrict__ part, const float* fin, int NC, int c, int64_t bh0,
                                                int nh, uint32_t* flag, uint32_t epoch) {
  constexpr int Q4 = kPartStride / 4;
  for (int hl = 0; hl < nh; ++hl) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(part + ((bh0 + hl) * NC + c) * kPartStride, kPartStride * 4);
    for (int j = threadIdx.x; j < Q4; j += blockDim.x)
      buffer_store16_dev(r, (uint32_t)(j * 16), *reinterpret_cast<const u32x4*>(fin + hl * kPartStride + 4 * j));
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0 polls the NC (<= 64) flags until all carry the tag or `spin` ticks of the 100 MHz clock have
// passed; every thread gets the mask of chunks still missing.
__device__ __forceinline__ uint64_t wait_flags(const uint32_t* flags, int NC, uint32_t epoch, uint32_t spin) {
  __shared__ uint64_t missing_s;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const uint64_t want = NC >= 64 ? ~0ull : ((1ull << NC) - 1ull);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    uint64_t ready;
    for (;;) {
      const uint32_t f =
          lane < NC ? __hip_atomic_load(const_cast<uint32_t*>(flags) + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                    : 0u;
      ready = __ballot(f == epoch) & want;
      if (ready == want || __builtin_amdgcn_s_memrealtime() - t0 >= spin) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (lane == 0) missing_s = want & ~ready;
  }
  __syncthreads();
  return missing_s;
}

// Slice c of the pair's summed state (16-byte column groups [c*per, (c+1)*per) of the nh*kPartStride
// floats), summed over the NC chunks in chunk order, then written as operands.  Chunks in `missing` are
// formed here (chunk_state into fin) instead of being loaded.
template <bool NORM, bool F16>
__device__ __forceinline__ void reduce_slice(const float* __restrict__ part, uint64_t missing, int NC, int c, int64_t bh0,
                                             int h0, int nh, const uint16_t* __restrict__ k,
                                             const uint16_t* __restrict__ v, int64_t ld, const float* __restrict__ r_k,
                                             const float* __restrict__ gq, const float* __restrict__ gk, int N, int H,
                                             int b, int p, int Tc, uint16_t* Ks, uint16_t* Vs, float* rs, float* fin,
                                             f32x4* accs, uint16_t* __restrict__ Sop, uint16_t* __restrict__ zop) {
  constexpr int Q4 = kPartStride / 4;
  const int cols = nh * Q4;
  const int per = (cols + NC - 1) / NC;
  const int j0 = c * per, j1 = min(cols, j0 + per);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(part + bh0 * NC * kPartStride, (uint32_t)(nh * NC * kPartStride * 4));
  auto emit4 = [&](int j, f32x4 s) {
    const int hl = j / Q4, off = 4 * (j - hl * Q4);
#pragma unroll
    for (int e = 0; e < 4; ++e) emit_state<NORM>(bh0 + hl, h0 + hl, off + e, s[e], gq, gk, Sop, zop);
  };
  auto src_off = [&](int j, int u) {  // byte offset of column group j of chunk u
    const int hl = j / Q4;
    return (uint32_t)(((hl * NC + u) * kPartStride + 4 * (j - hl * Q4)) * 4);
  };
  if (missing == 0) {
    for (int j = j0 + (int)threadIdx.x; j < j1; j += blockDim.x) {
      f32x4 x[kMaxRendezvousChunks];
#pragma unroll
      for (int u = 0; u < kMaxRendezvousChunks; ++u)
        x[u] = as_f32x4(buffer_load16_dev(r, u < NC ? src_off(j, u) : kOutOfRange));
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < kMaxRendezvousChunks; ++u)
        if (u < NC) {
          s[0] += x[u][0];
          s[1] += x[u][1];
          s[2] += x[u][2];
          s[3] += x[u][3];
        }
      emit4(j, s);
    }
    return;
  }
  // Some partial is missing: the same sums, chunk by chunk, accumulated in LDS (each thread its own
  // column groups), with the missing chunks formed by this block.
  for (int j = j0 + (int)threadIdx.x; j < j1; j += blockDim.x) accs[j - j0] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int u = 0; u < NC; ++u) {
    if ((missing >> u) & 1ull) {
      chunk_state<NORM, F16>(k, v, ld, r_k, gk, N, H, b, p, u, Tc, Ks, Vs, rs, fin);
      for (int j = j0 + (int)threadIdx.x; j < j1; j += blockDim.x) {
        const int hl = j / Q4;
        accs[j - j0] += *reinterpret_cast<const f32x4*>(fin + hl * kPartStride + 4 * (j - hl * Q4));
      }
      __syncthreads();  // fin is reused by the next chunk formed here
    } else {
      for (int j = j0 + (int)threadIdx.x; j < j1; j += blockDim.x)
        accs[j - j0] += as_f32x4(buffer_load16_dev(r, src_off(j, u)));
    }
  }
  for (int j = j0 + (int)threadIdx.x; j < j1; j += blockDim.x) emit4(j, accs[j - j0]);
}

// ---------------------------------------------------------------------------------------------
// KV state pass.  Block (c, p, b): chunk c of heads 2p, 2p+1 of sample b (chunk_state).  One chunk per
// sequence: the block writes the operands itself.  Several: with flags set, the chunk rendezvous above;
// otherwise the block writes its partial for kv_reduce_bf16.
// ---------------------------------------------------------------------------------------------
template <bool NORM, bool F16, bool NTV = false>
__global__ __launch_bounds__(256, 5) void kv_state_bf16(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                     int64_t ld, const float* __restrict__ r_k,
                                                     const float* __restrict__ gq, const float* __restrict__ gk,
                                                     int N, int H, int Tc, int NC, float* __restrict__ part,
                                                     uint16_t* __restrict__ Sop, uint16_t* __restrict__ zop,
                                                     uint32_t* __restrict__ gsg, uint32_t* __restrict__ flags,
                                                     uint32_t epoch, uint32_t spin) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kStateSB * kStatePitch];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kStateSB * kStatePitch];
  __shared__ __attribute__((aligned(16))) float rs[kStateSB];
  __shared__ __attribute__((aligned(16))) float fin[2 * kPartStride];  // wave hand-over, then the block's state

  const int c = blockIdx.x, p = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  chunk_state<NORM, F16, NTV>(k, v, ld, r_k, gk, N, H, b, p, c, Tc, Ks, Vs, rs, fin);
  const int h0 = 2 * p;
  const int nh = min(2, H - h0);
  const int64_t bh0 = (int64_t)b * H + h0;
  if ((NC == 1 || (flags != nullptr && c == 0)) && b == 0 && tid < nh * kSgnPerHead) {
    const int h = h0 + tid / kSgnPerHead, i = tid % kSgnPerHead;
    gsg[h * kSgnPerHead + i] = sign_word<NORM>(gq, h, i / 4, i & 3);
  }
  if (NC == 1) {
    for (int i = tid; i < nh * kPartStride; i += 256) {
      const int hl = i / kPartStride, off = i - hl * kPartStride;
      emit_state<NORM>(bh0 + hl, h0 + hl, off, fin[i], gq, gk, Sop, zop);
    }
    return;
  }
  if (flags == nullptr) {
    for (int i = tid; i < nh * kPartStride; i += 256) {
      const int hl = i / kPartStride, off = i - hl * kPartStride;
      part[((bh0 + hl) * NC + c) * kPartStride + off] = fin[i];
    }
    return;
  }
  __shared__ f32x4 accs[(2 * kPartStride / 4 + 1) / 2];  // slow route of the rendezvous (NC >= 2)
  uint32_t* pf = flags + ((int64_t)b * gridDim.y + p) * NC;
  publish_partial(part, fin, NC, c, bh0, nh, pf + c, epoch);
  const uint64_t missing = wait_flags(pf, NC, epoch, spin);
  reduce_slice<NORM, F16>(part, missing, NC, c, bh0, h0, nh, k, v, ld, r_k, gq, gk, N, H, b, p, Tc, Ks, Vs, rs, fin,
                          accs, Sop, zop);
}

// r[row] = 1 / sqrt(sum_j part[row * nparts + j] / C + eps): the QK-Norm scale from per-row partial
// sums of squares over column panels (summed in panel order), one thread per row.
__global__ __launch_bounds__(256) void rowfinish_kernel(const float* __restrict__ part, int nparts, int64_t rows,
                                                        float inv_C, float eps, float* __restrict__ r) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const float* p = part + row * nparts;
  float ss = 0.f;
  for (int j = 0; j < nparts; ++j) ss += p[j];
  r[row] = 1.0f / sqrtf(ss * inv_C + eps);
}

// One thread per state element (b, h, i): sum of the chunk partials in chunk order (8 loads in flight
// per step), then the output kernel's operands.
template <bool NORM>
__global__ __launch_bounds__(256) void kv_reduce_bf16(const float* __restrict__ part, int NC, int H, int64_t BH,
                                                      const float* __restrict__ gq, const float* __restrict__ gk,
                                                      uint16_t* __restrict__ Sop, uint16_t* __restrict__ zop,
                                                      uint32_t* __restrict__ gsg) {
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gi < (int64_t)H * kSgnPerHead)
    gsg[gi] = sign_word<NORM>(gq, (int)(gi / kSgnPerHead), (int)(gi / 4) & 3, (int)gi & 3);
  if (gi >= BH * kPartStride) return;
  const int64_t bh = gi / kPartStride;
  const int i = (int)(gi - bh * kPartStride);
  const float* src = part + bh * NC * kPartStride + i;
  // All loads of a batch are issued before the in-order sum.
  float s = 0.f;
  for (int c = 0; c < NC; c += 32) {
    float x[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) x[u] = c + u < NC ? src[(int64_t)(c + u) * kPartStride] : 0.f;
#pragma unroll
    for (int u = 0; u < 32; ++u)
      if (c + u < NC) s += x[u];
  }
  emit_state<NORM>(bh, (int)(bh % H), i, s, gq, gk, Sop, zop);
}

// ---------------------------------------------------------------------------------------------
// Per-head output math shared by both output kernels.  qv: lane l = t + 16*kg holds query dims
// 8kg..8kg+7 of token t (bf16 pairs); sg: the sign masks of those dims; a0/a1: the two e-blocks of
// S'^T; zh/zl: z' hi and lo at those dims; epsr = eps / r_q of token t; even_row: lane index even.
// Returns output channels 8kg..8kg+7 of token t as bf16 (1/den by v_rcp_f32, 1 ulp).
// ---------------------------------------------------------------------------------------------
template <bool F16>
__device__ __forceinline__ u32x4 head_out(u32x4 qv, u32x4 sg, bf16x8 a0, bf16x8 a1, u32x4 zh, u32x4 zl, float epsr,
                                          bool even_row, float* den = nullptr) {
  u32x4 psi;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    psi[u] = relu_bf16x2(qv[u] ^ sg[u]);
    if (F16) psi[u] = cvt_pk_bf16(f16_lo(psi[u]), f16_hi(psi[u]));  // the contraction runs on bf16 operands
  }
  const bf16x8 Bq = as_bf16x8(psi);
  // z-block of S'^T: rows with even index hold z' hi, odd rows z' lo, so result registers 0 and 1 of
  // every lane are psi.z'_hi and psi.z'_lo of its token, and their sum is the denominator.
  const u32x4 zsel = {even_row ? zh[0] : zl[0], even_row ? zh[1] : zl[1], even_row ? zh[2] : zl[2],
                      even_row ? zh[3] : zl[3]};
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f}, oz = {0.f, 0.f, 0.f, 0.f};
  o0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, Bq, o0, 0, 0, 0);
  o1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, Bq, o1, 0, 0, 0);
  oz = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(zsel), Bq, oz, 0, 0, 0);
  const float d = oz[0] + oz[1];
  if (den) *den = d;
  const float inv = __builtin_amdgcn_rcpf(d + epsr);
  return u32x4{cvt_pk_h<F16>(o0[0] * inv, o0[1] * inv), cvt_pk_h<F16>(o0[2] * inv, o0[3] * inv),
               cvt_pk_h<F16>(o1[0] * inv, o1[1] * inv), cvt_pk_h<F16>(o1[2] * inv, o1[3] * inv)};
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Copies `bytes` (a multiple of 16) from global memory to LDS with direct global->LDS loads; waves
// take 1 KB chunks round robin.  The caller waits (s_waitcnt) and synchronises before reading.
__device__ __forceinline__ void dma_to_lds(const void* src, void* lds, int bytes, int w, int nw, int lane) {
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(lds);
  for (int c = w; c * 1024 < bytes; c += nw) {
    const int off = c * 1024 + lane * 16;
    if (off < bytes) __builtin_amdgcn_global_load_lds(s + off, (lds_ptr_t)(d + c * 1024), 16, 0, 0);
  }
}

// Lane swap between the two 8-lane halves of every 16-lane row (DPP row_ror:8): lanes whose bank
// (4-lane group within the row) is enabled in `banks` take `src` from the lane 8 away; the others
// keep `old`.
template <int BANKS>
__device__ __forceinline__ u32x4 swap_halves(u32x4 old, u32x4 src) {
  u32x4 r;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    r[u] = (uint32_t)__builtin_amdgcn_update_dpp((int)old[u], (int)src[u], 0x128 /* row_ror:8 */, 0xf, BANKS, false);
  return r;
}

// ---------------------------------------------------------------------------------------------
// Persistent output kernel.  One block per CU keeps S', z' and the query sign masks of the current
// sample in LDS and walks a sequence of 16-token tiles: a contiguous run, or tiles b, b + G, b + 2G,
// ... (G blocks; all blocks then sweep the tensor together, which reads and writes HBM faster when a
// sample spans many tiles per block).  Wave w owns head pairs [w*PPW, w*PPW + PPW).  A head pair of
// one token is one 128-byte span of the Q or O row, so every load and store instruction touches 8
// whole rows x 128 bytes:
// load j of a pair gives lane (n = l%16, kg = l/16) the 16 bytes (token 8j + n%8, head 2p + n/8,
// dims 8kg..8kg+7), and one DPP swap of the row halves turns the two loads into the MFMA B operands
// of the two heads (lane (n, kg) = token n, dims 8kg..8kg+7); stores use the inverse swap.  Q tiles
// rotate through three register sets: each step first issues the loads of the tile two steps ahead
// and then consumes the current one.  Loads and stores are range-checked buffer operations over the tile's
// rows, so rows past the end and a next tile that does not exist cost no memory traffic while every
// step still issues the same instructions (the waits for a tile's loads never cover other
// operations).  The row sums of squares are combined across waves through LDS in a fixed order.
// ---------------------------------------------------------------------------------------------
template <int PPW, bool NORM, bool F16>
__global__ __launch_bounds__(768) void out_persist_bf16(const uint16_t* __restrict__ q, int64_t ldq,
                                                        const uint32_t* __restrict__ gsg,
                                                        const uint16_t* __restrict__ Sop,
                                                        const uint16_t* __restrict__ zop, int B, int N, int H, float eps,
                                                        float inv_C, uint16_t* __restrict__ out, int64_t ldo,
                                                        int tiles_per_block) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint16_t* Ss = reinterpret_cast<uint16_t*>(smem);                          // [H][kOpPerHead]
  uint16_t* Zs = Ss + (size_t)H * kOpPerHead;                                // [H][kZopPerHead]
  uint32_t* Gs = reinterpret_cast<uint32_t*>(Zs + (size_t)H * kZopPerHead);  // [H][kSgnPerHead]
  float* ssq = reinterpret_cast<float*>(Gs + (size_t)H * kSgnPerHead);       // [2][kPersistMaxWaves][16]

  const int NW = blockDim.x >> 6;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, kg = lane >> 4;
  const int tok8 = n16 & 7, hsel = n16 >> 3;  // load/store role of this lane within a head pair
  const int tiles_per_sample = (N + 15) / 16;
  const int64_t total = (int64_t)B * tiles_per_sample;
  const int G = gridDim.x;
  // Tiles t < lim belong to this block's sequence; t >= lim means "none".
  // tiles_per_block = 0: tiles b, b + G, b + 2G, ... (all blocks sweep the tensor together);
  // tiles_per_block = -g: blocks [s*g, s*g + g) share sample s, block s*g + j taking its tiles j, j + g,
  // j + 2g, ... (the group sweeps the sample together); tiles_per_block > 0: a contiguous run.
  const bool strided = tiles_per_block == 0, grouped = tiles_per_block < 0;
  int64_t T0, lim, tile_step;
  if (strided) {
    T0 = blockIdx.x;
    lim = total;
    tile_step = G;
  } else if (grouped) {
    // Consecutive block ids go to the 8 XCDs in turn; when the grid divides evenly, ids are remapped
    // so that the blocks of a sample share an XCD (and its L2 copy of the sample's S', z').
    const int g = -tiles_per_block;
    const int lb = G % 8 == 0 ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int64_t s = lb / g;
    T0 = s * tiles_per_sample + lb % g;
    lim = min(total, (s + 1) * tiles_per_sample);
    tile_step = g;
  } else {
    T0 = (int64_t)blockIdx.x * tiles_per_block;
    lim = min(total, T0 + tiles_per_block);
    tile_step = 1;
  }
  if (T0 >= lim) return;
  const int64_t T1 = T0 + tile_step;

  // Raw loads of one tile: qr[2*i + j] = load j of pair w*PPW + i; all zero, without memory traffic,
  // for rows past N and for t >= lim.  Head indices are clamped into the row; lanes past N or H are
  // never stored.
  auto load_tile = [&](int64_t t, u32x4* qr) {
    const bool valid = t < lim;
    const int64_t tt = valid ? t : T0;
    const int64_t bb = tt / tiles_per_sample;
    const int n0 = (int)(tt - bb * tiles_per_sample) * 16;
    const int rows = valid ? min(16, N - n0) : 0;
    const __amdgpu_buffer_rsrc_t rsrc =
        make_rsrc(q + (bb * N + n0) * ldq, rows > 0 ? (uint32_t)(((rows - 1) * ldq + (int64_t)H * kHeadDim) * 2) : 0u);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t roff = (uint32_t)(((8 * j + tok8) * ldq + kg * 8) * 2);
#pragma unroll
      for (int i = 0; i < PPW; ++i)
        qr[2 * i + j] = buffer_load16(rsrc, roff + (uint32_t)(min(2 * (w * PPW + i) + hsel, H - 1) * kHeadDim * 2));
    }
  };

  int64_t cur_b = -1;
  auto step = [&](int k, int64_t tau, int64_t tau_next, u32x4* cur, u32x4* nxt) {
    const int64_t bb = tau / tiles_per_sample;
    const int n0 = (int)(tau - bb * tiles_per_sample) * 16;
    if (bb != cur_b) {  // uniform across the block
      __syncthreads();
      // S' and z' of the sample go straight from global memory to LDS (global_load_lds_dwordx4:
      // 1 KB per wave instruction, lane l writing bytes [16l, 16l + 16) of the chunk).
      dma_to_lds(Sop + bb * H * kOpPerHead, Ss, H * kOpPerHead * 2, w, NW, lane);
      dma_to_lds(zop + bb * H * kZopPerHead, Zs, H * kZopPerHead * 2, w, NW, lane);
      if (cur_b < 0) dma_to_lds(gsg, Gs, H * kSgnPerHead * 4, w, NW, lane);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      cur_b = bb;
    }
    load_tile(tau_next, nxt);
    // MFMA operand layout: lane (n16, kg) = token n16 of the tile, dims 8kg..8kg+7.
    u32x4 bq[2 * PPW];
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      bq[2 * i] = swap_halves<0xc>(cur[2 * i], cur[2 * i + 1]);
      bq[2 * i + 1] = swap_halves<0x3>(cur[2 * i + 1], cur[2 * i]);
    }
    float epsr = eps;
    if (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 2 * PPW; ++i)
        if (2 * w * PPW + i < H) {
#pragma unroll
          for (int u = 0; u < 4; ++u) ss = dot2_h<F16>(bq[i][u], bq[i][u], ss);
        }
      ss = sum_over_lane_groups(ss);
      float* sb = ssq + (k & 1) * kPersistMaxWaves * 16;
      if (kg == 0) sb[w * 16 + n16] = ss;
      __syncthreads();
      float tot = 0.f;
      for (int ww = 0; ww < NW; ++ww) tot += sb[ww * 16 + n16];
      epsr = eps * sqrtf(tot * inv_C + eps);  // eps / r_q
    }
    // Output rows of this tile as one range-checked buffer: every store instruction is issued (lanes
    // past N or H get an out-of-range offset), so the store count per step is fixed.
    const int rows = min(16, N - n0);
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc(out + (bb * N + n0) * ldo, (uint32_t)(((rows - 1) * ldo + (int64_t)H * kHeadDim) * 2));
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int h0 = 2 * (w * PPW + i);
      {
        u32x4 o[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int h = min(h0 + j, H - 1);
          const uint16_t* sh = Ss + h * kOpPerHead + lane * 8;
          const uint16_t* zh = Zs + h * kZopPerHead + kg * 8;
          o[j] = head_out<F16>(bq[2 * i + j], *reinterpret_cast<const u32x4*>(Gs + h * kSgnPerHead + kg * 4),
                          as_bf16x8(*reinterpret_cast<const u32x4*>(sh)),
                          as_bf16x8(*reinterpret_cast<const u32x4*>(sh + 512)), *reinterpret_cast<const u32x4*>(zh),
                          *reinterpret_cast<const u32x4*>(zh + kHeadDim), epsr, (lane & 1) == 0);
        }
        const u32x4 st[2] = {swap_halves<0xc>(o[0], o[1]), swap_halves<0x3>(o[1], o[0])};
        const int h = h0 + hsel;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = 8 * j + tok8;
          const uint32_t off = (r < rows && h < H) ? (uint32_t)((r * ldo + h * kHeadDim + kg * 8) * 2) : kOutOfRange;
          buffer_store16_nt(orsrc, off, st[j]);
        }
      }
    }
  };

  u32x4 qa[2 * PPW], qb[2 * PPW], qc[2 * PPW];  // three tiles: one consumed, two loading
  {
    // Each wave copies the first sample's operands of its own heads (the only ones it reads until the
    // sample changes) ahead of its first Q tile, so its waits cover only them (vmcnt retires in issue
    // order) and need no block-wide barrier; the tile's loads stay in flight.  (Staging through
    // registers measured 0.9 us per call faster here than direct global->LDS loads.)
    const int64_t b0 = T0 / tiles_per_sample;
    const int hb = min(H, 2 * w * PPW), he = min(H, 2 * (w + 1) * PPW);
    // Range-checked buffer loads (lanes past the region read zeros, no traffic), the first tile's loads
    // behind them, then LDS stores of the region only.
    const int nh = max(0, he - hb);
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(Sop + (b0 * H + hb) * kOpPerHead, (uint32_t)(nh * kOpPerHead * 2));
    const __amdgpu_buffer_rsrc_t rZ = make_rsrc(zop + (b0 * H + hb) * kZopPerHead, (uint32_t)(nh * kZopPerHead * 2));
    const __amdgpu_buffer_rsrc_t rG = make_rsrc(gsg + hb * kSgnPerHead, (uint32_t)(nh * kSgnPerHead * 4));
    constexpr int CS = 2 * PPW * kOpPerHead * 2 / 1024, CZ = (2 * PPW * kZopPerHead * 2 + 1023) / 1024,
                  CG = (2 * PPW * kSgnPerHead * 4 + 1023) / 1024;
    u32x4 st[CS + CZ + CG];
#pragma unroll
    for (int c = 0; c < CS; ++c) st[c] = buffer_load16(rS, c * 1024 + lane * 16);
#pragma unroll
    for (int c = 0; c < CZ; ++c) st[CS + c] = buffer_load16(rZ, c * 1024 + lane * 16);
#pragma unroll
    for (int c = 0; c < CG; ++c) st[CS + CZ + c] = buffer_load16(rG, c * 1024 + lane * 16);
    __asm__ __volatile__("" ::: "memory");
    load_tile(T0, qa);
    load_tile(T1, qb);
    __asm__ __volatile__("" ::: "memory");
    char* dS = reinterpret_cast<char*>(Ss + hb * kOpPerHead);
    char* dZ = reinterpret_cast<char*>(Zs + hb * kZopPerHead);
    char* dG = reinterpret_cast<char*>(Gs + hb * kSgnPerHead);
#pragma unroll
    for (int c = 0; c < CS; ++c)
      if (c * 1024 + lane * 16 < nh * kOpPerHead * 2) store16(dS + c * 1024 + lane * 16, st[c]);
#pragma unroll
    for (int c = 0; c < CZ; ++c)
      if (c * 1024 + lane * 16 < nh * kZopPerHead * 2) store16(dZ + c * 1024 + lane * 16, st[CS + c]);
#pragma unroll
    for (int c = 0; c < CG; ++c)
      if (c * 1024 + lane * 16 < nh * kSgnPerHead * 4) store16(dG + c * 1024 + lane * 16, st[CS + CZ + c]);
    cur_b = b0;
  }
  // Each step consumes one register set and starts the loads of the tile two steps ahead into the set
  // freed by the step before (qa, qb, qc rotate; two tiles ahead measured 26.0 against 26.7 us per
  // launch for one tile ahead on the 16384-token workload).  The first step is peeled so that the loop
  // is entered, like its back edge, with the same loads and stores outstanding; the loop's three steps
  // run unconditionally, so no control-flow merge of different outstanding counts lets the compiler's
  // waits for a tile's loads cover earlier stores.
  int64_t t1 = T1;
  step(0, T0, T1 + tile_step, qa, qc);
  int k = 1;
  while (t1 < lim) {
    step(k, t1, t1 + 2 * tile_step, qb, qa);
    if (t1 + tile_step >= lim) break;
    step(k + 1, t1 + tile_step, t1 + 3 * tile_step, qc, qb);
    if (t1 + 2 * tile_step >= lim) break;
    step(k + 2, t1 + 2 * tile_step, t1 + 4 * tile_step, qa, qc);
    t1 += 3 * tile_step;
    k += 3;
  }
}

// ---------------------------------------------------------------------------------------------
// Non-persistent output kernel (few tiles, or H too large for the LDS-resident state).  Block =
// 4 waves over 16 tokens of sample b and up to 4*HPW heads (blockIdx.z); wave w owns heads
// [g0 + w*HPW, g0 + w*HPW + HPW).  PRE_R = false: the block covers all H heads and forms r_q from the
// Q rows it holds; PRE_R = true: r_q comes from a row-statistics pass (H > 4*HPW).
// ---------------------------------------------------------------------------------------------
template <int HPW, bool NORM, bool PRE_R, bool F16>
__global__ __launch_bounds__(256) void out_bf16(const uint16_t* __restrict__ q, int64_t ldq,
                                                const uint32_t* __restrict__ gsg, const uint16_t* __restrict__ Sop,
                                                const uint16_t* __restrict__ zop, const float* __restrict__ r_q, int N,
                                                int H, float eps, float inv_C, uint16_t* __restrict__ out,
                                                int64_t ldo) {
  __shared__ float ssq[4][16];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int t = lane & 15, kg = lane >> 4;
  const int n = blockIdx.x * 16 + t;
  const int hbeg = blockIdx.z * 4 * HPW + w * HPW;
  const int hcnt = max(0, min(HPW, H - hbeg));
  const int64_t row0 = (int64_t)b * N;
  const uint16_t* row = q + (row0 + min(n, N - 1)) * ldq + kg * 8;

  u32x4 qr[HPW];
#pragma unroll
  for (int i = 0; i < HPW; ++i) qr[i] = load16(row + min(hbeg + i, H - 1) * kHeadDim);
  float epsr = eps;
  if (NORM && PRE_R) {
    epsr = eps / r_q[row0 + min(n, N - 1)];
  } else if (NORM) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < HPW; ++i)
      if (i < hcnt) {
#pragma unroll
        for (int u = 0; u < 4; ++u) ss = dot2_h<F16>(qr[i][u], qr[i][u], ss);
      }
    ss = sum_over_lane_groups(ss);
    if (kg == 0) ssq[w][t] = ss;
    __syncthreads();
    const float tot = ((ssq[0][t] + ssq[1][t]) + ssq[2][t]) + ssq[3][t];
    epsr = eps * sqrtf(tot * inv_C + eps);
  }
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    if (i < hcnt) {
      const int h = hbeg + i;
      const int64_t bh = (int64_t)b * H + h;
      const u32x4 sg = load16(gsg + h * kSgnPerHead + kg * 4);
      const uint16_t* sh = Sop + bh * kOpPerHead + lane * 8;
      const uint16_t* zh = zop + bh * kZopPerHead + kg * 8;
      const u32x4 o = head_out<F16>(qr[i], sg, as_bf16x8(load16(sh)), as_bf16x8(load16(sh + 512)), load16(zh),
                               load16(zh + kHeadDim), epsr, (lane & 1) == 0);
      if (n < N) store16_nt(out + (row0 + n) * ldo + h * kHeadDim + kg * 8, o);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Host launch of the bf16 path.
// ---------------------------------------------------------------------------------------------

size_t out_persist_lds_bytes(int H) {
  return (size_t)H * (kOpPerHead * 2 + kZopPerHead * 2 + kSgnPerHead * 4) + 2 * kPersistMaxWaves * 16 * 4;
}

size_t bf16_operand_bytes(int64_t BH, int H) {
  return (size_t)BH * (kOpPerHead + kZopPerHead) * 2 + (size_t)H * kSgnPerHead * 4;
}

template <bool F16>
static hipError_t launch_attn_16(const AttnPlan& p, const uint16_t* q, int64_t ldq, const uint16_t* k,
                                 const uint16_t* v, int64_t ldkv, const float* gq, const float* gk, float eps,
                                 uint16_t* out, int64_t ldo, void* ws, int num_cus, hipStream_t stream,
                                 const float* k_ssq, int k_parts) {
  char* base = static_cast<char*>(ws);
  float* r_k = reinterpret_cast<float*>(base + p.off_rk);
  float* part = reinterpret_cast<float*>(base + p.off_part);
  uint16_t* Sop = reinterpret_cast<uint16_t*>(base + p.off_Sop);
  uint16_t* zop = Sop + (size_t)p.B * p.H * kOpPerHead;
  uint32_t* gsg = reinterpret_cast<uint32_t*>(zop + (size_t)p.B * p.H * kZopPerHead);
  const int B = p.B, N = p.N, H = p.H, C = H * kHeadDim;
  const int64_t rows = (int64_t)B * N;
  const int64_t BH = (int64_t)B * H;
  const unsigned rs_blocks = (unsigned)((rows + 3) / 4);

  const float inv_C = 1.0f / (float)C;
  float* r_q = reinterpret_cast<float*>(base + p.off_rq);
  const bool groups = p.out_kind == kOutTileGroups;
  const bool xchg = p.state_xchg && p.norm && !k_ssq && !groups;
  if (xchg) {
    const hipError_t e = launch_kv_state_x(F16, k, v, ldkv, gq, gk, B, N, H, p.Tc, p.NC, eps, base + p.off_xchg,
                                           next_epoch(), p.xchg_spin, part, Sop, zop, gsg, stream);
    if (e != hipSuccess) return e;
  } else if (p.norm && groups)  // r_k and r_q in one launch (the output blocks see only some heads of a row)
    launch_kernel("rowstats_kq", rowstats_kernel<uint16_t, F16>, (unsigned)((2 * rows + 3) / 4), 256, 0, stream, k,
                  ldkv, rows, C, eps, r_k, q, ldq, r_q);
  else if (p.norm && k_ssq)
    launch_kernel("rowfinish_k", rowfinish_kernel, (unsigned)((rows + 255) / 256), 256, 0, stream, k_ssq, k_parts, rows,
                  inv_C, eps, r_k);
  else if (p.norm)
    launch_kernel("rowstats_k", p.nt_v ? rowstats_kernel<uint16_t, F16, true> : rowstats_kernel<uint16_t, F16>,
                  rs_blocks, 256, 0, stream, k, ldkv, rows, C, eps, r_k,
                  nullptr, 0, nullptr);
  const dim3 grid(p.NC, (H + 1) / 2, B);
  // Several chunks: reduced by the state blocks themselves (rendezvous) or by kv_reduce_bf16.
  const bool rdv = p.rendezvous && !xchg;
  uint32_t* flags = rdv ? reinterpret_cast<uint32_t*>(base + p.off_flags) : nullptr;
  const uint32_t epoch = rdv ? next_epoch() : 0u;
  const bool ntv = p.nt_v;  // non-temporal K and V loads (the planner's choice)
  if (xchg) {
  } else if (p.norm)
    launch_kernel("kv_state", ntv ? kv_state_bf16<true, F16, true> : kv_state_bf16<true, F16, false>, grid, 256, 0,
                  stream, k, v, ldkv, r_k, gq, gk, N, H, p.Tc, p.NC, part, Sop, zop, gsg, flags, epoch, p.xchg_spin);
  else
    launch_kernel("kv_state", ntv ? kv_state_bf16<false, F16, true> : kv_state_bf16<false, F16, false>, grid, 256, 0,
                  stream, k, v, ldkv, nullptr, nullptr, nullptr, N, H, p.Tc, p.NC, part, Sop, zop, gsg, flags, epoch,
                  p.xchg_spin);
  if (p.NC > 1 && !rdv) {
    const unsigned blocks = (unsigned)((BH * kPartStride + 255) / 256);
    if (p.norm)
      launch_kernel("kv_reduce", kv_reduce_bf16<true>, blocks, 256, 0, stream, part, p.NC, H, BH, gq, gk, Sop, zop,
                    gsg);
    else
      launch_kernel("kv_reduce", kv_reduce_bf16<false>, blocks, 256, 0, stream, part, p.NC, H, BH, nullptr, nullptr,
                    Sop, zop, gsg);
  }

  if (p.out_kind == kOutPersist) {
    const int64_t tiles = (int64_t)B * ((N + 15) / 16);
    const int blocks = (int)std::min<int64_t>(num_cus, tiles);
    const int per = (int)((tiles + blocks - 1) / blocks);
    // Strided over the tensor, grouped per sample, or contiguous runs (kernel argument 0, -g, run).
    const int nblk = p.out_strided ? blocks : p.out_group > 0 ? B * p.out_group : (int)((tiles + per - 1) / per);
    const int per_arg = p.out_strided ? 0 : p.out_group > 0 ? -p.out_group : per;
    const size_t lds = out_persist_lds_bytes(H);
    const int nw = ((H + 1) / 2 + kPersistPPW - 1) / kPersistPPW;
    if (nw > kPersistMaxWaves) return hipErrorInvalidValue;  // the planner never picks this kernel then
    const hipError_t ea =
        p.norm ? ensure_max_lds(reinterpret_cast<const void*>(&out_persist_bf16<kPersistPPW, true, F16>), 160 * 1024)
               : ensure_max_lds(reinterpret_cast<const void*>(&out_persist_bf16<kPersistPPW, false, F16>), 160 * 1024);
    if (ea != hipSuccess) return ea;
    final_launch();
    if (p.norm)
      launch_kernel("out", out_persist_bf16<kPersistPPW, true, F16>, nblk, nw * 64, lds, stream, q, ldq, gsg, Sop, zop,
                    B, N, H, eps, inv_C, out, ldo, per_arg);
    else
      launch_kernel("out", out_persist_bf16<kPersistPPW, false, F16>, nblk, nw * 64, lds, stream, q, ldq, gsg, Sop, zop,
                    B, N, H, eps, inv_C, out, ldo, per_arg);
    return hipGetLastError();
  }
  if (groups) {
    constexpr int HPWG = 2;  // 8 heads per block (20 per block: 1024-token call 17.6 against 16.8 us)
    const dim3 ogrid((N + 15) / 16, B, (H + 4 * HPWG - 1) / (4 * HPWG));
    final_launch();
    if (p.norm)
      launch_kernel("out", out_bf16<HPWG, true, true, F16>, ogrid, 256, 0, stream, q, ldq, gsg, Sop, zop, r_q, N, H,
                    eps, inv_C, out, ldo);
    else
      launch_kernel("out", out_bf16<HPWG, false, true, F16>, ogrid, 256, 0, stream, q, ldq, gsg, Sop, zop, nullptr, N,
                    H, eps, inv_C, out, ldo);
    return hipGetLastError();
  }
  constexpr int HPW = 18;
  if (H <= 4 * HPW) {
    const dim3 ogrid((N + 15) / 16, B, 1);
    final_launch();
    if (p.norm)
      launch_kernel("out", out_bf16<HPW, true, false, F16>, ogrid, 256, 0, stream, q, ldq, gsg, Sop, zop, nullptr, N, H,
                    eps, inv_C, out, ldo);
    else
      launch_kernel("out", out_bf16<HPW, false, false, F16>, ogrid, 256, 0, stream, q, ldq, gsg, Sop, zop, nullptr, N,
                    H, eps, inv_C, out, ldo);
  } else {
    const dim3 ogrid((N + 15) / 16, B, (H + 4 * HPW - 1) / (4 * HPW));
    if (p.norm) {
      launch_kernel("rowstats_q", rowstats_kernel<uint16_t, F16>, rs_blocks, 256, 0, stream, q, ldq, rows, C, eps, r_q,
                    nullptr, 0, nullptr);
      final_launch();
      launch_kernel("out", out_bf16<HPW, true, true, F16>, ogrid, 256, 0, stream, q, ldq, gsg, Sop, zop, r_q, N, H, eps,
                    inv_C, out, ldo);
    } else {
      final_launch();
      launch_kernel("out", out_bf16<HPW, false, true, F16>, ogrid, 256, 0, stream, q, ldq, gsg, Sop, zop, nullptr, N, H,
                    eps, inv_C, out, ldo);
    }
  }
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnPlan& p, const uint16_t* q, int64_t ldq, const uint16_t* k, const uint16_t* v,
                            int64_t ldkv, const float* gq, const float* gk, float eps, uint16_t* out, int64_t ldo,
                            void* ws, int num_cus, hipStream_t stream, const float* k_ssq, int k_parts) {
  if (p.dtype == kDtypeF16)
    return launch_attn_16<true>(p, q, ldq, k, v, ldkv, gq, gk, eps, out, ldo, ws, num_cus, stream, k_ssq, k_parts);
  return launch_attn_16<false>(p, q, ldq, k, v, ldkv, gq, gk, eps, out, ldo, ws, num_cus, stream, k_ssq, k_parts);
}

}  // namespace sanala

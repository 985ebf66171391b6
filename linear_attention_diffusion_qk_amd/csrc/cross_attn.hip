// Cross-attention with QK-Norm on gfx950: queries from the image tokens, keys and values from the text
// tokens, softmax over each sample's valid text tokens ("SANA 1.5: Efficient Scaling of Training-Time
// and Inference-Time Compute in Linear Diffusion Transformer" (research notes), model architecture: the
// Linear DiT block's vanilla cross-attention, and the QK Norm bullet: RMSNorm on its queries and keys).
//
// Launches on one stream:
//   cross_prep  (QK-Norm on) one wave per row.  Text tokens: r_k = 1/sqrt(mean_c k^2 + eps) and
//               k^ = bf16(k * r_k * gk), the normalised keys the MFMA takes.  Image tokens: r_q.
//               Norm off: no launch, k^ = k.
//   cross_attn  block = (chunk of queries, head, sample), 8 waves.  The head's k^ and v of the sample go
//               to LDS once per block (k^ row-major with an XOR swizzle, v transposed); then each wave
//               takes 32 queries at a time: q^ = bf16(q * r_q * gq) in registers, S^T = k^ q^T on
//               v_mfma_f32_32x32x16_bf16, so that a lane holds one query's logits for 16 of every 32
//               keys and the softmax's max and sum are in-lane plus one exchange between the two lane
//               halves.  The logits are exact products of the bf16 operands (fp32 sums).  With the
//               norm on, q^ carries the softmax scale log2(e)/sqrt(D) (one rounding either way) and
//               the subtracted constant m is added on the MFMA, so P = exp2 of the accumulator; without
//               it q and k are used as given, and the scale and m are applied in fp32 by one FMA per
//               logit (folding the scale into a bf16 operand would round logits of a few hundred by a
//               whole unit).  m is the Cauchy-Schwarz bound |q^| max|k^| where that keeps the weights
//               in range, else the exact row maximum from a first pass over the keys (the logits are
//               formed again rather than kept).  P is rounded to bf16 (its row sum taken over those
//               rounded values) and O^T = V^T P^T runs on the same MFMA with P taken straight from the
//               S^T registers: the MFMA's k index runs over the keys in the order the accumulator holds
//               them (lane half g: keys 4g..4g+3 and 8+4g..8+4g+3 of each 16), and V^T is read from LDS
//               in that order.  o = O / sum, stored as bf16.
#include "common.h"

#include <algorithm>
#include <atomic>
#include <cmath>

namespace sanala {

namespace {
constexpr int kCrossWaves = 8;      // waves per cross_attn block: they share one staged head
constexpr int kCrossPrepUnits = 8;  // 16-byte units per lane in cross_prep: rows of up to 4096 channels
constexpr float kLog2e = 1.4426950408889634f;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Byte offset of 16-byte unit u (dims 8u..8u+7) of key j in the staged k^ tile (64-byte rows).  The
// XOR with bits 2-3 of j puts the same unit of any 16 consecutive keys in 16 different bank slots.
__device__ __forceinline__ int khat_off(int j, int u) { return j * 64 + 16 * (u ^ ((j >> 2) & 3)); }
}  // namespace

// Rows [0, krows): text tokens of k -> khat; rows [krows, krows + qrows): r_q of q.
__global__ __launch_bounds__(256) void cross_prep(const uint16_t* __restrict__ k, const uint16_t* __restrict__ q,
                                                  const float* __restrict__ gk, int64_t krows, int64_t qrows, int C,
                                                  float eps, uint16_t* __restrict__ khat, float* __restrict__ r_q) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= krows + qrows) return;
  const bool is_k = row < krows;  // uniform per wave
  const uint16_t* src = is_k ? k + row * C : q + (row - krows) * C;
  const int nvec = C / 8;
  u32x4 w[kCrossPrepUnits];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kCrossPrepUnits; ++j) {
    const int i = lane + 64 * j;
    w[j] = i < nvec ? load16(src + 8 * i) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u) ss = dot2_bf16(w[j][u], w[j][u], ss);
  }
  const float r = 1.0f / sqrtf(wave_sum(ss) / (float)C + eps);
  if (!is_k) {
    if (lane == 0) r_q[row - krows] = r;
    return;
  }
#pragma unroll
  for (int j = 0; j < kCrossPrepUnits; ++j) {
    const int i = lane + 64 * j;
    if (i < nvec) {
      const f32x4 g0 = loadf4(gk + 8 * i), g1 = loadf4(gk + 8 * i + 4);
      const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
      u32x4 o;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        o[u] = cvt_pk_bf16(bf16_lo(w[j][u]) * r * g[2 * u], bf16_hi(w[j][u]) * r * g[2 * u + 1]);
      store16(khat + row * C + 8 * i, o);
    }
  }
}

// q, out: [B, N, C]; khat (k itself without the norm), v: [B, L, C]; C = 32 H; sc = log2(e)/sqrt(D).
// kv_len: valid text tokens per sample (NULL: L), clamped to [0, L]; a sample with none gets zeros.
// Block (x, h, b) of W = kCrossWaves waves, gridDim.x = P blocks per (head, sample), sized so that the
// whole grid is resident at once: the block stages head h once and takes the 32-query tiles
// x, x + P, x + 2P, ..., wave w every W-th of those.
template <bool NORM>
__global__ __launch_bounds__(64 * kCrossWaves, 4) void cross_attn_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ khat,
                                                       const uint16_t* __restrict__ v, const float* __restrict__ r_q,
                                                       const float* __restrict__ gq, const int* __restrict__ kv_len,
                                                       int N, int L, int Lp, int H, float sc,
                                                       uint16_t* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* const Ks = lds;                          // Lp keys x 64 bytes, swizzled (khat_off)
  uint16_t* const Vt = reinterpret_cast<uint16_t*>(lds + Lp * 64);  // 32 dims x vpitch bf16 (v transposed)
  const int vpitch = Lp + 4;  // in bf16: 2*Lp + 8 bytes, an odd multiple of 8 bytes, so the 32 rows of
                              // an 8-byte read at one key offset fall in 32 different bank pairs
  const int h = blockIdx.y, b = blockIdx.z;
  const int C = H * kHeadDim;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, hf = lane >> 5;
  const int kvl = kv_len ? min(max(kv_len[b], 0), L) : L;

  // Stage k^ and v^T of head h (keys past L are zero), and the largest squared norm of a valid key
  // (the four lanes holding one key's four units are adjacent).
  __shared__ float kmax_w[kCrossWaves];
  const int64_t kv0 = (int64_t)b * L;
  float kmax = 0.f;
  for (int i = tid; i < Lp * 4; i += 64 * kCrossWaves) {
    const int j = i >> 2, u = i & 3;
    u32x4 kk = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (j < L) {
      kk = load16(khat + (kv0 + j) * C + h * kHeadDim + 8 * u);
      vv = load16(v + (kv0 + j) * C + h * kHeadDim + 8 * u);
    }
    float kn = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) kn = dot2_bf16(kk[e], kk[e], kn);
    kn += __shfl_xor(kn, 1);
    kn += __shfl_xor(kn, 2);
    if (j < kvl) kmax = fmaxf(kmax, kn);
    store16(Ks + khat_off(j, u), kk);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      Vt[(8 * u + e) * vpitch + j] = (uint16_t)((e & 1) ? (vv[e >> 1] >> 16) : (vv[e >> 1] & 0xffffu));
  }
#pragma unroll
  for (int o = 32; o >= 4; o >>= 1) kmax = fmaxf(kmax, __shfl_xor(kmax, o));
  if (lane == 0) kmax_w[w] = kmax;

  __syncthreads();

  const int ktiles = (kvl + 31) / 32;  // key tiles holding a valid key
  kmax = kmax_w[0];
#pragma unroll
  for (int i = 1; i < kCrossWaves; ++i) kmax = fmaxf(kmax, kmax_w[i]);
  const int64_t qrow0 = (int64_t)b * N;
  const int P = gridDim.x, ntile = (N + 31) / 32;
  const int qtiles = (ntile - (int)blockIdx.x + P * kCrossWaves - 1 - P * w) / (P * kCrossWaves);  // this wave's
  auto qload = [&](int t, u32x4& qa, u32x4& qb, float& rq) {
    const int n = min(((int)blockIdx.x + P * (w + kCrossWaves * t)) * 32 + ql, N - 1);
    const uint16_t* qr = q + (qrow0 + n) * C + h * kHeadDim + 8 * hf;
    qa = load16(qr);
    qb = load16(qr + 16);
    rq = NORM ? r_q[qrow0 + n] : 1.f;
  };
  u32x4 qa, qb;
  float rq;
  qload(0, qa, qb, rq);
  for (int t = 0; t < qtiles; ++t) {
    const int n0 = ((int)blockIdx.x + P * (w + kCrossWaves * t)) * 32;
    // q^ = bf16(q * r_q * gq) (the gains of this lane's dims 8hf..8hf+7 and 16+8hf..16+8hf+7 are read
    // again per tile from the cache rather than held in registers); the next tile's loads go out now.
    u32x4 qh[2] = {qa, qb};
    if (NORM) {
      rq *= sc;  // the softmax scale rides on the one rounding q^ takes anyway
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const float* gp = gq + h * kHeadDim + 16 * ks + 8 * hf;
        const f32x4 g0 = loadf4(gp), g1 = loadf4(gp + 4);
        const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
        const u32x4 x = ks ? qb : qa;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          qh[ks][u] = cvt_pk_bf16(bf16_lo(x[u]) * rq * g[2 * u], bf16_hi(x[u]) * rq * g[2 * u + 1]);
      }
    }
    if (t + 1 < qtiles) qload(t + 1, qa, qb, rq);

    // The logits are formed on the MFMA; the next tile's logits are issued before this tile's vector
    // work (two accumulator sets taken in turn), so the wave covers the MFMA latency itself.  Only the
    // tile holding the last valid key is masked.  A wave raises its issue priority while it issues
    // MFMAs (s_setprio), so that the matrix core of its SIMD is fed ahead of the other waves' vector work.
    //
    // With the norm on, q^ carries the scale sc, and the constant the softmax subtracts is added on the
    // MFMA too: a product of a ones column of the keys with (-m_hi, -m_lo) in the queries' first two
    // slots (32x32x8, m = m_hi + m_lo to 2^-17 relative, the same for every key of a query) adds -m to
    // each logit, so a weight is exp2 of the accumulator itself.  Without the norm q and k are used as
    // given, so folding the scale into a bf16 operand would add a rounding the logits do not otherwise
    // take: there the scale and the constant are applied in fp32 by one FMA per logit.
    const f32x16 zero = {};
    const i16x4 kone = {(short)(hf == 0 ? 0x3f80 : 0), (short)(hf == 0 ? 0x3f80 : 0), 0, 0};  // A[key][0..1] = 1
    i16x4 qbias = {0, 0, 0, 0};
    auto logits = [&](int tt) {
      const u32x4 a0 = load16(Ks + khat_off(32 * tt + ql, hf));
      const u32x4 a1 = load16(Ks + khat_off(32 * tt + ql, 2 + hf));
      f32x16 st;
      __builtin_amdgcn_s_setprio(1);
      if constexpr (NORM) {
        st = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(kone, qbias, zero, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), as_bf16x8(qh[0]), st, 0, 0, 0);
      } else {
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), as_bf16x8(qh[0]), zero, 0, 0, 0);
      }
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1), as_bf16x8(qh[1]), st, 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
      // st[r]: query n0 + ql, key 32 tt + 8 (r / 4) + 4 hf + r % 4
      if (32 * tt + 32 > kvl) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * tt + 8 * (r >> 2) + 4 * hf + (r & 3) >= kvl) st[r] = -INFINITY;
      }
      return st;
    };
    // The constant subtracted before the exponential: softmax does not depend on it, and fp32 and bf16
    // keep their relative precision over the whole exponent range, so any m >= every logit serves as
    // long as it does not exceed them by so much that the weights leave the normal range.  By
    // Cauchy-Schwarz m = |q^| max_j |k^_j| bounds every logit, and its overshoot is at most 2m; where
    // 2m <= 64 in exponent units for every query of the tile (always with the norm at SANA's scales)
    // that bound is used and the logits are formed once; otherwise a first pass takes the exact row
    // maximum.
    float qn = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) qn = dot2_bf16(qh[1][u], qh[1][u], dot2_bf16(qh[0][u], qh[0][u], qn));
    qn += __shfl_xor(qn, 32);
    float m = sqrtf(qn * kmax) * (1.0f + 0x1p-12f) + 0x1p-100f;
    const float scl = NORM ? 1.f : sc;  // scale still to apply to an accumulator value
    f32x16 s0, s1;
    if (__ballot(scl * 2.f * m > 64.f) != 0) {  // uniform per wave
      m = -INFINITY;
      auto take_max = [&](const f32x16& st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, st[r]);
      };
      s0 = logits(0);
      for (int tt = 0; tt < ktiles; tt += 2) {
        if (tt + 1 < ktiles) s1 = logits(tt + 1);
        take_max(s0);
        if (tt + 2 < ktiles) s0 = logits(tt + 2);
        if (tt + 1 < ktiles) take_max(s1);
      }
      m = fmaxf(m, __shfl_xor(m, 32));
      if (!(m > -INFINITY)) m = 0.f;  // no valid key: every weight is zero anyway
    }
    if constexpr (NORM) {
      const uint32_t hi = f32_to_bf16_bits(-m) & 0xffffu;
      const uint32_t lo = f32_to_bf16_bits(-m - __uint_as_float(hi << 16)) & 0xffffu;
      qbias = {(short)(hf == 0 ? hi : 0u), (short)(hf == 0 ? lo : 0u), 0, 0};
    }
    const float cm = -scl * m;  // the fp32 path's constant
    // The row sum is taken over the bf16-rounded weights the value product uses (v_dot2 against
    // ones), in two halves for a shorter dependency chain.
    float l0 = 0.f, l1 = 0.f;
    constexpr uint32_t kOnes = 0x3f803f80u;  // two bf16 ones
    f32x16 o = zero;
    // Half jj of a key tile: keys 16 jj .. 16 jj + 15 (accumulator entries 8 jj .. 8 jj + 7).
    auto consume_half = [&](const f32x16& st, int tt, int jj) {
      uint32_t pk[4];
#pragma unroll
      for (int r = 8 * jj; r < 8 * jj + 8; r += 2) {
        if constexpr (NORM)
          pk[(r >> 1) & 3] = cvt_pk_bf16(__builtin_amdgcn_exp2f(st[r]), __builtin_amdgcn_exp2f(st[r + 1]));
        else
          pk[(r >> 1) & 3] = cvt_pk_bf16(__builtin_amdgcn_exp2f(fmaf(st[r], scl, cm)),
                                         __builtin_amdgcn_exp2f(fmaf(st[r + 1], scl, cm)));
      }
      l0 = dot2_bf16(pk[0], kOnes, l0);
      l1 = dot2_bf16(pk[1], kOnes, l1);
      l0 = dot2_bf16(pk[2], kOnes, l0);
      l1 = dot2_bf16(pk[3], kOnes, l1);
      const int kb = 32 * tt + 16 * jj + 4 * hf;
      const u32x2 a0 = *reinterpret_cast<const u32x2*>(Vt + ql * vpitch + kb);
      const u32x2 a1 = *reinterpret_cast<const u32x2*>(Vt + ql * vpitch + kb + 8);
      const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
      const u32x4 bp = {pk[0], pk[1], pk[2], pk[3]};
      __builtin_amdgcn_s_setprio(1);
      o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(bp), o, 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
    };
    // The upper half of the tile holding the last valid key is skipped when it holds none.
    auto consume = [&](const f32x16& st, int tt) {
      consume_half(st, tt, 0);
      if (32 * tt + 16 < kvl) consume_half(st, tt, 1);
    };
    s0 = logits(0);
    for (int tt = 0; tt < ktiles; tt += 2) {
      if (tt + 1 < ktiles) s1 = logits(tt + 1);
      consume(s0, tt);
      if (tt + 2 < ktiles) s0 = logits(tt + 2);
      if (tt + 1 < ktiles) consume(s1, tt + 1);
    }
    const float l_run = l0 + l1;
    // o[r]: dim 8 (r / 4) + 4 hf + r % 4 of query n0 + ql.
    const float lt = l_run + __shfl_xor(l_run, 32);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int n = n0 + ql;
    if (n < N) {
      uint16_t* orow = out + (qrow0 + n) * C + h * kHeadDim + 4 * hf;
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const u32x2 pv = {cvt_pk_bf16(o[4 * gi] * inv, o[4 * gi + 1] * inv),
                          cvt_pk_bf16(o[4 * gi + 2] * inv, o[4 * gi + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 8 * gi) = pv;  // ordinary stores: 8-26% faster than non-temporal
      }
    }
  }
}

size_t cross_attn_workspace_bytes(int64_t B, int64_t N, int64_t L, int H) {
  const size_t khat = ((size_t)B * L * H * kHeadDim * 2 + 255) / 256 * 256;
  return khat + (size_t)B * N * 4;
}

int cross_attn_max_keys() { return 1024; }
int cross_attn_max_heads() { return 64 * kCrossPrepUnits * 8 / kHeadDim; }

hipError_t launch_cross_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* gq, const float* gk,
                             const int* kv_len, int B, int N, int L, int H, float eps, uint16_t* out, void* ws,
                             hipStream_t stream) {
  const int C = H * kHeadDim;
  uint16_t* khat = static_cast<uint16_t*>(ws);
  float* r_q = reinterpret_cast<float*>(static_cast<char*>(ws) + ((size_t)B * L * C * 2 + 255) / 256 * 256);
  const bool norm = gq != nullptr;
  const int64_t krows = (int64_t)B * L, qrows = (int64_t)B * N;
  const float c = kLog2e / std::sqrt((float)kHeadDim);
  if (norm)
    launch_kernel("cross_prep", cross_prep, (unsigned)((krows + qrows + 3) / 4), 256, 0, stream, k, q, gk, krows, qrows,
                  C, eps, khat, r_q);
  const uint16_t* kh = norm ? khat : k;
  const int Lp = (L + 31) / 32 * 32;
  const size_t lds = (size_t)Lp * 64 + (size_t)kHeadDim * (Lp + 4) * 2;
  // Blocks per (head, sample): as many as keep the grid resident at once (two 8-wave blocks per CU),
  // at most one per 8 query tiles.
  static std::atomic<int> cus_of[64];  // compute units per device, queried once
  int dev = 0, num_cus = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    num_cus = cus_of[dev].load(std::memory_order_relaxed);
    if (num_cus <= 0 && hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cus_of[dev].store(num_cus, std::memory_order_relaxed);
  }
  if (num_cus <= 0) num_cus = 256;
  const int64_t per_head = std::max<int64_t>(1, 2 * (int64_t)num_cus / ((int64_t)H * B));
  const int P = (int)std::min<int64_t>(per_head, ((N + 31) / 32 + kCrossWaves - 1) / kCrossWaves);
  const dim3 grid((unsigned)P, (unsigned)H, (unsigned)B);
  const void* kern = norm ? reinterpret_cast<const void*>(&cross_attn_bf16<true>)
                          : reinterpret_cast<const void*>(&cross_attn_bf16<false>);
  // Dynamic LDS of up to 128.3 KB (1024 text tokens); the kernel's static LDS takes the rest of the
  // 160 KB a block may use.
  const hipError_t ea = ensure_max_lds(kern, 159 * 1024);
  if (ea != hipSuccess) return ea;
  final_launch();
  if (norm)
    launch_kernel("cross_attn", cross_attn_bf16<true>, grid, 64 * kCrossWaves, lds, stream, q, kh, v, r_q, gq, kv_len, N, L, Lp, H,
                  c, out);
  else
    launch_kernel("cross_attn", cross_attn_bf16<false>, grid, 64 * kCrossWaves, lds, stream, q, kh, v, r_q, gq, kv_len, N, L, Lp, H,
                  c, out);
  return hipGetLastError();
}

}  // namespace sanala

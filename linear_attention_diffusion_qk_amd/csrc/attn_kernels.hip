// HIP kernels (gfx950) for ReLU linear self-attention with QK-RMSNorm.
//
// Operation: "Sana: Efficient High-Resolution Image Synthesis with Linear Diffusion Transformers"
// (paper notes), section 2.1, Eq. (1), evaluated per head in the precompute-then-apply order that
// the notes give right after Eq. (1): first the per-head state S = sum_j phi(K_j)^T V_j and
// z = sum_j phi(K_j), then O(D^2) work per token.  phi(x) = ReLU(RMSNorm(x) * g) with the RMSNorm
// over all channels of a token ("SANA 1.5: Efficient Scaling of Training-Time and Inference-Time
// Compute in Linear Diffusion Transformer" (research notes), model architecture, QK Norm).
//
// Because the row scale r = 1/sqrt(mean x^2 + eps) is positive, phi(x) = r * ReLU(x * g) and the
// scale can be applied either before or after the ReLU; the kernels use r * x * g then ReLU.
//
// Pipeline (one stream, four launches):
//   rowstats   r_k[b,n] for every K row (needs the whole 2240-channel row)
//   kv_partial per (b, head pair, token chunk): partial S (32x32) and z (32) in fp32;
//              bf16 path on MFMA v_mfma_f32_32x32x16_bf16 with phi split into bf16 hi + lo
//   kv_reduce  per (b, head): fixed-order sum over chunks -> S, z (fp32) and, for the bf16 path,
//              S as bf16 hi/lo operands laid out for the output kernel's MFMA
//   out        per (b, token tile): r_q from the full Q rows held in registers, then per head
//              O^T = S^T phi(Q)^T on v_mfma_f32_16x16x32_bf16, den = phi(Q).z in fp32 VALU.
#include "common.h"

#include <algorithm>
#include <cstdlib>

namespace sanala {

constexpr int kPartStride = kHeadDim * kHeadDim + kHeadDim;  // 1056 floats: S row-major then z

// ---------------------------------------------------------------------------------------------
// Row statistics: r[row] = 1 / sqrt(mean_c x[row, c]^2 + eps), one wave per row.
// ---------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void rowstats_kernel(const T* __restrict__ x, int64_t ld, int64_t rows,
                                                       int C, float eps, float* __restrict__ r) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const char* p = reinterpret_cast<const char*>(x + row * ld);
  const int nvec = C * (int)sizeof(T) / 16;
  float ss = 0.f;
  for (int i = lane; i < nvec; i += 64) {
    const u32x4 w = load16(p + 16 * (int64_t)i);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float a = bf16_lo(w[u]), b = bf16_hi(w[u]);
        ss += a * a + b * b;
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float a = __uint_as_float(w[u]);
        ss += a * a;
      }
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) r[row] = 1.0f / sqrtf(ss / (float)C + eps);
}

// ---------------------------------------------------------------------------------------------
// Split-N KV partial state, bf16 storage, MFMA.
// Block = 4 waves; block (c, p, b) owns heads 2p, 2p+1 and tokens [c*Tc, min(N, (c+1)*Tc)).
// Wave w: head 2p + (w & 1), token half (w >> 1) of each 64-token sub-block.
// MFMA 32x32x16: A[d][t] = phi(K)[t][d] (lane d + 32*g holds tokens 8g..8g+7), B[t][e] = V[t][e].
// ---------------------------------------------------------------------------------------------
template <bool NORM>
__global__ __launch_bounds__(256) void kv_partial_bf16(const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v, int64_t ld,
                                                       const float* __restrict__ r_k,
                                                       const float* __restrict__ gk, int N, int H,
                                                       int Tc, int NC, float* __restrict__ part) {
  constexpr int PITCH = 72;  // bf16 per staged row (64 used)
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * PITCH];
  __shared__ float rs[64];
  __shared__ float red[2][64 * 17];

  const int c = blockIdx.x, p = blockIdx.y, b = blockIdx.z;
  const int h0 = 2 * p;
  const int nh = min(2, H - h0);
  const int n_begin = c * Tc;
  const int n_end = min(N, n_begin + Tc);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int hh = w & 1, th = w >> 1;
  const int d = lane & 31, grp = lane >> 5;
  const bool head_ok = hh < nh;
  const float g = (NORM && head_ok) ? gk[(h0 + hh) * kHeadDim + d] : 1.0f;
  const int64_t row0 = (int64_t)b * N;

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  float zacc = 0.f;

  for (int n0 = n_begin; n0 < n_end; n0 += 64) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int i = tid + it * 256;
      const int row = i >> 3, cu = i & 7;  // cu: 16-byte unit of the 128-byte head pair
      const int n = n0 + row;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (n < n_end && (cu >> 2) < nh) {
        const int64_t off = (row0 + n) * ld + h0 * kHeadDim + cu * 8;
        kv = load16(k + off);
        vv = load16(v + off);
      }
      store16(&Ks[row * PITCH + cu * 8], kv);
      store16(&Vs[row * PITCH + cu * 8], vv);
    }
    if (tid < 64) {
      const int n = n0 + tid;
      rs[tid] = (NORM && n < n_end) ? r_k[row0 + n] : 1.0f;  // rows past the end are zero anyway
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int tb = 32 * th + 16 * s + 8 * grp;  // this lane's tokens tb .. tb+7
      uint32_t ahi[4], alo[4], bw[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const int t0 = tb + j, t1 = tb + j + 1;
        float k0 = __uint_as_float((uint32_t)Ks[t0 * PITCH + hh * kHeadDim + d] << 16);
        float k1 = __uint_as_float((uint32_t)Ks[t1 * PITCH + hh * kHeadDim + d] << 16);
        if (NORM) {
          k0 = k0 * rs[t0] * g;
          k1 = k1 * rs[t1] * g;
        }
        k0 = fmaxf(k0, 0.f);
        k1 = fmaxf(k1, 0.f);
        zacc += k0 + k1;
        const float h0f = round_bf16(k0), h1f = round_bf16(k1);
        ahi[j / 2] = pack_bf16x2(h0f, h1f);
        alo[j / 2] = pack_bf16x2(k0 - h0f, k1 - h1f);
        bw[j / 2] = (uint32_t)Vs[t0 * PITCH + hh * kHeadDim + d] |
                    ((uint32_t)Vs[t1 * PITCH + hh * kHeadDim + d] << 16);
      }
      const bf16x8 A_hi = as_bf16x8(u32x4{ahi[0], ahi[1], ahi[2], ahi[3]});
      const bf16x8 Bv = as_bf16x8(u32x4{bw[0], bw[1], bw[2], bw[3]});
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A_hi, Bv, acc, 0, 0, 0);
      if (NORM) {
        const bf16x8 A_lo = as_bf16x8(u32x4{alo[0], alo[1], alo[2], alo[3]});
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A_lo, Bv, acc, 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // Combine the two token halves of each head in a fixed order: wave hh + 2 hands over to wave hh.
  if (th == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[hh][lane * 17 + r] = acc[r];
    red[hh][lane * 17 + 16] = zacc;
  }
  __syncthreads();
  if (th == 0 && head_ok) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += red[hh][lane * 17 + r];
    zacc += red[hh][lane * 17 + 16];
    zacc += __shfl_xor(zacc, 32);  // lanes d and d + 32 hold the two token octets of dim d
    const int h = h0 + hh;
    float* dst = part + (((int64_t)b * H + h) * NC + c) * kPartStride;
    // accumulator layout: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * grp + (r & 3);
      dst[row * kHeadDim + d] = acc[r];
    }
    if (grp == 0) dst[kHeadDim * kHeadDim + d] = zacc;
  }
}

// ---------------------------------------------------------------------------------------------
// Split-N KV partial state, fp32 storage, fp32 VALU (the fp32-I/O path).
// Block (c, h, b), 256 threads; thread owns S[d][e0..e0+3], d = tid/8, e0 = 4*(tid%8).
// ---------------------------------------------------------------------------------------------
template <bool NORM>
__global__ __launch_bounds__(256) void kv_partial_f32(const float* __restrict__ k, const float* __restrict__ v,
                                                      int64_t ld, const float* __restrict__ r_k,
                                                      const float* __restrict__ gk, int N, int H, int Tc,
                                                      int NC, float* __restrict__ part) {
  __shared__ float Kf[64][kHeadDim + 1];
  __shared__ float Vf[64][kHeadDim + 1];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n_begin = c * Tc;
  const int n_end = min(N, n_begin + Tc);
  const int tid = threadIdx.x;
  const int d = tid >> 3, e0 = (tid & 7) * 4;
  const int64_t row0 = (int64_t)b * N;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float zacc = 0.f;
  for (int n0 = n_begin; n0 < n_end; n0 += 64) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int i = tid + it * 256;
      const int row = i >> 3, c4 = (i & 7) * 4;
      const int n = n0 + row;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (n < n_end) {
        const int64_t off = (row0 + n) * ld + h * kHeadDim + c4;
        kv = loadf4(k + off);
        vv = loadf4(v + off);
        const float r = NORM ? r_k[row0 + n] : 1.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float gg = NORM ? gk[h * kHeadDim + c4 + u] : 1.f;
          kv[u] = fmaxf(NORM ? kv[u] * r * gg : kv[u], 0.f);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        Kf[row][c4 + u] = kv[u];
        Vf[row][c4 + u] = vv[u];
      }
    }
    __syncthreads();
    const int cnt = min(64, n_end - n0);
    for (int t = 0; t < cnt; ++t) {
      const float kd = Kf[t][d];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = fmaf(kd, Vf[t][e0 + u], acc[u]);
      zacc += kd;
    }
    __syncthreads();
  }
  float* dst = part + (((int64_t)b * H + h) * NC + c) * kPartStride;
#pragma unroll
  for (int u = 0; u < 4; ++u) dst[d * kHeadDim + e0 + u] = acc[u];
  if ((tid & 7) == 0) dst[kHeadDim * kHeadDim + d] = zacc;
}

// ---------------------------------------------------------------------------------------------
// Fixed-order reduction over the NC chunks of each (b, h).  Writes S (fp32, row-major [d][e]),
// z (fp32) and, when Sop is given, S as bf16 hi/lo A-operands of v_mfma_f32_16x16x32_bf16 in the
// layout the output kernel loads: block (eb, hl) of 64 lanes x 8 bf16; lane l = m + 16*kg holds
// S[8*kg + j][e(eb, m)] for j = 0..7, with e(eb, m) = 8*(m/4) + 4*eb + m%4.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kv_reduce(const float* __restrict__ part, int NC, int H,
                                                 float* __restrict__ S32, float* __restrict__ z,
                                                 uint16_t* __restrict__ Sop) {
  __shared__ float Sf[kPartStride];
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t bh = (int64_t)b * H + h;
  const float* src = part + bh * NC * kPartStride;
  for (int i = threadIdx.x; i < kPartStride; i += 256) {
    float s = 0.f;
    for (int c = 0; c < NC; ++c) s += src[(int64_t)c * kPartStride + i];
    Sf[i] = s;
    if (i < kHeadDim * kHeadDim) S32[bh * kHeadDim * kHeadDim + i] = s;
    else z[bh * kHeadDim + (i - kHeadDim * kHeadDim)] = s;
  }
  if (Sop == nullptr) return;
  __syncthreads();
  const int t = threadIdx.x;
  const int eb = t >> 7, hl = (t >> 6) & 1, l = t & 63;
  const int m = l & 15, kg = l >> 4;
  const int e = 8 * (m >> 2) + 4 * eb + (m & 3);
  uint32_t wd[4];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    float s0 = Sf[(8 * kg + j) * kHeadDim + e];
    float s1 = Sf[(8 * kg + j + 1) * kHeadDim + e];
    if (hl) {
      s0 -= round_bf16(s0);
      s1 -= round_bf16(s1);
    }
    wd[j / 2] = pack_bf16x2(s0, s1);
  }
  store16(Sop + (bh * 4 + eb * 2 + hl) * 512 + l * 8, u32x4{wd[0], wd[1], wd[2], wd[3]});
}

// ---------------------------------------------------------------------------------------------
// Output, bf16 storage.  Block = 4 waves over a tile of 16*TG tokens of sample b and a group of up
// to 4*HPW heads (blockIdx.z); wave w owns heads [g0 + w*HPW, g0 + w*HPW + HPW).  Lane l = t + 16*kg
// holds dims 8kg..8kg+7 of token t for each of its heads (one 16-byte load), which is exactly the B
// operand of v_mfma_f32_16x16x32_bf16 for O^T = S^T phi^T.  The result lane (t, kg) receives
// channels 8kg..8kg+7 of token t: one 16-byte store.
// PRE_R = false: the block covers all H heads and forms r_q from the Q rows it holds in registers.
// PRE_R = true: r_q comes from a row-statistics pass (used when H > 4*HPW).
// ---------------------------------------------------------------------------------------------
template <int HPW, int TG, bool NORM, bool PRE_R>
__global__ __launch_bounds__(256) void out_bf16(const uint16_t* __restrict__ q, int64_t ldq,
                                                const float* __restrict__ gq, const uint16_t* __restrict__ Sop,
                                                const float* __restrict__ zg, const float* __restrict__ r_q,
                                                int N, int H, float eps, float inv_C, uint16_t* __restrict__ out,
                                                int64_t ldo) {
  __shared__ float ssq[4][16 * TG];
  const int b = blockIdx.y;
  const int n0 = blockIdx.x * 16 * TG;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int t = lane & 15, kg = lane >> 4;
  const int hbeg = blockIdx.z * 4 * HPW + w * HPW;
  const int hcnt = max(0, min(HPW, H - hbeg));
  const int64_t row0 = (int64_t)b * N;

  u32x4 qr[TG][HPW];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int n = n0 + 16 * tg + t;
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
      u32x4 val = {0u, 0u, 0u, 0u};
      if (i < hcnt && n < N) val = load16(q + (row0 + n) * ldq + (hbeg + i) * kHeadDim + kg * 8);
      qr[tg][i] = val;
    }
  }
  float r[TG];
  if (NORM && PRE_R) {
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const int n = n0 + 16 * tg + t;
      r[tg] = n < N ? r_q[row0 + n] : 0.f;
    }
  } else if (NORM) {
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < HPW; ++i) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float a = bf16_lo(qr[tg][i][u]), c2 = bf16_hi(qr[tg][i][u]);
          ss += a * a + c2 * c2;
        }
      }
      ss = sum_over_lane_groups(ss);
      if (kg == 0) ssq[w][16 * tg + t] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const int j = 16 * tg + t;
      const float tot = ((ssq[0][j] + ssq[1][j]) + ssq[2][j]) + ssq[3][j];
      r[tg] = 1.0f / sqrtf(tot * inv_C + eps);
    }
  } else {
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) r[tg] = 1.f;
  }

#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    if (i < hcnt) {
    const int h = hbeg + i;
    const int64_t bh = (int64_t)b * H + h;
    float gv[8], zv[8];
    if (NORM) {
      const f32x4 g0 = loadf4(gq + h * kHeadDim + kg * 8), g1 = loadf4(gq + h * kHeadDim + kg * 8 + 4);
#pragma unroll
      for (int u = 0; u < 4; ++u) { gv[u] = g0[u]; gv[4 + u] = g1[u]; }
    }
    {
      const f32x4 z0 = loadf4(zg + bh * kHeadDim + kg * 8), z1 = loadf4(zg + bh * kHeadDim + kg * 8 + 4);
#pragma unroll
      for (int u = 0; u < 4; ++u) { zv[u] = z0[u]; zv[4 + u] = z1[u]; }
    }
    const uint16_t* sb = Sop + bh * 4 * 512 + lane * 8;
    const bf16x8 a00 = as_bf16x8(load16(sb)), a01 = as_bf16x8(load16(sb + 512));
    const bf16x8 a10 = as_bf16x8(load16(sb + 1024)), a11 = as_bf16x8(load16(sb + 1536));
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      uint32_t bw[4];
      float den = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float x0 = bf16_lo(qr[tg][i][u]), x1 = bf16_hi(qr[tg][i][u]);
        if (NORM) {
          x0 = x0 * r[tg] * gv[2 * u];
          x1 = x1 * r[tg] * gv[2 * u + 1];
        }
        x0 = round_bf16(fmaxf(x0, 0.f));
        x1 = round_bf16(fmaxf(x1, 0.f));
        den = fmaf(x0, zv[2 * u], den);
        den = fmaf(x1, zv[2 * u + 1], den);
        bw[u] = (__float_as_uint(x0) >> 16) | (__float_as_uint(x1) & 0xffff0000u);
      }
      den = sum_over_lane_groups(den);
      const bf16x8 Bq = as_bf16x8(u32x4{bw[0], bw[1], bw[2], bw[3]});
      f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
      o0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a00, Bq, o0, 0, 0, 0);
      o0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a01, Bq, o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a10, Bq, o1, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a11, Bq, o1, 0, 0, 0);
      const float dd = den + eps;
      const int n = n0 + 16 * tg + t;
      if (n < N) {
        const u32x4 pk = {pack_bf16x2(o0[0] / dd, o0[1] / dd), pack_bf16x2(o0[2] / dd, o0[3] / dd),
                          pack_bf16x2(o1[0] / dd, o1[1] / dd), pack_bf16x2(o1[2] / dd, o1[3] / dd)};
        store16(out + (row0 + n) * ldo + h * kHeadDim + kg * 8, pk);
      }
    }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Output, fp32 storage, fp32 VALU.  Block = 4 waves, one token per wave; the token's phi(Q) row is
// staged in LDS, then lane (h parity, e) computes one output channel per head pair.
// ---------------------------------------------------------------------------------------------
template <bool NORM>
__global__ __launch_bounds__(256) void out_f32(const float* __restrict__ q, int64_t ldq, const float* __restrict__ gq,
                                               const float* __restrict__ S32, const float* __restrict__ zg,
                                               int N, int H, float eps, float* __restrict__ out, int64_t ldo) {
  extern __shared__ float qs[];  // [4][C]
  const int C = H * kHeadDim;
  const int b = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + w;
  const bool valid = n < N;
  const int64_t row = (int64_t)b * N + n;
  float* qw = qs + w * C;
  float ss = 0.f;
  if (valid) {
    for (int c4 = lane * 4; c4 < C; c4 += 256) {
      const f32x4 x = loadf4(q + row * ldq + c4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        qw[c4 + u] = x[u];
        ss += x[u] * x[u];
      }
    }
  }
  ss = wave_sum(ss);
  const float r = NORM ? 1.0f / sqrtf(ss / (float)C + eps) : 1.f;
  __syncthreads();
  if (valid) {
    for (int c = lane; c < C; c += 64) {
      const float x = NORM ? qw[c] * r * gq[c] : qw[c];
      qw[c] = fmaxf(x, 0.f);
    }
  }
  __syncthreads();
  if (!valid) return;
  const int e = lane & 31;
  for (int hp = 0; 2 * hp < H; ++hp) {
    const int h = 2 * hp + (lane >> 5);
    if (h >= H) continue;
    const int64_t bh = (int64_t)b * H + h;
    const float* S = S32 + bh * kHeadDim * kHeadDim;
    const float* zz = zg + bh * kHeadDim;
    float num = 0.f, den = 0.f;
#pragma unroll 8
    for (int dd = 0; dd < kHeadDim; ++dd) {
      const float pq = qw[h * kHeadDim + dd];
      num = fmaf(pq, S[dd * kHeadDim + e], num);
      den = fmaf(pq, zz[dd], den);
    }
    out[row * ldo + h * kHeadDim + e] = num / (den + eps);
  }
}

// ---------------------------------------------------------------------------------------------
// Host side: plan and launch.
// ---------------------------------------------------------------------------------------------
static int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  const int v = std::atoi(s);
  return v > 0 ? v : dflt;
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

AttnPlan plan_attn(int B, int N, int H, int dtype, bool norm) {
  AttnPlan p{};
  p.B = B;
  p.N = N;
  p.H = H;
  p.dtype = dtype;
  p.norm = norm;
  const int groups = dtype == kDtypeBf16 ? (H + 1) / 2 : H;
  const int64_t per_chunk = (int64_t)B * groups;
  int nc = (int)std::max<int64_t>(1, (1024 + per_chunk - 1) / per_chunk);
  const int n64 = (N + 63) / 64 * 64;
  int Tc = ((N + nc - 1) / nc + 63) / 64 * 64;
  Tc = std::max(Tc, std::min(256, n64));
  Tc = env_int("SANA_KV_CHUNK", Tc);
  Tc = std::max(64, (Tc + 63) / 64 * 64);
  p.Tc = Tc;
  p.NC = (N + Tc - 1) / Tc;
  const size_t BH = (size_t)B * H;
  size_t off = 0;
  p.off_rk = off;   off = align_up(off + (norm ? (size_t)B * N * 4 : 0), 256);
  p.off_rq = off;   off = align_up(off + (norm && dtype == kDtypeBf16 && H > 72 ? (size_t)B * N * 4 : 0), 256);
  p.off_part = off; off = align_up(off + BH * p.NC * kPartStride * 4, 256);
  p.off_S32 = off;  off = align_up(off + BH * kHeadDim * kHeadDim * 4, 256);
  p.off_z = off;    off = align_up(off + BH * kHeadDim * 4, 256);
  p.off_Sop = off;  off = align_up(off + (dtype == kDtypeBf16 ? BH * 2048 * 2 : 0), 256);
  p.ws_bytes = off;
  return p;
}

hipError_t launch_attn(const AttnPlan& p, const void* q, int64_t ldq, const void* k, const void* v, int64_t ldkv,
                       const float* gq, const float* gk, float eps, void* out, int64_t ldo, void* ws,
                       hipStream_t stream) {
  char* base = static_cast<char*>(ws);
  float* r_k = reinterpret_cast<float*>(base + p.off_rk);
  float* part = reinterpret_cast<float*>(base + p.off_part);
  float* S32 = reinterpret_cast<float*>(base + p.off_S32);
  float* z = reinterpret_cast<float*>(base + p.off_z);
  uint16_t* Sop = reinterpret_cast<uint16_t*>(base + p.off_Sop);
  const int B = p.B, N = p.N, H = p.H, C = H * kHeadDim;
  const int64_t rows = (int64_t)B * N;
  const bool bf = p.dtype == kDtypeBf16;

  if (p.norm) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (bf)
      rowstats_kernel<uint16_t><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(k), ldkv, rows, C, eps, r_k);
    else
      rowstats_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(k), ldkv, rows, C, eps, r_k);
  }
  if (bf) {
    const dim3 grid(p.NC, (H + 1) / 2, B);
    if (p.norm)
      kv_partial_bf16<true><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                                                      ldkv, r_k, gk, N, H, p.Tc, p.NC, part);
    else
      kv_partial_bf16<false><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                                                       ldkv, nullptr, nullptr, N, H, p.Tc, p.NC, part);
  } else {
    const dim3 grid(p.NC, H, B);
    if (p.norm)
      kv_partial_f32<true><<<grid, 256, 0, stream>>>(static_cast<const float*>(k), static_cast<const float*>(v), ldkv,
                                                     r_k, gk, N, H, p.Tc, p.NC, part);
    else
      kv_partial_f32<false><<<grid, 256, 0, stream>>>(static_cast<const float*>(k), static_cast<const float*>(v), ldkv,
                                                      nullptr, nullptr, N, H, p.Tc, p.NC, part);
  }
  kv_reduce<<<dim3(H, B), 256, 0, stream>>>(part, p.NC, H, S32, z, bf ? Sop : nullptr);
  if (bf) {
    constexpr int HPW = 18, TG = 1;
    const float inv_C = 1.0f / (float)C;
    const auto* qb = static_cast<const uint16_t*>(q);
    auto* ob = static_cast<uint16_t*>(out);
    if (H <= 4 * HPW) {
      const dim3 grid((N + 16 * TG - 1) / (16 * TG), B, 1);
      if (p.norm)
        out_bf16<HPW, TG, true, false><<<grid, 256, 0, stream>>>(qb, ldq, gq, Sop, z, nullptr, N, H, eps, inv_C, ob, ldo);
      else
        out_bf16<HPW, TG, false, false><<<grid, 256, 0, stream>>>(qb, ldq, nullptr, Sop, z, nullptr, N, H, eps, inv_C,
                                                                   ob, ldo);
    } else {
      const dim3 grid((N + 16 * TG - 1) / (16 * TG), B, (H + 4 * HPW - 1) / (4 * HPW));
      float* r_q = reinterpret_cast<float*>(base + p.off_rq);
      if (p.norm) {
        rowstats_kernel<uint16_t><<<dim3((unsigned)((rows + 3) / 4)), 256, 0, stream>>>(qb, ldq, rows, C, eps, r_q);
        out_bf16<HPW, TG, true, true><<<grid, 256, 0, stream>>>(qb, ldq, gq, Sop, z, r_q, N, H, eps, inv_C, ob, ldo);
      } else {
        out_bf16<HPW, TG, false, true><<<grid, 256, 0, stream>>>(qb, ldq, nullptr, Sop, z, nullptr, N, H, eps, inv_C,
                                                                  ob, ldo);
      }
    }
  } else {
    const dim3 grid((N + 3) / 4, B);
    const size_t lds = (size_t)4 * C * sizeof(float);
    if (p.norm)
      out_f32<true><<<grid, 256, lds, stream>>>(static_cast<const float*>(q), ldq, gq, S32, z, N, H, eps,
                                                static_cast<float*>(out), ldo);
    else
      out_f32<false><<<grid, 256, lds, stream>>>(static_cast<const float*>(q), ldq, nullptr, S32, z, N, H, eps,
                                                 static_cast<float*>(out), ldo);
  }
  return hipGetLastError();
}

int out_bf16_max_heads() { return 320; }  // fp32 output kernel stages 4 rows of C floats in LDS

}  // namespace sanala

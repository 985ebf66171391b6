// fp32-storage path of the linear attention (fp32 arithmetic throughout, on the VALU).
//
// "Sana: Efficient High-Resolution Image Synthesis with Linear Diffusion Transformers" (paper notes),
// section 2.1, Eq. (1), per head, in the precompute-then-apply order the notes give after Eq. (1);
// phi(x) = ReLU(x / sqrt(mean_c x_c^2 + eps) * g) over all channels of a token ("SANA 1.5: Efficient
// Scaling of Training-Time and Inference-Time Compute in Linear Diffusion Transformer" (research
// notes), model architecture, QK Norm).
//
// Launches: rowstats (r_k and r_q), kv_partial_f32 (per chunk), kv_reduce_f32 (chunk order; only when a
// sample spans several chunks), out_f32.
#include "rowstats.h"

namespace sanala {

// Split-N KV partial state.  Block (c, h, b), 4 waves; the phi(K) and V rows of 64 tokens are staged in
// LDS (the next 64 tokens' loads in flight while the current ones are summed), wave w takes tokens
// w, w + 4, ... of them and lane l owns S[l/2][16*(l%2) .. 16*(l%2) + 15] and z[l/2] (fp32 FMAs in token
// order); at the end the waves' sums are added in wave order.  With one chunk per sample (NC = 1) the
// block writes S and z themselves, and no reduction launch follows.
template <bool NORM>
__global__ __launch_bounds__(256) void kv_partial_f32(const float* __restrict__ k, const float* __restrict__ v,
                                                      int64_t ld, const float* __restrict__ r_k,
                                                      const float* __restrict__ gk, int N, int H, int Tc, int NC,
                                                      float* __restrict__ part, float* __restrict__ S32,
                                                      float* __restrict__ zg) {
  __shared__ float Kf[64][kHeadDim + 1];
  __shared__ __attribute__((aligned(16))) float Vf[64][kHeadDim];
  __shared__ __attribute__((aligned(16))) float red[3][kPartStride];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n_begin = c * Tc;
  const int n_end = min(N, n_begin + Tc);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int d = lane >> 1, e0 = 16 * (lane & 1);
  const int64_t row0 = (int64_t)b * N;
  float acc[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) acc[u] = 0.f;
  float zacc = 0.f;
  f32x4 kv[2], vv[2];
  float rr[2];
  auto load = [&](int n0) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int i = tid + it * 256;
      const int row = i >> 3, c4 = (i & 7) * 4;
      const int n = n0 + row;
      kv[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      vv[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      rr[it] = 0.f;
      if (n < n_end) {
        const int64_t off = (row0 + n) * ld + h * kHeadDim + c4;
        kv[it] = loadf4(k + off);
        vv[it] = loadf4(v + off);
        rr[it] = NORM ? r_k[row0 + n] : 1.f;
      }
    }
  };
  if (n_begin < n_end) load(n_begin);
  for (int n0 = n_begin; n0 < n_end; n0 += 64) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int i = tid + it * 256;
      const int row = i >> 3, c4 = (i & 7) * 4;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float gg = NORM ? gk[h * kHeadDim + c4 + u] : 1.f;
        Kf[row][c4 + u] = fmaxf(NORM ? kv[it][u] * rr[it] * gg : kv[it][u], 0.f);  // rows past the end: 0
      }
      *reinterpret_cast<f32x4*>(&Vf[row][c4]) = vv[it];
    }
    __syncthreads();
    if (n0 + 64 < n_end) load(n0 + 64);
    const int cnt = min(64, n_end - n0);
    for (int t = w; t < cnt; t += 4) {
      const float kd = Kf[t][d];
      const f32x4* vr = reinterpret_cast<const f32x4*>(&Vf[t][e0]);
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        const f32x4 vq = vr[w4];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[4 * w4 + u] = fmaf(kd, vq[u], acc[4 * w4 + u]);
      }
      zacc += kd;
    }
    __syncthreads();
  }
  // waves 1..3 hand their sums to wave 0, which adds them in wave order
  if (w > 0) {
#pragma unroll
    for (int u = 0; u < 16; ++u) red[w - 1][d * kHeadDim + e0 + u] = acc[u];
    if ((lane & 1) == 0) red[w - 1][kHeadDim * kHeadDim + d] = zacc;
  }
  __syncthreads();
  if (w > 0) return;
#pragma unroll
  for (int u = 0; u < 16; ++u)
    acc[u] = ((acc[u] + red[0][d * kHeadDim + e0 + u]) + red[1][d * kHeadDim + e0 + u]) + red[2][d * kHeadDim + e0 + u];
  zacc = ((zacc + red[0][kHeadDim * kHeadDim + d]) + red[1][kHeadDim * kHeadDim + d]) + red[2][kHeadDim * kHeadDim + d];
  const int64_t bh = (int64_t)b * H + h;
  float* Sd = NC == 1 ? S32 + bh * kHeadDim * kHeadDim : part + (bh * NC + c) * kPartStride;
  float* zd = NC == 1 ? zg + bh * kHeadDim : part + (bh * NC + c) * kPartStride + kHeadDim * kHeadDim;
#pragma unroll
  for (int w4 = 0; w4 < 4; ++w4)
    *reinterpret_cast<f32x4*>(Sd + d * kHeadDim + e0 + 4 * w4) =
        f32x4{acc[4 * w4], acc[4 * w4 + 1], acc[4 * w4 + 2], acc[4 * w4 + 3]};
  if ((lane & 1) == 0) zd[d] = zacc;
}

// One thread per state element: sum of the chunk partials in chunk order (deterministic).
__global__ __launch_bounds__(256) void kv_reduce_f32(const float* __restrict__ part, int NC, int64_t BH,
                                                     float* __restrict__ S32, float* __restrict__ zg) {
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gi >= BH * kPartStride) return;
  const int64_t bh = gi / kPartStride;
  const int i = (int)(gi - bh * kPartStride);
  const float* src = part + bh * NC * kPartStride + i;
  float s = 0.f;
  for (int c = 0; c < NC; ++c) s += src[(int64_t)c * kPartStride];
  if (i < kHeadDim * kHeadDim) S32[bh * kHeadDim * kHeadDim + i] = s;
  else zg[bh * kHeadDim + (i - kHeadDim * kHeadDim)] = s;
}

// Output.  Block = 16 tokens x 8 heads (blockIdx.z picks the head group); S and z of the group and the
// block's phi(Q) rows are staged in LDS (phi(q) = ReLU(q * r_q * gq), r_q from the row-statistics
// launch).  Thread (t, h, half) forms output channels 16*half .. 16*half + 15 of token t, head h:
// num_e = sum_d phi_d S[d][e] and den = sum_d phi_d z[d], both fp32 FMAs in order d = 0..31, then
// num / (den + eps).
constexpr int kF32OutHeads = 8;
template <bool NORM>
__global__ __launch_bounds__(256) void out_f32(const float* __restrict__ q, int64_t ldq, const float* __restrict__ gq,
                                               const float* __restrict__ r_q, const float* __restrict__ S32,
                                               const float* __restrict__ zg, int N, int H, float eps,
                                               float* __restrict__ out, int64_t ldo) {
  constexpr int HG = kF32OutHeads;
  __shared__ __attribute__((aligned(16))) float Ss[HG][kHeadDim][kHeadDim];
  __shared__ float Zs[HG][kHeadDim];
  __shared__ float Ps[16][HG][kHeadDim + 1];
  const int b = blockIdx.y, n0 = blockIdx.x * 16, hg0 = blockIdx.z * HG;
  const int nh = min(HG, H - hg0);
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)b * N;
  const int64_t bh0 = (int64_t)b * H + hg0;
  // S, z of the group and phi(Q) of the tile: all loads of a thread issued before its LDS stores.
  f32x4 sreg[HG], qreg[4];
  float zreg = 0.f, rq[4];
#pragma unroll
  for (int j = 0; j < HG; ++j) {
    const int i = tid + 256 * j;  // float4 index into the group's S (256 per head)
    sreg[j] = i < nh * 256 ? loadf4(S32 + bh0 * kHeadDim * kHeadDim + 4 * i) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (tid < nh * kHeadDim) zreg = zg[bh0 * kHeadDim + tid];
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // float4 i: token i / 64, channels 4 * (i % 64) .. of the group's 256
    const int i = tid + 256 * j, t = i >> 6, c4 = 4 * (i & 63);
    const int n = n0 + t;
    const bool ok = n < N && c4 < nh * kHeadDim;
    qreg[j] = ok ? loadf4(q + (row0 + n) * ldq + hg0 * kHeadDim + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
    rq[j] = (NORM && ok) ? r_q[row0 + n] : 1.f;
  }
#pragma unroll
  for (int j = 0; j < HG; ++j) reinterpret_cast<f32x4*>(&Ss[0][0][0])[tid + 256 * j] = sreg[j];
  if (tid < HG * kHeadDim) Zs[tid / kHeadDim][tid % kHeadDim] = zreg;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + 256 * j, t = i >> 6, c4 = 4 * (i & 63);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cc = c4 + u;
      const float g = (NORM && cc < nh * kHeadDim) ? gq[hg0 * kHeadDim + cc] : 1.f;
      Ps[t][cc / kHeadDim][cc % kHeadDim] = fmaxf(NORM ? qreg[j][u] * rq[j] * g : qreg[j][u], 0.f);
    }
  }
  __syncthreads();
  const int t = tid >> 4, hl = (tid >> 1) & 7, half = tid & 1;
  const int n = n0 + t;
  if (n >= N || hl >= nh) return;
  float num[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) num[u] = 0.f;
  float den = 0.f;
#pragma unroll 4
  for (int dd = 0; dd < kHeadDim; ++dd) {
    const float pq = Ps[t][hl][dd];
    const f32x4* srow = reinterpret_cast<const f32x4*>(&Ss[hl][dd][16 * half]);
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      const f32x4 sv = srow[w4];
#pragma unroll
      for (int u = 0; u < 4; ++u) num[4 * w4 + u] = fmaf(pq, sv[u], num[4 * w4 + u]);
    }
    den = fmaf(pq, Zs[hl][dd], den);
  }
  const float dv = den + eps;
  float* o = out + (row0 + n) * ldo + (hg0 + hl) * kHeadDim + 16 * half;
#pragma unroll
  for (int w4 = 0; w4 < 4; ++w4)
    *reinterpret_cast<f32x4*>(o + 4 * w4) =
        f32x4{num[4 * w4] / dv, num[4 * w4 + 1] / dv, num[4 * w4 + 2] / dv, num[4 * w4 + 3] / dv};
}

hipError_t launch_attn_f32(const AttnPlan& p, const float* q, int64_t ldq, const float* k, const float* v,
                           int64_t ldkv, const float* gq, const float* gk, float eps, float* out, int64_t ldo,
                           void* ws, hipStream_t stream) {
  char* base = static_cast<char*>(ws);
  float* r_k = reinterpret_cast<float*>(base + p.off_rk);
  float* r_q = reinterpret_cast<float*>(base + p.off_rq);
  float* part = reinterpret_cast<float*>(base + p.off_part);
  float* S32 = reinterpret_cast<float*>(base + p.off_S32);
  float* z = reinterpret_cast<float*>(base + p.off_z);
  const int B = p.B, N = p.N, H = p.H, C = H * kHeadDim;
  const int64_t rows = (int64_t)B * N;
  if (p.norm)  // r_k and r_q in one launch
    launch_kernel("rowstats_kq", rowstats_kernel<float>, (unsigned)((2 * rows + 3) / 4), 256, 0, stream, k, ldkv, rows,
                  C, eps, r_k, q, ldq, r_q);
  const dim3 grid(p.NC, H, B);
  if (p.norm)
    launch_kernel("kv_partial", kv_partial_f32<true>, grid, 256, 0, stream, k, v, ldkv, r_k, gk, N, H, p.Tc, p.NC,
                  part, S32, z);
  else
    launch_kernel("kv_partial", kv_partial_f32<false>, grid, 256, 0, stream, k, v, ldkv, nullptr, nullptr, N, H, p.Tc,
                  p.NC, part, S32, z);
  if (p.NC > 1) {
    const int64_t elems = (int64_t)B * H * kPartStride;
    launch_kernel("kv_reduce", kv_reduce_f32, (unsigned)((elems + 255) / 256), 256, 0, stream, part, p.NC,
                  (int64_t)B * H, S32, z);
  }
  const dim3 ogrid((N + 15) / 16, B, (H + kF32OutHeads - 1) / kF32OutHeads);
  final_launch();
  if (p.norm)
    launch_kernel("out", out_f32<true>, ogrid, 256, 0, stream, q, ldq, gq, r_q, S32, z, N, H, eps, out, ldo);
  else
    launch_kernel("out", out_f32<false>, ogrid, 256, 0, stream, q, ldq, nullptr, nullptr, S32, z, N, H, eps, out, ldo);
  return hipGetLastError();
}

}  // namespace sanala

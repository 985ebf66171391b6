// fp32-storage path of the linear attention (fp32 arithmetic throughout, on the VALU).
//
// "Sana: Efficient High-Resolution Image Synthesis with Linear Diffusion Transformers" (paper notes),
// section 2.1, Eq. (1), per head, in the precompute-then-apply order the notes give after Eq. (1);
// phi(x) = ReLU(x / sqrt(mean_c x_c^2 + eps) * g) over all channels of a token ("SANA 1.5: Efficient
// Scaling of Training-Time and Inference-Time Compute in Linear Diffusion Transformer" (research
// notes), model architecture, QK Norm).
//
// Launches: rowstats (r_k), kv_partial_f32 (per chunk), kv_reduce_f32 (chunk order), out_f32.
#include "rowstats.h"

namespace sanala {

// Split-N KV partial state.  Block (c, h, b), 256 threads; thread owns S[d][e0..e0+3], d = tid/8,
// e0 = 4*(tid%8); phi(K) and V rows of 64 tokens are staged in LDS.
template <bool NORM>
__global__ __launch_bounds__(256) void kv_partial_f32(const float* __restrict__ k, const float* __restrict__ v,
                                                      int64_t ld, const float* __restrict__ r_k,
                                                      const float* __restrict__ gk, int N, int H, int Tc, int NC,
                                                      float* __restrict__ part) {
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

// Output.  Block = 4 waves, one token per wave; the token's phi(Q) row is staged in LDS, then lane
// (h parity, e) computes one output channel per head pair: phi(Q) S[:, e] / (phi(Q).z + eps).
template <bool NORM>
__global__ __launch_bounds__(256) void out_f32(const float* __restrict__ q, int64_t ldq, const float* __restrict__ gq,
                                               const float* __restrict__ S32, const float* __restrict__ zg, int N,
                                               int H, float eps, float* __restrict__ out, int64_t ldo) {
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
        ss = fmaf(x[u], x[u], ss);
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

hipError_t launch_attn_f32(const AttnPlan& p, const float* q, int64_t ldq, const float* k, const float* v,
                           int64_t ldkv, const float* gq, const float* gk, float eps, float* out, int64_t ldo,
                           void* ws, hipStream_t stream) {
  char* base = static_cast<char*>(ws);
  float* r_k = reinterpret_cast<float*>(base + p.off_rk);
  float* part = reinterpret_cast<float*>(base + p.off_part);
  float* S32 = reinterpret_cast<float*>(base + p.off_S32);
  float* z = reinterpret_cast<float*>(base + p.off_z);
  const int B = p.B, N = p.N, H = p.H, C = H * kHeadDim;
  const int64_t rows = (int64_t)B * N;
  if (p.norm)
    launch_kernel("rowstats_k", rowstats_kernel<float>, (unsigned)((rows + 3) / 4), 256, 0, stream, k, ldkv, rows, C,
                  eps, r_k, nullptr, 0, nullptr);
  const dim3 grid(p.NC, H, B);
  if (p.norm)
    launch_kernel("kv_partial", kv_partial_f32<true>, grid, 256, 0, stream, k, v, ldkv, r_k, gk, N, H, p.Tc, p.NC,
                  part);
  else
    launch_kernel("kv_partial", kv_partial_f32<false>, grid, 256, 0, stream, k, v, ldkv, nullptr, nullptr, N, H, p.Tc,
                  p.NC, part);
  const int64_t elems = (int64_t)B * H * kPartStride;
  launch_kernel("kv_reduce", kv_reduce_f32, (unsigned)((elems + 255) / 256), 256, 0, stream, part, p.NC, (int64_t)B * H,
                S32, z);
  const dim3 ogrid((N + 3) / 4, B);
  const size_t lds = (size_t)4 * C * sizeof(float);  // up to 160 KB at H = 320
  if (lds > 64 * 1024) {
    const hipError_t ea = p.norm ? ensure_max_lds(reinterpret_cast<const void*>(&out_f32<true>), (int)lds)
                                 : ensure_max_lds(reinterpret_cast<const void*>(&out_f32<false>), (int)lds);
    if (ea != hipSuccess) return ea;
  }
  if (p.norm)
    launch_kernel("out", out_f32<true>, ogrid, 256, lds, stream, q, ldq, gq, S32, z, N, H, eps, out, ldo);
  else
    launch_kernel("out", out_f32<false>, ogrid, 256, lds, stream, q, ldq, nullptr, S32, z, N, H, eps, out, ldo);
  return hipGetLastError();
}

}  // namespace sanala

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

// Split-N KV partial state.  Block (c, h, b) of kF32StateWaves waves; the chunk is taken in sub-blocks
// of 64 tokens whose phi(K) and V rows are staged in LDS (two buffers), with the loads of the next
// kF32Ring sub-blocks in flight in registers, so a short chunk costs one memory round trip rather than
// one per sub-block.  Wave w takes tokens w, w + W, ... of a sub-block; lane l owns the 4 x 4 block
// S[4*(l/8) + i][4*(l%8) + j] and z[4*(l/8) + i], so a token costs each lane two 16-byte LDS reads
// (four phi(k) values, four v values) for its 16 FMAs (fp32, in token order per element); at the end
// the waves' sums are added in wave order.  With one chunk per sample (NC = 1) the block writes S and
// z themselves, and no reduction launch follows.
constexpr int kF32Ring = 4;
constexpr int kF32StateWaves = 8;
template <bool NORM>
__global__ __launch_bounds__(64 * kF32StateWaves) void kv_partial_f32(
    const float* __restrict__ k, const float* __restrict__ v, int64_t ld, const float* __restrict__ r_k,
    const float* __restrict__ gk, int N, int H, int Tc, int NC, float* __restrict__ part, float* __restrict__ S32,
    float* __restrict__ zg) {
  constexpr int R = kF32Ring;
  constexpr int W = kF32StateWaves, NT = 64 * W, LD = 512 / NT;  // float4s of K (and of V) per thread
  __shared__ __attribute__((aligned(16))) float Kf[2][64][kHeadDim];
  __shared__ __attribute__((aligned(16))) float Vf[2][64][kHeadDim];
  // wave w's sums: piece i of lane l (its S row 4*(l/8) + i) at 256*i + 4*l, z at 1024
  __shared__ __attribute__((aligned(16))) float red[W - 1][kPartStride];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n_begin = c * Tc;
  const int n_end = min(N, n_begin + Tc);
  const int nsub = n_end > n_begin ? (n_end - n_begin + 63) / 64 : 0;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int d4 = 4 * (lane >> 3), e4 = 4 * (lane & 7);
  const int64_t row0 = (int64_t)b * N;
  float gg[4];  // the K gains of this thread's staging columns (the same for each of its float4s)
#pragma unroll
  for (int u = 0; u < 4; ++u) gg[u] = NORM ? gk[h * kHeadDim + (tid & 7) * 4 + u] : 1.f;
  float acc[16];  // acc[4*i + j] = S[d4 + i][e4 + j]
#pragma unroll
  for (int u = 0; u < 16; ++u) acc[u] = 0.f;
  float zacc[4] = {0.f, 0.f, 0.f, 0.f};
  f32x4 kv[R][LD], vv[R][LD];
  float rr[R][LD];
  // sub-block j of the chunk into ring slot s (rows past the chunk end: zeros)
  auto load = [&](int s, int j) {
    const int n0 = n_begin + 64 * j;
#pragma unroll
    for (int it = 0; it < LD; ++it) {
      const int i = tid + it * NT;
      const int row = i >> 3, c4 = (i & 7) * 4;
      const int n = n0 + row;
      kv[s][it] = f32x4{0.f, 0.f, 0.f, 0.f};
      vv[s][it] = f32x4{0.f, 0.f, 0.f, 0.f};
      rr[s][it] = 0.f;
      if (n < n_end) {
        const int64_t off = (row0 + n) * ld + h * kHeadDim + c4;
        kv[s][it] = loadf4(k + off);
        vv[s][it] = loadf4(v + off);
        rr[s][it] = NORM ? r_k[row0 + n] : 1.f;
      }
    }
  };
#pragma unroll
  for (int s = 0; s < R; ++s)
    if (s < nsub) load(s, s);
  for (int j0 = 0; j0 < nsub; j0 += R) {
#pragma unroll
    for (int s = 0; s < R; ++s) {
      const int j = j0 + s;  // sub-block; buffer j % 2 = s % 2 (R is even)
      if (j >= nsub) break;
      const int bs = s & 1;
#pragma unroll
      for (int it = 0; it < LD; ++it) {
        const int i = tid + it * NT;
        const int row = i >> 3, c4 = (i & 7) * 4;
        f32x4 kf;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          kf[u] = fmaxf(NORM ? kv[s][it][u] * rr[s][it] * gg[u] : kv[s][it][u], 0.f);  // rows past the end: 0
        *reinterpret_cast<f32x4*>(&Kf[bs][row][c4]) = kf;
        *reinterpret_cast<f32x4*>(&Vf[bs][row][c4]) = vv[s][it];
      }
      // One barrier per sub-block: buffer bs is written again two sub-blocks later, after every wave has
      // passed the next sub-block's barrier and so finished reading it.
      __syncthreads();
      if (j + R < nsub) load(s, j + R);
      const int cnt = min(64, n_end - (n_begin + 64 * j));
#pragma unroll 4
      for (int t = w; t < cnt; t += W) {
        const f32x4 kq = *reinterpret_cast<const f32x4*>(&Kf[bs][t][d4]);
        const f32x4 vq = *reinterpret_cast<const f32x4*>(&Vf[bs][t][e4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[4 * i + jj] = fmaf(kq[i], vq[jj], acc[4 * i + jj]);
          zacc[i] += kq[i];
        }
      }
    }
  }
  // waves 1..W-1 hand their sums to wave 0, which adds them in wave order
  if (w > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<f32x4*>(&red[w - 1][256 * i + 4 * lane]) =
          f32x4{acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
    if (e4 == 0)
      *reinterpret_cast<f32x4*>(&red[w - 1][kHeadDim * kHeadDim + d4]) = f32x4{zacc[0], zacc[1], zacc[2], zacc[3]};
  }
  __syncthreads();
  if (w > 0) return;
#pragma unroll
  for (int r = 0; r < W - 1; ++r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 p = *reinterpret_cast<const f32x4*>(&red[r][256 * i + 4 * lane]);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[4 * i + jj] += p[jj];
    }
    const f32x4 pz = *reinterpret_cast<const f32x4*>(&red[r][kHeadDim * kHeadDim + d4]);
#pragma unroll
    for (int i = 0; i < 4; ++i) zacc[i] += pz[i];
  }
  const int64_t bh = (int64_t)b * H + h;
  float* Sd = NC == 1 ? S32 + bh * kHeadDim * kHeadDim : part + (bh * NC + c) * kPartStride;
  float* zd = NC == 1 ? zg + bh * kHeadDim : part + (bh * NC + c) * kPartStride + kHeadDim * kHeadDim;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<f32x4*>(Sd + (d4 + i) * kHeadDim + e4) =
        f32x4{acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
  if (e4 == 0) *reinterpret_cast<f32x4*>(zd + d4) = f32x4{zacc[0], zacc[1], zacc[2], zacc[3]};
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

// Output.  Block = 16 tokens x 4 heads (blockIdx.z picks the head group), so that even a 256-token
// sample spreads over a few hundred blocks; S and z of the group and the block's phi(Q) rows are staged
// in LDS (phi(q) = ReLU(q * r_q * gq), r_q from the row-statistics launch).  Thread (t, h, qtr) forms
// output channels 8*qtr .. 8*qtr + 7 of token t, head h: num_e = sum_d phi_d S[d][e] and
// den = sum_d phi_d z[d], both fp32 FMAs in order d = 0..31, then num / (den + eps).
//
// LDS layout of S: head h at word h * kF32HeadStride, row d at d * 32 within it, and within a row the
// 16-byte piece w (0, 1) of quarter qtr at word 16*w + 4*qtr.  The 16 lanes that read together (one
// token, 4 heads x 4 quarters) then touch 64 distinct banks: the head stride is 16 words past a multiple
// of 64 and the quarters' pieces are interleaved.  (A plain [h][d][e] layout put all heads of a read on
// the same banks.)
constexpr int kF32OutHeads = 4;
constexpr int kF32HeadStride = kHeadDim * kHeadDim + 16;
template <bool NORM>
__global__ __launch_bounds__(256) void out_f32(const float* __restrict__ q, int64_t ldq, const float* __restrict__ gq,
                                               const float* __restrict__ r_q, const float* __restrict__ S32,
                                               const float* __restrict__ zg, int N, int H, float eps,
                                               float* __restrict__ out, int64_t ldo) {
  constexpr int HG = kF32OutHeads;
  constexpr int GC = HG * kHeadDim;  // channels of the group
  __shared__ __attribute__((aligned(16))) float Ss[HG * kF32HeadStride];
  __shared__ float Zs[HG][kHeadDim + 1];
  __shared__ float Ps[16][HG][kHeadDim + 1];
  const int b = blockIdx.y, n0 = blockIdx.x * 16, hg0 = blockIdx.z * HG;
  const int nh = min(HG, H - hg0);
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)b * N;
  const int64_t bh0 = (int64_t)b * H + hg0;
  // S, z of the group and phi(Q) of the tile: all loads of a thread issued before its LDS stores.
  constexpr int SJ = HG * kHeadDim * kHeadDim / 4 / 256;  // float4s of S per thread
  constexpr int QJ = 16 * GC / 4 / 256;                   // float4s of Q per thread
  f32x4 sreg[SJ], qreg[QJ];
  float zreg = 0.f, rq[QJ];
#pragma unroll
  for (int j = 0; j < SJ; ++j) {
    const int i = tid + 256 * j;  // float4 index into the group's S (256 per head)
    sreg[j] = i < nh * 256 ? loadf4(S32 + bh0 * kHeadDim * kHeadDim + 4 * i) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (tid < nh * kHeadDim) zreg = zg[bh0 * kHeadDim + tid];
#pragma unroll
  for (int j = 0; j < QJ; ++j) {  // float4 i: token i / 32, channels 4 * (i % 32) .. of the group's 128
    const int i = tid + 256 * j, t = i >> 5, c4 = 4 * (i & 31);
    const int n = n0 + t;
    const bool ok = n < N && c4 < nh * kHeadDim;
    qreg[j] = ok ? loadf4(q + (row0 + n) * ldq + hg0 * kHeadDim + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
    rq[j] = (NORM && ok) ? r_q[row0 + n] : 1.f;
  }
#pragma unroll
  for (int j = 0; j < SJ; ++j) {
    const int i = tid + 256 * j, hl = i >> 8, d = (i >> 3) & 31, e4 = i & 7;  // e = 4 * e4 = 8*qtr + 4*w
    *reinterpret_cast<f32x4*>(&Ss[hl * kF32HeadStride + d * kHeadDim + 16 * (e4 & 1) + 4 * (e4 >> 1)]) = sreg[j];
  }
  if (tid < HG * kHeadDim) Zs[tid / kHeadDim][tid % kHeadDim] = zreg;
#pragma unroll
  for (int j = 0; j < QJ; ++j) {
    const int i = tid + 256 * j, t = i >> 5, c4 = 4 * (i & 31);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cc = c4 + u;
      const float g = (NORM && cc < nh * kHeadDim) ? gq[hg0 * kHeadDim + cc] : 1.f;
      Ps[t][cc / kHeadDim][cc % kHeadDim] = fmaxf(NORM ? qreg[j][u] * rq[j] * g : qreg[j][u], 0.f);
    }
  }
  __syncthreads();
  const int t = tid >> 4, hl = (tid >> 2) & 3, qtr = tid & 3;
  const int n = n0 + t;
  if (n >= N || hl >= nh) return;
  float num[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) num[u] = 0.f;
  float den = 0.f;
  const f32x4* srow = reinterpret_cast<const f32x4*>(&Ss[hl * kF32HeadStride + 4 * qtr]);
#pragma unroll 8
  for (int dd = 0; dd < kHeadDim; ++dd) {
    const float pq = Ps[t][hl][dd];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const f32x4 sv = srow[dd * (kHeadDim / 4) + 4 * w];
#pragma unroll
      for (int u = 0; u < 4; ++u) num[4 * w + u] = fmaf(pq, sv[u], num[4 * w + u]);
    }
    den = fmaf(pq, Zs[hl][dd], den);
  }
  const float dv = den + eps;
  float* o = out + (row0 + n) * ldo + (hg0 + hl) * kHeadDim + 8 * qtr;
#pragma unroll
  for (int w = 0; w < 2; ++w)
    *reinterpret_cast<f32x4*>(o + 4 * w) =
        f32x4{num[4 * w] / dv, num[4 * w + 1] / dv, num[4 * w + 2] / dv, num[4 * w + 3] / dv};
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
    launch_kernel("kv_partial", kv_partial_f32<true>, grid, 64 * kF32StateWaves, 0, stream, k, v, ldkv, r_k, gk, N, H, p.Tc, p.NC,
                  part, S32, z);
  else
    launch_kernel("kv_partial", kv_partial_f32<false>, grid, 64 * kF32StateWaves, 0, stream, k, v, ldkv, nullptr, nullptr, N, H, p.Tc,
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

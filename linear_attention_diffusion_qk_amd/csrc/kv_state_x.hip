// KV state of the 16-bit path with the QK-Norm statistics of K formed inside the same pass, so that K
// is read from HBM once.
//
// "Sana: Efficient High-Resolution Image Synthesis with Linear Diffusion Transformers" (paper notes),
// section 2.1, the sums after Eq. (1): S = sum_j phi(K_j)^T V_j and z = sum_j phi(K_j), with
// phi(k) = ReLU(k * r_k * g_k) and r_k = 1/sqrt(mean_c k_c^2 + eps) over all C channels of a token
// ("SANA 1.5: Efficient Scaling of Training-Time and Inference-Time Compute in Linear Diffusion
// Transformer" (research notes), model architecture, QK Norm).
//
// A block owns one head pair of one token chunk (as the plain state kernel does), so r_k of a token
// needs the other head pairs' share of its sum of squares.  The blocks of a chunk exchange them:
//   1. a block reads K of a 64-token sub-block L - 1 steps ahead of its use, keeps it in an LDS ring,
//      and publishes its head pair's partial sum of squares of each token;
//   2. block p of the chunk sums the P partials of tokens p, p + P, ... of a sub-block in pair order
//      and publishes r_k of those tokens;
//   3. every block reads r_k of the sub-block it multiplies.
// Each published value carries the call's epoch in the upper half of a 64-bit word and is written and
// read with single-copy-atomic agent-scope accesses, so a value is either this call's or visibly stale;
// no fences or counters are needed and nothing has to be cleared between calls.  Every wait is bounded
// by a time limit; past it the block forms the missing values itself from the full K rows, with the
// same arithmetic in the same order (head-pair partials from the same per-lane sums and the same
// 8-lane tree, summed in pair order), so the result does not depend on which route was taken.
#include "state_ops.h"

namespace sanala {

namespace {
constexpr int kSB = 64;     // tokens per sub-block
constexpr int kPitch = 72;  // bf16 per staged LDS row (64 used)

__device__ __forceinline__ void put_tagged(uint64_t* p, float x, uint32_t epoch) {
  __hip_atomic_store(p, ((uint64_t)epoch << 32) | __float_as_uint(x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_tagged(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(uint64_t v, uint32_t epoch) { return (uint32_t)(v >> 32) == epoch; }
__device__ __forceinline__ float tagged_value(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }  // 100 MHz
// The same agent-scope (sc1) 8-byte accesses as range-checked buffer operations: a lane whose offset is
// out of range loads zero (tag 0, never an epoch) and stores nothing, so every wave issues the same
// instructions in every step and the compiler's waits count exactly the loads they need.
constexpr int kSc1 = 16;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint64_t buffer_get_tagged(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kSc1);
  return ((uint64_t)x[1] << 32) | x[0];
}
__device__ __forceinline__ void buffer_put_tagged(__amdgpu_buffer_rsrc_t r, uint32_t off, float x, uint32_t epoch) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(x), epoch}, r, off, 0, kSc1);
}

// Sum of squares of one 16-byte unit (8 values, v_dot2 on the packed pairs, in order).
template <bool F16>
__device__ __forceinline__ float unit_ssq(u32x4 w) {
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) ss = dot2_h<F16>(w[u], w[u], ss);
  return ss;
}

// r = 1/sqrt(ss/C + eps) as v_rsq_f32 of ss * (1/C) + eps (about 1 ulp; both routes use it, and a
// relative error near 1e-7 in r is far below what the 16-bit output keeps).
__device__ __forceinline__ float r_from_ssq(float ss, float inv_C, float eps) {
  return __builtin_amdgcn_rsqf(fmaf(ss, inv_C, eps));
}

// The order in which a token's P head-pair partials are summed (the same on every route): with G the
// smallest power of two >= min(P, 64), lane s of a G-lane segment adds the partials k = s, s + G,
// s + 2G, ... (k < P) in that order, starting from 0, and the segment then sums its lanes with an xor
// butterfly (every lane of the segment ends with the same value).
__device__ __forceinline__ int seg_lanes(int P) {
  int G = 1;
  while (G < P && G < 64) G *= 2;
  return G;
}
// Pairing at each level: lanes differing in bit 0, then bit 1 (DPP quad permutations), then the two
// 4-lane halves of each 8 mirrored, the two 8-lane halves of each 16 mirrored (DPP), then xor 16 (LDS
// swizzle) and xor 32 (permute).  After each level all lanes of a group hold the same value, so any
// pairing of whole groups keeps every lane of the segment bit-identical.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sum over the 8 consecutive lanes that hold the 8 units of one head pair's 128 bytes of a row (DPP:
// lanes differing in bit 0, then bit 1, then the two 4-lane halves mirrored): every lane of the group
// ends with the same value, since fp32 addition is commutative.
__device__ __forceinline__ float group8_sum(float x) {
  x = dpp_add<0xB1>(x);
  x = dpp_add<0x4E>(x);
  return dpp_add<0x141>(x);
}
__device__ __forceinline__ float seg_butterfly(float x, int G) {
  if (G >= 2) x = dpp_add<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  if (G >= 4) x = dpp_add<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  if (G >= 8) x = dpp_add<0x141>(x);  // row_half_mirror
  if (G >= 16) x = dpp_add<0x140>(x);  // row_mirror
  if (G >= 32) x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));  // xor 16
  if (G >= 64) x += __shfl_xor(x, 32);
  return x;
}

// r_k of one token from its full row, by one wave: each head pair's partial formed exactly as the
// state pass forms it (8 lanes per pair), then summed in the order above.  Every lane returns the value.
template <bool F16>
__device__ float row_r(const uint16_t* __restrict__ krow, int H, int P, float inv_C, float eps, int lane) {
  const int cu = lane & 7, slot = lane >> 3;
  const int G = seg_lanes(P);
  float acc = 0.f;
  for (int p0 = 0; p0 < P; p0 += 8) {
    const int pp = p0 + slot;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (pp < P && 2 * pp + (cu >> 2) < H) w = load16(krow + pp * 2 * kHeadDim + cu * 8);
    const float s = group8_sum(unit_ssq<F16>(w));
    for (int q = 0; q < 8 && p0 + q < P; ++q) {
      const float x = __shfl(s, 8 * q);
      if ((p0 + q) % G == lane) acc += x;
    }
  }
  return r_from_ssq(__shfl(seg_butterfly(acc, G), 0), inv_C, eps);
}
}  // namespace

// Block (p, c, b): head pair p of token chunk c of sample b; 4 waves, wave w multiplying head
// 2p + (w & 1) over token half (w >> 1) of each sub-block (as in the plain state kernel).  Wave 1
// also does the block's share of step 2, wave 0 the polling of step 3.
// xpart: tagged partials [B*N][P]; xr: tagged r_k [B*N]; spin: wait limit in 100 MHz ticks.
template <int L, bool F16>
__global__ __launch_bounds__(256, 2) void kv_state_x(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                     int64_t ld, const float* __restrict__ gq,
                                                     const float* __restrict__ gk, int N, int H, int Tc, int NC,
                                                     float eps, uint64_t* __restrict__ xpart,
                                                     uint64_t* __restrict__ xr, uint32_t epoch, uint32_t spin,
                                                     float* __restrict__ part, uint16_t* __restrict__ Sop,
                                                     uint16_t* __restrict__ zop, uint32_t* __restrict__ gsg) {
  // Sub-block m: partials published early in step m - L + 1 (movers), polled early in step m - A - 1
  // and summed in step m - A (leader), r_k published late in step m - A and polled early in step m - 1
  // (consumer), used in step m.  Each wave checks the polls it issued a step earlier and issues the
  // next ones right away, so every load has a full step to return; with L = 6, A = 3 every store also
  // has at least a step before the load that reads it.
  constexpr int A = 3;
  static_assert(L >= A + 3, "each hop of the exchange needs a full step");
  // The K ring, then V, r and the leader's partials; the ring is reused for the end-of-chunk combine.
  __shared__ __attribute__((aligned(16))) uint16_t Kr[L * kSB * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kSB * kPitch];
  __shared__ __attribute__((aligned(16))) float rs[kSB];
  __shared__ uint64_t missing;
  static_assert(L * kSB * kPitch * 2 >= 2 * kPartStride * 4, "the combine reuses the K ring");
  float* fin = reinterpret_cast<float*>(Kr);

  const int p = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int P = (H + 1) / 2;
  const float inv_C = 1.0f / (float)(H * kHeadDim);
  const int h0 = 2 * p;
  const int nh = min(2, H - h0);
  const int n_begin = c * Tc;
  const int n_end = min(N, n_begin + Tc);
  const int S = (n_end - n_begin + kSB - 1) / kSB;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int hh = w & 1, th = w >> 1;
  const int d = lane & 31, grp = lane >> 5;
  const int hcol = min(h0 + hh, H - 1) * kHeadDim + d;
  const uint32_t sgn = gk[hcol] < 0.f ? 0x80008000u : 0u;  // flips both tokens of a pair
  const int64_t row0 = (int64_t)b * N;
  constexpr uint32_t kOne2 = F16 ? 0x3c003c00u : 0x3f803f80u;  // two 1.0 values
  const u32x4 ones = {kOne2, kOne2, kOne2, kOne2};

  // Waves 2 and 3 move the data: thread i = tid - 128 + it * 128 stages 16 bytes, row i >> 3 of the
  // sub-block, unit i & 7 of the pair.  Range-checked buffer loads: rows past the chunk and the missing
  // second head of an odd head count read zeros without a memory access.  Waves 0 and 1 issue only the
  // exchange's loads, so their waits never cover data loads or the partials' write-through stores.
  const bool mover = w >= 2;
  u32x4 pk[4], pv[4];
  auto load_rows = [&](const uint16_t* src, int j, u32x4* dst) {
    const int n0 = n_begin + j * kSB;
    const int rows = (j >= 0 && j < S) ? min(kSB, n_end - n0) : 0;
    const __amdgpu_buffer_rsrc_t rsrc =
        make_rsrc(src + (row0 + (rows > 0 ? n0 : 0)) * ld + h0 * kHeadDim,
                  rows > 0 ? (uint32_t)(((rows - 1) * ld + 2 * kHeadDim) * 2) : 0u);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int i = tid - 128 + it * 128;
      const int row = i >> 3, cu = i & 7;
      const uint32_t off = (row < rows && (cu >> 2) < nh) ? (uint32_t)((row * ld + cu * 8) * 2) : kOutOfRange;
      dst[it] = buffer_load16(rsrc, off);
    }
  };
  auto stage = [&](uint16_t* dstl, const u32x4* src) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int i = tid - 128 + it * 128;
      store16(&dstl[(i >> 3) * kPitch + (i & 7) * 8], src[it]);
    }
  };

  f32x16 acc, accz;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc[r] = 0.f;
    accz[r] = 0.f;
  }

#pragma unroll
  for (int it = 0; it < 4; ++it) pv[it] = u32x4{0u, 0u, 0u, 0u};

  // Leader (wave 1) poll state for one sub-block: load slot q of a lane is, for P <= 64, pass q, token
  // q * (64 / G) + lane / G, partial lane % G; for P > 64 (one owned token at most), partial lane + 64 q.
  // At most 4 slots are ever needed.
  const int G = seg_lanes(P);
  const int lgG = __builtin_ctz(G);
  const int tpp = 64 >> lgG;
  uint64_t lx0[4] = {0, 0, 0, 0};
  int ltok[4] = {0, 0, 0, 0}, lk[4] = {0, 0, 0, 0};
  bool lvalid[4] = {false, false, false, false};
  int lnm0 = 0, lowned = 0;
  auto leader_issue = [&](int mm) {
    const bool in = mm >= 0 && mm < S;
    lnm0 = n_begin + (in ? mm : 0) * kSB;
    const int mrows = in ? min(kSB, n_end - lnm0) : 0;
    lowned = p < mrows ? (mrows - 1 - p) / P + 1 : 0;
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(xpart + (row0 + lnm0) * P, (uint32_t)(mrows * P * 8));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ltok[q] = P <= 64 ? q * tpp + (lane >> lgG) : 0;
      lk[q] = P <= 64 ? lane & (G - 1) : lane + 64 * q;
      lvalid[q] = ltok[q] < lowned && lk[q] < P && (P <= 64 || q < 3);
      lx0[q] = buffer_get_tagged(rl, lvalid[q] ? (uint32_t)(((p + ltok[q] * P) * P + lk[q]) * 8) : kOutOfRange);
    }
  };
  // Consumer (wave 0) poll of r_k for one sub-block, one token per lane.
  uint64_t rx0 = 0;
  auto consumer_issue = [&](int jj) {
    const bool in = jj >= 0 && jj < S;
    const int n0 = n_begin + (in ? jj : 0) * kSB;
    const int crows = in ? min(kSB, n_end - n0) : 0;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(xr + row0 + n0, (uint32_t)(crows * 8));
    rx0 = buffer_get_tagged(rc, lane < crows ? (uint32_t)(lane * 8) : kOutOfRange);
  };
  if (w == 1) leader_issue(-(L - 1) + A);  // the first step's sub-block m (negative: no loads)
  if (w == 0) consumer_issue(-(L - 1));  // likewise
  if (mover) load_rows(k, 0, pk);
  for (int j = -(L - 1); j < S; ++j) {
    const int jk = j + L - 1;
    if (mover) {
      // (1) K of sub-block j + L - 1 (in registers since the previous step) into the ring, and this head
      //     pair's partial sum of squares of each of its tokens published; V of sub-block j staged; the
      //     loads of the next K and V issued.
      // The same instructions in every step (the compiler's waits then count exactly): both stagings
      // come before the partials' stores, so that no wait for a load covers a store; outside the chunk
      // the registers hold zeros (a ring slot that is not read again, V before its first use) and the
      // stores are out of range.
      stage(Kr + ((jk + L) % L) * kSB * kPitch, pk);
      stage(Vs, pv);
      float part[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) part[it] = group8_sum(unit_ssq<F16>(pk[it]));
      load_rows(k, jk + 1, pk);
      load_rows(v, j + 1, pv);
      {
        // vmcnt counts loads and stores in issue order: the write-through stores go after the loads
        // that the next step waits for, so that no wait covers their acknowledgement.
        const int nk0 = n_begin + jk * kSB;
        const int rows = (jk >= 0 && jk < S) ? min(kSB, n_end - nk0) : 0;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(xpart + (row0 + (rows > 0 ? nk0 : 0)) * P, (uint32_t)(rows * P * 8));
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int i = tid - 128 + it * 128;
          buffer_put_tagged(rx, (i & 7) == 0 ? (uint32_t)(((i >> 3) * P + p) * 8) : kOutOfRange, part[it], epoch);
        }
      }
    }
    // (2) Tokens p, p + P, ... of sub-block m: their P partials summed, r_k published.
    const int m = j + A;
    if (w == 1) {
      // Polls for sub-block m were issued in the previous step: check them and form r_k of the owned
      // tokens; then issue the polls for sub-block m + 1 (published a step ago), to be checked in the
      // next step; then store r_k.  vmcnt counts loads and stores in issue order, so the stores go
      // after the loads the next step waits for, and every step issues the same four stores (lanes
      // with nothing to store get an out-of-range offset).
      const bool in_m = m >= 0 && m < S;
      const __amdgpu_buffer_rsrc_t rr = make_rsrc(xr + row0 + lnm0, in_m ? (uint32_t)(min(kSB, n_end - lnm0) * 8) : 0u);
      float rq[4] = {0.f, 0.f, 0.f, 0.f};
      uint32_t roff[4] = {kOutOfRange, kOutOfRange, kOutOfRange, kOutOfRange};
      bool ready = false;
      float val[4] = {0.f, 0.f, 0.f, 0.f};
      const int owned_m = lowned;
      int tok_m[4];
      bool valid_m[4];
      if (in_m) {
        bool mine = true;
#pragma unroll
        for (int q = 0; q < 4; ++q) mine = mine && (!lvalid[q] || tag_is(lx0[q], epoch));
        ready = __all(mine);
        if (!ready) {
          const uint64_t t0 = now_ticks();
          while (now_ticks() - t0 <= spin) {
            __builtin_amdgcn_s_sleep(2);
            mine = true;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (lvalid[q]) {
                lx0[q] = get_tagged(xpart + (row0 + lnm0 + p + ltok[q] * P) * P + lk[q]);
                mine = mine && tag_is(lx0[q], epoch);
              }
            if (__all(mine)) {
              ready = true;
              break;
            }
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        val[q] = lvalid[q] ? tagged_value(lx0[q]) : 0.f;
        tok_m[q] = ltok[q];
        valid_m[q] = lvalid[q];
      }
      const int nm0 = lnm0;
      leader_issue(m + 1);  // a full step before they are checked
      if (in_m) {
        if (ready) {
          if (P <= 64) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (q * tpp >= owned_m) break;  // uniform
              const float x = seg_butterfly(valid_m[q] ? 0.f + val[q] : 0.f, G);
              rq[q] = r_from_ssq(x, inv_C, eps);
              if ((lane & (G - 1)) == 0 && tok_m[q] < owned_m) roff[q] = (uint32_t)((p + tok_m[q] * P) * 8);
            }
          } else if (owned_m > 0) {
            float a = 0.f;
#pragma unroll
            for (int q = 0; q < 3; ++q)
              if (valid_m[q]) a += val[q];
            rq[0] = r_from_ssq(seg_butterfly(a, 64), inv_C, eps);
            if (lane == 0) roff[0] = (uint32_t)(p * 8);
          }
        } else {
          for (int i = 0; i < owned_m; ++i) {  // a partial is late: the whole rows, same arithmetic
            const int64_t row = row0 + nm0 + p + i * P;
            const float r = row_r<F16>(k + row * ld, H, P, inv_C, eps, lane);
            if (lane == 0) put_tagged(xr + row, r, epoch);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) buffer_put_tagged(rr, roff[q], rq[q], epoch);
    }
    // (3) r_k of sub-block j (wave 0, one token per lane).
    if (w == 0) {
      // The poll for sub-block j was issued in the previous step; the one for j + 1 goes out as soon as
      // this one has been read.
      const uint64_t got = rx0;
      consumer_issue(j + 1);
      if (j >= 0) {
        const int n0 = n_begin + j * kSB;
        const int crows = min(kSB, n_end - n0);
        float r = 1.0f;  // rows past the end hold zeros
        bool have = lane >= crows;
        if (!have && tag_is(got, epoch)) {
          r = tagged_value(got);
          have = true;
        }
        const uint64_t t0 = now_ticks();
        while (!have && now_ticks() - t0 <= spin) {
          __builtin_amdgcn_s_sleep(2);
          const uint64_t x = get_tagged(xr + row0 + n0 + lane);
          if (tag_is(x, epoch)) {
            r = tagged_value(x);
            have = true;
          }
        }
        rs[lane] = r;
        const uint64_t late = __ballot(!have);
        if (lane == 0) missing = late;
      }
    }
    __syncthreads();
    if (j >= 0 && missing != 0) {  // uniform: r_k of late tokens from their full rows
      const uint64_t late = missing;
      for (int t = w; t < kSB; t += 4)
        if ((late >> t) & 1) {
          const float r = row_r<F16>(k + (row0 + n_begin + j * kSB + t) * ld, H, P, inv_C, eps, lane);
          if (lane == 0) rs[t] = r;
        }
      __syncthreads();
    }
    if (j >= 0) {
      const uint16_t* Ks = Kr + (j % L) * kSB * kPitch;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int tb = 32 * th + 16 * s + 8 * grp;  // this lane's tokens tb .. tb+7
        const int col = hh * kHeadDim + d;
        uint32_t aw[4], bw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t0 = tb + 2 * u;
          const uint32_t kp = (uint32_t)Ks[t0 * kPitch + col] | ((uint32_t)Ks[(t0 + 1) * kPitch + col] << 16);
          bw[u] = (uint32_t)Vs[t0 * kPitch + col] | ((uint32_t)Vs[(t0 + 1) * kPitch + col] << 16);
          aw[u] = relu_bf16x2(kp ^ sgn);
        }
        const f32x4 r0 = *reinterpret_cast<const f32x4*>(&rs[tb]);
        const f32x4 r1 = *reinterpret_cast<const f32x4*>(&rs[tb + 4]);
        const float rr[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          aw[u] = cvt_pk_h<F16>(h_lo<F16>(aw[u]) * rr[2 * u], h_hi<F16>(aw[u]) * rr[2 * u + 1]);
        const u32x4 Aop = {aw[0], aw[1], aw[2], aw[3]};
        const u32x4 Bv = {bw[0], bw[1], bw[2], bw[3]};
        if constexpr (F16) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(Aop), as_f16x8(Bv), acc, 0, 0, 0);
          accz = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(Aop), as_f16x8(ones), accz, 0, 0, 0);
        } else {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Aop), as_bf16x8(Bv), acc, 0, 0, 0);
          accz = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(Aop), as_bf16x8(ones), accz, 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // Combine the two token halves of each head in a fixed order (wave hh + 2 hands over to wave hh),
  // leaving the block's state of head hh as S~[d][e] and z~[d] in `fin` (the K ring, free now).
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
  const int64_t bh0 = (int64_t)b * H + h0;
  if (NC == 1) {
    for (int i = tid; i < nh * kPartStride; i += 256) {
      const int hl = i / kPartStride, off = i - hl * kPartStride;
      emit_state<true>(bh0 + hl, h0 + hl, off, fin[i], gq, gk, Sop, zop);
    }
    if (b == 0 && tid < nh * kSgnPerHead) {
      const int h = h0 + tid / kSgnPerHead, i = tid % kSgnPerHead;
      gsg[h * kSgnPerHead + i] = sign_word<true>(gq, h, i / 4, i & 3);
    }
    return;
  }
  for (int i = tid; i < nh * kPartStride; i += 256) {
    const int hl = i / kPartStride, off = i - hl * kPartStride;
    part[((bh0 + hl) * NC + c) * kPartStride + off] = fin[i];
  }
}

size_t kv_state_x_exchange_bytes(int64_t rows, int H) {
  const size_t P = (size_t)(H + 1) / 2;
  return (size_t)rows * (P + 1) * sizeof(uint64_t);
}

hipError_t launch_kv_state_x(bool f16, const uint16_t* k, const uint16_t* v, int64_t ld, const float* gq,
                             const float* gk, int B, int N, int H, int Tc, int NC, float eps, void* xchg,
                             uint32_t epoch, uint32_t spin_ticks, float* part, uint16_t* Sop, uint16_t* zop,
                             uint32_t* gsg, hipStream_t stream) {
  constexpr int L = 6;
  const int P = (H + 1) / 2;
  uint64_t* xpart = static_cast<uint64_t*>(xchg);
  uint64_t* xr = xpart + (size_t)B * N * P;
  const dim3 grid(P, NC, B);
  if (f16)
    launch_kernel("kv_state", kv_state_x<L, true>, grid, 256, 0, stream, k, v, ld, gq, gk, N, H, Tc, NC, eps, xpart,
                  xr, epoch, spin_ticks, part, Sop, zop, gsg);
  else
    launch_kernel("kv_state", kv_state_x<L, false>, grid, 256, 0, stream, k, v, ld, gq, gk, N, H, Tc, NC, eps, xpart,
                  xr, epoch, spin_ticks, part, Sop, zop, gsg);
  return hipGetLastError();
}

}  // namespace sanala

// Mix-FFN of SANA's Linear DiT block on gfx950: pointwise expansion, 3x3 depthwise convolution with
// zero padding over the token grid, GLU, pointwise projection.
//
// The Sana notes (section 2.2, Mix-FFN) replace the MLP feed-forward by an inverted residual block,
// a 3x3 depthwise convolution and a GLU; section 2.3 (NoPE) relies on the zero padding of that
// convolution for position information.  Width 5600 at 2240 channels (SANA 1.5 notes, architecture).
//
// The two pointwise projections are dense contractions and run on the MFMA GEMM of gemm_kernel.hip.
// Between them sits one HBM-bound kernel that reads the expanded activations once and writes the gated
// result once: block (chunk, b, band) owns 64 value channels [64 chunk, 64 chunk + 64) and the matching
// 64 gate channels (+F) of sample b and walks the band's grid rows top to bottom, keeping three rows in an LDS
// ring (each with a zero column on either side); the loads of the next two rows are in flight while
// the current output row is formed.  Each lane holds the 9 taps of its 4 value and 4 gate channels in
// registers, and two blocks share a CU.
#include "common.h"

#include <algorithm>

namespace sanala {

namespace {
constexpr int kCh = 64;                 // value channels per block (and as many gate channels)
constexpr int kTokBytes = 2 * kCh * 2;  // LDS bytes per token: 64 value + 64 gate bf16
constexpr int kThreads = 256;
}  // namespace

int mix_ffn_max_width() { return 128; }

// h: bf16, chunk-major [2F/32][M][32] (channel c of token m at ((c / 32) * M + m) * 32 + c % 32, M =
// B*Hg*Wg; values are channels [0, F), gates [F, 2F)), as the expansion GEMM stores it; kdw: [2F][9] bf16
// (tap 3p + q reads row i+p-1, column j+q-1); g: bf16, K-blocked for the projection, [F/32][M][32].
// gridDim.y = B.  F is a multiple of 32; Wg <= 16 * UNITS.  Row loads are masked (rows past Hg and
// channels past F read zeros without memory traffic), two rows ahead of the row being formed, in two
// register sets.
template <int UNITS>
__global__ __launch_bounds__(kThreads, 2) void dwconv_glu_kernel(const uint16_t* __restrict__ h,
                                                                 const uint16_t* __restrict__ kdw,
                                                                 uint16_t* __restrict__ g, int Hg, int Wg, int F,
                                                                 int rows_per_block) {
  extern __shared__ __attribute__((aligned(16))) char ring[];  // [3][roundup(Wg, 4) + 2][kTokBytes]
  const int chunk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int r0 = blockIdx.z * rows_per_block, r1 = min(Hg, r0 + rows_per_block);  // output rows of the block
  const int c0 = chunk * kCh;
  const int N = Hg * Wg;
  const int64_t Mtot = (int64_t)gridDim.y * N;
  const int slot_bytes = ((Wg + 3) / 4 * 4 + 2) * kTokBytes;  // halo column, Wg rounded up to 4, halo

  // This lane's channel group (4 value channels c0 + 4cg.., the gates F + the same) and its taps.
  const int cg = tid & 15;
  const int cv = c0 + 4 * cg;
  const bool cvalid = cv < F;  // F is a multiple of 8: a group is wholly inside or outside
  float wa[4][9], wb[4][9];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int t = 0; t < 9; ++t) {
      wa[e][t] = cvalid ? __uint_as_float((uint32_t)kdw[(int64_t)(cv + e) * 9 + t] << 16) : 0.f;
      wb[e][t] = cvalid ? __uint_as_float((uint32_t)kdw[(int64_t)(F + cv + e) * 9 + t] << 16) : 0.f;
    }

  // Unit u of a row: chunk q = u / (4 Wg) (q = 0, 1: value channels c0 + 32q ..; q = 2, 3: the gates
  // F + c0 + 32(q - 2) ..), token t = (u / 4) % Wg, 16-byte piece w = u % 4; so one wave's load covers 16
  // tokens of one chunk, 1 KB of consecutive bytes.  In LDS the unit goes to token t, part 4q + w
  // (0..7 values, 8..15 gates).  The roles do not depend on the row: the row adds i * Wg * 64 bytes.
  const int units = Wg * 16;
  const uint16_t* src[UNITS];
  int lds_off[UNITS];
  bool uok[UNITS];
#pragma unroll
  for (int k = 0; k < UNITS; ++k) {
    const int u = tid + k * kThreads;
    const int q = u / (4 * Wg), rem = u - q * 4 * Wg, t = rem >> 2, w = rem & 3;
    const int ch = ((q < 2 ? c0 : F + c0) >> 5) + (q & 1);  // F and c0 are multiples of 32
    uok[k] = u < units && c0 + 32 * (q & 1) + 8 * w < F;
    src[k] = h + (((int64_t)ch * Mtot + (int64_t)b * N + t) << 5) + 8 * w;
    lds_off[k] = (t + 1) * kTokBytes + (4 * q + w) * 16;
  }
  auto load_row = [&](int i, u32x4 (&pre)[UNITS]) {
    const bool row_ok = i >= 0 && i < Hg;
#pragma unroll
    for (int k = 0; k < UNITS; ++k)
      pre[k] = row_ok && uok[k] ? load16(src[k] + ((int64_t)i * Wg << 5)) : u32x4{0u, 0u, 0u, 0u};
  };
  auto store_row = [&](int slot, const u32x4 (&pre)[UNITS]) {
    char* base = ring + slot * slot_bytes;
#pragma unroll
    for (int k = 0; k < UNITS; ++k) {
      const int u = tid + k * kThreads;
      if (u < units) store16(base + lds_off[k], pre[k]);
    }
  };
  auto slot_of = [&](int i) { return (i - r0 + 1) % 3; };  // i >= r0 - 1
  auto compute_row = [&](int i) {
    const char* rows[3] = {ring + slot_of(i - 1) * slot_bytes, ring + slot_of(i) * slot_bytes,
                           ring + slot_of(i + 1) * slot_bytes};
    // Lane (run r, group cg) forms tokens 4r .. 4r + 3 of the row from the six columns 4r - 1 ..
    // 4r + 4 of each of the three rows (1.5 LDS reads per tap instead of 9 per token).
    for (int r = tid >> 4; 4 * r < Wg; r += kThreads / 16) {
      const int j0 = 4 * r;
      float a[4][4], z[4][4];  // [token][channel]
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) a[k][e] = z[k][e] = 0.f;
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        uint2 va[6], vb[6];
#pragma unroll
        for (int c = 0; c < 6; ++c) {
          const char* tok = rows[p] + (j0 + c) * kTokBytes;  // column j0 + c - 1, shifted by the halo
          va[c] = *reinterpret_cast<const uint2*>(tok + 8 * cg);
          vb[c] = *reinterpret_cast<const uint2*>(tok + 128 + 8 * cg);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            const int t = 3 * p + q;
            const uint2 xa = va[k + q], xb = vb[k + q];
            a[k][0] = fmaf(wa[0][t], bf16_lo(xa.x), a[k][0]);
            a[k][1] = fmaf(wa[1][t], bf16_hi(xa.x), a[k][1]);
            a[k][2] = fmaf(wa[2][t], bf16_lo(xa.y), a[k][2]);
            a[k][3] = fmaf(wa[3][t], bf16_hi(xa.y), a[k][3]);
            z[k][0] = fmaf(wb[0][t], bf16_lo(xb.x), z[k][0]);
            z[k][1] = fmaf(wb[1][t], bf16_hi(xb.x), z[k][1]);
            z[k][2] = fmaf(wb[2][t], bf16_lo(xb.y), z[k][2]);
            z[k][3] = fmaf(wb[3][t], bf16_hi(xb.y), z[k][3]);
          }
      }
      if (cvalid) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (j0 + k >= Wg) break;
          float gv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) gv[e] = a[k][e] * __builtin_amdgcn_rcpf(1.f + __expf(-z[k][e]));
          // g is stored K-blocked for the projection GEMM: [F/32][M][32], M = B * N.
          const int64_t m = (int64_t)b * N + (int64_t)i * Wg + j0 + k;
          *reinterpret_cast<uint2*>(g + (((int64_t)(cv >> 5) * gridDim.y * N + m) << 5) + (cv & 31)) =
              make_uint2(cvt_pk_bf16(gv[0], gv[1]), cvt_pk_bf16(gv[2], gv[3]));
        }
      }
    }
  };

  // Zero the three slots (the halo and padding columns are never written again).
  for (int o = tid * 16; o < 3 * slot_bytes; o += kThreads * 16) store16(ring + o, u32x4{0u, 0u, 0u, 0u});
  u32x4 ra[UNITS], rb[UNITS];
  load_row(r0 - 1, ra);  // zeros above the grid
  load_row(r0, rb);
  __syncthreads();
  store_row(slot_of(r0 - 1), ra);
  store_row(slot_of(r0), rb);
  load_row(r0 + 1, ra);
  load_row(r0 + 2, rb);
  // Row i is formed from the slots of rows i - 1, i, i + 1; at its start the registers hold rows
  // i + 1 and i + 2 (ra, rb alternate), and the loads of row i + 3 go out as row i + 1 is stored.
  for (int i = r0; i < r1; i += 2) {
    store_row(slot_of(i + 1), ra);
    load_row(i + 3, ra);
    __syncthreads();
    compute_row(i);
    __syncthreads();  // the slot of row i - 1 is overwritten next
    if (i + 1 >= r1) break;
    store_row(slot_of(i + 2), rb);
    load_row(i + 4, rb);
    __syncthreads();
    compute_row(i + 1);
    __syncthreads();
  }
}

hipError_t launch_mix_ffn(const uint16_t* x, const uint16_t* w1, const uint16_t* kdw, const uint16_t* w2, int B, int Hg,
                          int Wg, int C, int F, uint16_t* out, void* ws, hipStream_t stream) {
  const int64_t M = (int64_t)B * Hg * Wg;
  uint16_t* hbuf = static_cast<uint16_t*>(ws);
  // The second region holds x K-blocked for the expansion GEMM, then g (K-blocked) for the projection.
  uint16_t* gbuf = hbuf + (M * 2 * F + 127) / 128 * 128;
  hipError_t e = launch_relayout_k32(x, M, C, gbuf, stream);
  if (e != hipSuccess) return e;
  e = launch_gemm_bf16(gbuf, w1, hbuf, M, C, 2 * F, stream, "gemm_expand", true);
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)3 * ((Wg + 3) / 4 * 4 + 2) * kTokBytes;
  e = Wg <= 64 ? ensure_max_lds(reinterpret_cast<const void*>(&dwconv_glu_kernel<4>), 160 * 1024)
              : ensure_max_lds(reinterpret_cast<const void*>(&dwconv_glu_kernel<8>), 160 * 1024);
  if (e != hipSuccess) return e;
  // Row bands: enough blocks for about three rounds of two blocks per CU (each band re-reads one grid
  // row above and below it), bands of at least 8 rows.
  const int chunks = (F + kCh - 1) / kCh;
  const int want = std::max(1, (6 * 256 + chunks * B / 2) / (chunks * B));
  const int bands = std::max(1, std::min(want, Hg / 8));
  const int rows_per_block = (Hg + bands - 1) / bands;
  const dim3 grid(chunks, B, (Hg + rows_per_block - 1) / rows_per_block);
  if (Wg <= 64)
    launch_kernel("dwconv_glu", dwconv_glu_kernel<4>, grid, kThreads, lds, stream, hbuf, kdw, gbuf, Hg, Wg, F,
                  rows_per_block);
  else
    launch_kernel("dwconv_glu", dwconv_glu_kernel<8>, grid, kThreads, lds, stream, hbuf, kdw, gbuf, Hg, Wg, F,
                  rows_per_block);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  final_launch();
  return launch_gemm_bf16(gbuf, w2, out, M, F, C, stream, "gemm_project");
}

size_t mix_ffn_workspace_bytes(int64_t M, int C, int F) {
  return (size_t)((M * 2 * F + 127) / 128 * 128) * 2 + (size_t)M * std::max(C, F) * 2;
}

}  // namespace sanala

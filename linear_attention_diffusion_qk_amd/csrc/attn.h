// Internal host interface between the C-ABI entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstddef>
#include <cstdint>

namespace sanala {

constexpr int kHeadDim = 32;  // D: the only head size with kernels
constexpr int kDtypeF32 = 0;
constexpr int kDtypeBf16 = 1;
constexpr int kDtypeF16 = 2;
// Persistent output kernel: head pairs per wave and the most waves per block (3 x 12 pairs: H <= 72,
// which is also the most heads whose operands fit in one CU's LDS).  Three pairs per wave (12 waves for
// 70 heads) measured 26.7 us against 28.2 us for five (7 waves) on the 16384-token workload.
constexpr int kPersistPPW = 3;
constexpr int kPersistMaxWaves = 12;
constexpr int kOutPersist = 1;  // bf16 output: one block per CU, all heads, operands in LDS
constexpr int kOutTile = 2;     // bf16 output: 16-token tiles over all heads, operands from global memory
constexpr int kOutTileGroups = 3;  // bf16 output for few tiles: 16 tokens x 8 heads per block, r_q from the
                                   // row-statistics launch (which then covers Q and K)

// Launch plan and scratch layout of one attention call.
struct AttnPlan {
  int B, N, H, dtype;
  bool norm;
  int Tc;               // tokens per KV chunk (multiple of 64)
  int NC;               // number of chunks per sample
  int out_kind;         // bf16 output kernel: kOutPersist, kOutTile or kOutTileGroups
  bool out_strided;     // persistent output kernel: block b takes tiles b, b + G, ... (else a contiguous run)
  int out_group;        // persistent output kernel, not strided: g > 0 blocks share each sample's tiles, block
                        // j of a sample taking tiles j, j + g, ... (0: each block a contiguous run)
  int num_cus;          // compute units of the current device
  bool state_xchg;      // 16-bit, QK-Norm on, r_q in the output kernel: r_k formed inside the state pass
  bool rendezvous;      // 16-bit, NC > 1: the state blocks reduce the chunk partials among themselves
  bool nt_v;            // 16-bit path reads K and V with non-temporal loads (see plan_attn)
  uint32_t xchg_spin;   // wait limit of the cross-block waits (exchange, rendezvous), 100 MHz ticks
  size_t off_rk, off_rq, off_part, off_S32, off_z, off_Sop, off_xchg, off_flags;
  size_t ws_bytes;
};

// fused: q, k and v come from the projection in front of the attention (the library's own scratch).
AttnPlan plan_attn(int B, int N, int H, int dtype, bool norm, bool fused = false);

// q is read with row stride ldq, k and v with ldkv, out written with ldo (all in elements).
// k_ssq (bf16 path only, optional): per-row partial sums of squares of K in k_parts column panels,
// row-major [B*N][k_parts] (from the projection epilogue); when given, r_k is formed from them and the
// row-statistics pass over K is skipped.
hipError_t launch_attn(const AttnPlan& p, const void* q, int64_t ldq, const void* k, const void* v, int64_t ldkv,
                       const float* gq, const float* gk, float eps, void* out, int64_t ldo, void* ws,
                       hipStream_t stream, const float* k_ssq = nullptr, int k_parts = 0);

hipError_t launch_attn_f32(const AttnPlan& p, const float* q, int64_t ldq, const float* k, const float* v,
                           int64_t ldkv, const float* gq, const float* gk, float eps, float* out, int64_t ldo,
                           void* ws, hipStream_t stream);
// 16-bit storage (bf16 or binary16, p.dtype).
hipError_t launch_attn_bf16(const AttnPlan& p, const uint16_t* q, int64_t ldq, const uint16_t* k, const uint16_t* v,
                            int64_t ldkv, const float* gq, const float* gk, float eps, uint16_t* out, int64_t ldo,
                            void* ws, int num_cus, hipStream_t stream, const float* k_ssq, int k_parts);
size_t out_persist_lds_bytes(int H);
// KV state with r_k formed in the same pass (kv_state_x.hip): tagged exchange buffers of
// kv_state_x_exchange_bytes(B*N, H) bytes at xchg; epoch unique per call (never 0).
size_t kv_state_x_exchange_bytes(int64_t rows, int H);
hipError_t launch_kv_state_x(bool f16, const uint16_t* k, const uint16_t* v, int64_t ld, const float* gq,
                             const float* gk, int B, int N, int H, int Tc, int NC, float eps, void* xchg,
                             uint32_t epoch, uint32_t spin_ticks, float* part, uint16_t* Sop, uint16_t* zop,
                             uint32_t* gsg, hipStream_t stream);
uint32_t next_epoch();
size_t bf16_operand_bytes(int64_t BH, int H);

int max_heads();

// x [M][K] bf16 row-major -> xb [K/32][M][32], the K-blocked x layout the bf16 GEMMs below take
// (K a multiple of 32).
hipError_t launch_relayout_k32(const uint16_t* x, int64_t M, int K, uint16_t* xb, hipStream_t stream);
// qkv[M, 3C] = x[M, C] @ w[C, 3C], bf16 in / bf16 out (fp32 accumulation); xb is x K-blocked
// (launch_relayout_k32), w row-major.  With k_ssq set, the blocks
// whose columns overlap the K block [C, 2C) also write, per row, the sum of squares of the bf16 outputs
// they hold in that block: k_ssq[m * qkv_gemm_k_parts(C, gemm_wide(M, 3C)) + j] for the j-th such
// column panel.
hipError_t launch_qkv_gemm(const uint16_t* xb, const uint16_t* w, uint16_t* qkv, int64_t M, int C,
                           hipStream_t stream, float* k_ssq = nullptr);
// Whether a bf16 GEMM of M rows by NO output columns runs on 256-column blocks (else 192).
bool gemm_wide(int64_t M, int NO);
// Column panels of the K block [C, 2C) for the given block width (the int8 form: wide = false).
int qkv_gemm_k_parts(int C, bool wide);
// W8A8 form: xq int8 K-blocked [C/64][M][64] (launch_quant_rows with k_blocked) with per-row scales
// s_x [M]; wt int8 K-blocked [C/64][3C][64] (launch_pack_k64 of W transposed, [3C, C]) with per-column
// scales s_w [3C]; qkv = bf16((sum_c xq*wt) * s_x[m] * s_w[n]).
// C must be a multiple of 64.  k_ssq as for launch_qkv_gemm.
hipError_t launch_qkv_gemm_i8(const int8_t* xq, const int8_t* wt, const float* s_x, const float* s_w, uint16_t* qkv,
                              int64_t M, int C, hipStream_t stream, float* k_ssq = nullptr);
// Plain bf16 GEMM y[M, NO] = x[M, K] @ w[K, NO] on the same kernel (K a multiple of 32, NO of 8); xb is
// x K-blocked, [K/32][M][32]; with y_blocked, y is stored the same way, [NO/32][M][32] (NO a multiple
// of 32).
hipError_t launch_gemm_bf16(const uint16_t* xb, const uint16_t* w, uint16_t* y, int64_t M, int K, int NO,
                            hipStream_t stream, const char* label = "gemm", bool y_blocked = false);
// Mix-FFN: y = GLU(dwconv3x3(x @ W1)) @ W2 over B grids of Hg x Wg tokens (C channels, width F).  ws
// holds mix_ffn_workspace_bytes(B*Hg*Wg, C, F) bytes.  C and F multiples of 32, Wg <= mix_ffn_max_width().
hipError_t launch_mix_ffn(const uint16_t* x, const uint16_t* w1, const uint16_t* kdw, const uint16_t* w2, int B, int Hg,
                          int Wg, int C, int F, uint16_t* out, void* ws, hipStream_t stream);
size_t mix_ffn_workspace_bytes(int64_t M, int C, int F);
int mix_ffn_max_width();
// Cross-attention with QK-Norm (cross_attn.hip): q, out [B, N, 32H]; k, v [B, L, 32H]; all bf16; gq, gk
// [32H] or both NULL; kv_len [B] int32 on the device or NULL.  ws holds
// cross_attn_workspace_bytes(B, N, L, H) bytes.  L <= cross_attn_max_keys(), H <= cross_attn_max_heads().
hipError_t launch_cross_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* gq, const float* gk,
                             const int* kv_len, int B, int N, int L, int H, float eps, uint16_t* out, void* ws,
                             hipStream_t stream);
size_t cross_attn_workspace_bytes(int64_t B, int64_t N, int64_t L, int H);
int cross_attn_max_keys();
int cross_attn_max_heads();

// int8 [rows, C] row-major -> K-blocked [C/64][rows][64] (C a multiple of 64).
hipError_t launch_pack_k64(const int8_t* src, int64_t rows, int C, int8_t* dst, hipStream_t stream);

// Per-row symmetric int8 quantisation of bf16 x [M, C] (C a multiple of 8); codes row-major, or
// K-blocked [C/64][M][64] for the int8 GEMM (C a multiple of 64).
hipError_t launch_quant_rows(const uint16_t* x, int64_t M, int C, int8_t* xq, float* s_x, hipStream_t stream,
                             bool k_blocked = false);

// Measurement hooks (no-ops unless timing is enabled on the calling host thread): an event pair is
// recorded on `s` around each kernel launch.
// Kernel timing (sana_timing_enable): the next pair of events of the calling thread, labelled `name`;
// false when timing is off.
bool timing_slot(const char* name, hipEvent_t* begin, hipEvent_t* end);

// The event the current call on this host thread signals when its work completes (the scratch buffer's
// last use), or nullptr.  A path calls final_launch() just before its last launch, which then carries
// the event as its dispatch's stop event (no marker packet in the queue); `carried` says whether the
// most recent launch carried it.  Only the last launch carries it: on MI355X a stop event on each of
// four small back-to-back launches cost 8.4 us per four, on the last one only 1.8 us, and an event
// recorded after them 3.7 us.
struct StopSignal {
  hipEvent_t event = nullptr;
  bool final = false;
  bool carried = false;
};
StopSignal& stop_signal();
inline void final_launch() { stop_signal().final = true; }

// Raises `kernel`'s dynamic-LDS limit to `bytes` on the current device, once per (kernel, device);
// safe to call from several host threads.
hipError_t ensure_max_lds(const void* kernel, int bytes);

// kernel<<<grid, block, lds, stream>>>(args...).  With timing on, the launch goes through
// hipExtLaunchKernelGGL with a start/stop event pair that the dispatch itself timestamps, so the
// recorded duration is the kernel's own (no event packets between kernels).
template <typename... P, typename... A>
inline void launch_kernel(const char* name, void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                          A... args) {
  hipEvent_t b = nullptr, e = nullptr;
  StopSignal& ss = stop_signal();
  ss.carried = false;
  if (timing_slot(name, &b, &e)) {
    hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)lds, stream, b, e, 0u, args...);
  } else if (ss.event && ss.final) {
    hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)lds, stream, nullptr, ss.event, 0u, args...);
    ss.carried = true;
  } else {
    kernel<<<grid, block, lds, stream>>>(args...);
  }
  ss.final = false;
}

}  // namespace sanala

// Internal host interface between the C-ABI entry points and the attention kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace sanala {

constexpr int kHeadDim = 32;  // D: the only head size with kernels
constexpr int kDtypeF32 = 0;
constexpr int kDtypeBf16 = 1;

// Launch plan and scratch layout of one attention call.
struct AttnPlan {
  int B, N, H, dtype;
  bool norm;
  int Tc;  // tokens per KV chunk (multiple of 64)
  int NC;  // number of chunks per sample
  size_t off_rk, off_rq, off_part, off_S32, off_z, off_Sop;
  size_t ws_bytes;
};

AttnPlan plan_attn(int B, int N, int H, int dtype, bool norm);

// q is read with row stride ldq, k and v with ldkv, out written with ldo (all in elements).
hipError_t launch_attn(const AttnPlan& p, const void* q, int64_t ldq, const void* k, const void* v, int64_t ldkv,
                       const float* gq, const float* gk, float eps, void* out, int64_t ldo, void* ws,
                       hipStream_t stream);

int out_bf16_max_heads();

// qkv[M, 3C] = x[M, C] @ w[C, 3C], bf16 in / bf16 out (fp32 accumulation).
hipError_t launch_qkv_gemm(const uint16_t* x, const uint16_t* w, uint16_t* qkv, int64_t M, int C, hipStream_t stream);

}  // namespace sanala

// C-ABI entry points of libsanala: argument checks, stream-ordered scratch, launches.
#include "../../include/sanala.h"
#include "attn.h"
#include "scratch_table.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_pool_once[kMaxDevices];

// Keep freed stream-ordered scratch in the device's default pool instead of returning it to the
// driver at every synchronisation, so steady-state calls do not allocate from the OS.
void init_pool(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return;
  std::call_once(g_pool_once[dev], [dev]() {
    hipMemPool_t pool;
    if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
      uint64_t threshold = UINT64_MAX;
      (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &threshold);
    }
  });
}

// Scratch kept per (device, stream): the lifecycle rules are those of ScratchTable (scratch_table.h).
// (Freeing scratch at every call cost about 15 us of host time per call, more than the 1024-token
// call's GPU time.)
struct HipBackend {
  int alloc_async(void** p, size_t bytes, void* s) {
    return hipMallocAsync(p, bytes, static_cast<hipStream_t>(s)) == hipSuccess ? 0 : 1;
  }
  int free_async(void* p, void* s) { return hipFreeAsync(p, static_cast<hipStream_t>(s)) == hipSuccess ? 0 : 1; }
  int event_create(void** ev) {
    // Used only to order later work after it: no timing, and no system-scope cache flush when it fires.
    return hipEventCreateWithFlags(reinterpret_cast<hipEvent_t*>(ev), hipEventDisableTiming | hipEventDisableSystemFence) ==
                   hipSuccess
               ? 0
               : 1;
  }
  int event_record(void* ev, void* s) {
    return hipEventRecord(static_cast<hipEvent_t>(ev), static_cast<hipStream_t>(s)) == hipSuccess ? 0 : 1;
  }
  int event_done(void* ev) { return hipEventQuery(static_cast<hipEvent_t>(ev)) == hipSuccess ? 1 : 0; }
  int stream_wait(void* s, void* ev) {
    return hipStreamWaitEvent(static_cast<hipStream_t>(s), static_cast<hipEvent_t>(ev), 0) == hipSuccess ? 0 : 1;
  }
};
HipBackend g_backend;
sanala::ScratchTable<HipBackend> g_table(g_backend);

// Per-host-thread kernel timing (measurement support).
struct TimedKernel {
  const char* name;
  hipEvent_t begin, end;
};
struct Timing {
  bool enabled = false;
  int count = 0;
  std::vector<TimedKernel> slots;
  ~Timing() {
    for (auto& t : slots) {
      (void)hipEventDestroy(t.begin);
      (void)hipEventDestroy(t.end);
    }
  }
};
thread_local Timing g_timing;

// A call's hold on its stream's scratch.  While held, the call's last kernel carries the buffer's
// last-use event as its stop event (launch_kernel after final_launch()); otherwise (kernel timing on,
// or a path whose last launch did not carry it) the event is recorded when the lease ends.
class ScratchLease {
 public:
  hipError_t acquire(int dev, hipStream_t stream, size_t bytes) {
    if (g_table.acquire(lease_, dev, stream, bytes) != 0) return hipErrorOutOfMemory;
    sanala::StopSignal& ss = sanala::stop_signal();
    ss = sanala::StopSignal{};
    if (!g_timing.enabled) ss.event = static_cast<hipEvent_t>(lease_.event());
    return hipSuccess;
  }
  ~ScratchLease() {
    sanala::StopSignal& ss = sanala::stop_signal();
    if (ss.event && ss.carried) lease_.attached();
    ss = sanala::StopSignal{};
  }
  void* ptr() const { return lease_.ptr(); }

 private:
  sanala::ScratchTable<HipBackend>::Lease lease_;
};

// Scratch of the allocation-free entry point: one static device array per GPU the library runs on,
// held until the process ends.  Host code never uses the array's name as an address (on the host it
// is only a stand-in for the symbol): each device's address comes from hipGetSymbolAddress, taken
// once per device with that device current.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
__device__ __attribute__((aligned(256))) static char scratch[kStaticScratchBytes];

std::once_flag g_static_once[kMaxDevices];
void* g_static_ptr[kMaxDevices];
hipError_t g_static_err[kMaxDevices];

// The current device's address of `scratch`, or nullptr (err set).  `dev` must be the current device.
void* static_scratch(int dev, hipError_t* err) {
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_static_once[dev], [dev]() {
    void* p = nullptr;
    g_static_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_static_ptr[dev] = g_static_err[dev] == hipSuccess ? p : nullptr;
  });
  *err = g_static_err[dev];
  return g_static_ptr[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

sana_status_t check_common(int B, int N, int H, int D, float eps, const float* gq, const float* gk) {
  if (B <= 0 || N <= 0 || H <= 0 || D <= 0) return SANA_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.f) return SANA_ERR_INVALID_ARG;
  if ((gq == nullptr) != (gk == nullptr)) return SANA_ERR_INVALID_ARG;
  if (D != sanala::kHeadDim) return SANA_ERR_UNSUPPORTED;
  if (H > sanala::max_heads()) return SANA_ERR_UNSUPPORTED;
  if (B > 65535) return SANA_ERR_UNSUPPORTED;
  const double elems = (double)B * (double)N * (double)H * (double)D;
  if (elems >= 1099511627776.0) return SANA_ERR_UNSUPPORTED;  // 2^40
  if ((gq && !aligned16(gq)) || (gk && !aligned16(gk))) return SANA_ERR_MISALIGNED;
  return SANA_OK;
}


}  // namespace

namespace sanala {
hipError_t ensure_max_lds(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::vector<std::pair<const void*, int>> done;  // (kernel, device) pairs already raised
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  for (const auto& d : done)
    if (d.first == kernel && d.second == dev) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.emplace_back(kernel, dev);
  return e;
}

StopSignal& stop_signal() {
  thread_local StopSignal ss;
  return ss;
}

bool timing_slot(const char* name, hipEvent_t* begin, hipEvent_t* end) {
  Timing& T = g_timing;
  if (!T.enabled) return false;
  if (T.count == (int)T.slots.size()) {
    TimedKernel k{name, nullptr, nullptr};
    if (hipEventCreate(&k.begin) != hipSuccess || hipEventCreate(&k.end) != hipSuccess) return false;
    T.slots.push_back(k);
  }
  TimedKernel& k = T.slots[T.count++];
  k.name = name;
  *begin = k.begin;
  *end = k.end;
  return true;
}
}  // namespace sanala

extern "C" sana_status_t sana_timing_enable(int enable) {
  g_timing.enabled = enable != 0;
  g_timing.count = 0;
  return SANA_OK;
}

extern "C" int sana_timing_last(const char** names, float* ms, int capacity) {
  Timing& T = g_timing;
  int n = 0;
  for (; n < T.count && n < capacity; ++n) {
    float t = -1.f;
    if (hipEventSynchronize(T.slots[n].end) == hipSuccess)
      (void)hipEventElapsedTime(&t, T.slots[n].begin, T.slots[n].end);
    if (names) names[n] = T.slots[n].name;
    if (ms) ms[n] = t;
  }
  return T.count;
}

extern "C" sana_status_t sana_release_scratch(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SANA_ERR_HIP;
  return g_table.release(dev, stream) == 0 ? SANA_OK : SANA_ERR_HIP;
}

extern "C" const char* sana_status_string(sana_status_t s) {
  switch (s) {
    case SANA_OK: return "ok";
    case SANA_ERR_INVALID_ARG: return "invalid argument";
    case SANA_ERR_UNSUPPORTED: return "unsupported shape or dtype (D must be 32, H <= 320, B <= 65535)";
    case SANA_ERR_MISALIGNED: return "tensor pointer not 16-byte aligned";
    case SANA_ERR_HIP: return "HIP runtime error";
    case SANA_ERR_SCRATCH_LIMIT:
      return "the call needs more scratch than the allocation-free entry point's static buffer (64 MiB per device)";
  }
  return "unknown status";
}

namespace {
sana_status_t check_attn(const void* q, const void* k, const void* v, const float* gq, const float* gk, int B, int N,
                         int H, int D, float eps, void* out, sana_dtype_t dtype) {
  if (!q || !k || !v || !out) return SANA_ERR_INVALID_ARG;
  if (dtype != SANA_F32 && dtype != SANA_BF16 && dtype != SANA_F16) return SANA_ERR_INVALID_ARG;
  sana_status_t st = check_common(B, N, H, D, eps, gq, gk);
  if (st != SANA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SANA_ERR_MISALIGNED;
  const size_t esz = dtype == SANA_F32 ? 4 : 2;
  const size_t tbytes = (size_t)B * N * H * D * esz;
  if (overlaps(out, tbytes, q, tbytes) || overlaps(out, tbytes, k, tbytes) || overlaps(out, tbytes, v, tbytes))
    return SANA_ERR_INVALID_ARG;
  return SANA_OK;
}

int dtype_code(sana_dtype_t dtype) {
  return dtype == SANA_BF16 ? sanala::kDtypeBf16 : dtype == SANA_F16 ? sanala::kDtypeF16 : sanala::kDtypeF32;
}
}  // namespace

extern "C" sana_status_t sana_linear_attn_fwd(const void* q, const void* k, const void* v, const float* gq,
                                              const float* gk, int B, int N, int H, int D, float eps, void* out,
                                              hipStream_t stream, sana_dtype_t dtype) {
  const sana_status_t st = check_attn(q, k, v, gq, gk, B, N, H, D, eps, out, dtype);
  if (st != SANA_OK) return st;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SANA_ERR_HIP;
  init_pool(dev);
  g_timing.count = 0;
  const bool norm = gq != nullptr;
  const sanala::AttnPlan plan = sanala::plan_attn(B, N, H, dtype_code(dtype), norm);
  ScratchLease lease;
  if (lease.acquire(dev, stream, plan.ws_bytes) != hipSuccess) return SANA_ERR_HIP;
  const int64_t C = (int64_t)H * D;
  const hipError_t e = sanala::launch_attn(plan, q, C, k, v, C, gq, gk, eps, out, C, lease.ptr(), stream);
  return e == hipSuccess ? SANA_OK : SANA_ERR_HIP;
}

extern "C" sana_status_t sana_linear_attn_fwd_noalloc(const void* q, const void* k, const void* v, const float* gq,
                                                      const float* gk, int B, int N, int H, int D, float eps,
                                                      void* out, hipStream_t stream, sana_dtype_t dtype) {
  const sana_status_t st = check_attn(q, k, v, gq, gk, B, N, H, D, eps, out, dtype);
  if (st != SANA_OK) return st;
  const sanala::AttnPlan plan = sanala::plan_attn(B, N, H, dtype_code(dtype), gq != nullptr);
  if (plan.ws_bytes > kStaticScratchBytes) return SANA_ERR_SCRATCH_LIMIT;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SANA_ERR_HIP;
  hipError_t e = hipSuccess;
  void* ws = static_scratch(dev, &e);
  if (!ws) return SANA_ERR_HIP;
  // Kernel timing would create events: it stays off for this call.
  const bool timing = g_timing.enabled;
  g_timing.enabled = false;
  g_timing.count = 0;
  const int64_t C = (int64_t)H * D;
  e = sanala::launch_attn(plan, q, C, k, v, C, gq, gk, eps, out, C, ws, stream);
  g_timing.enabled = timing;
  return e == hipSuccess ? SANA_OK : SANA_ERR_HIP;
}

extern "C" sana_status_t sana_qkv_linear_attn_fwd(const void* x, const void* Wqkv, const float* gq, const float* gk,
                                                  int B, int N, int H, int D, float eps, void* out,
                                                  hipStream_t stream) {
  if (!x || !Wqkv || !out) return SANA_ERR_INVALID_ARG;
  sana_status_t st = check_common(B, N, H, D, eps, gq, gk);
  if (st != SANA_OK) return st;
  if (!aligned16(x) || !aligned16(Wqkv) || !aligned16(out)) return SANA_ERR_MISALIGNED;
  const int64_t C = (int64_t)H * D;
  const int64_t M = (int64_t)B * N;
  const size_t xbytes = (size_t)M * C * 2;
  if (overlaps(out, xbytes, x, xbytes) || overlaps(out, xbytes, Wqkv, (size_t)C * 3 * C * 2))
    return SANA_ERR_INVALID_ARG;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SANA_ERR_HIP;
  init_pool(dev);
  g_timing.count = 0;
  const bool norm = gq != nullptr;
  const sanala::AttnPlan plan = sanala::plan_attn(B, N, H, sanala::kDtypeBf16, norm, true);
  // With the QK-Norm on, the projection's epilogue also leaves per-row partial sums of squares of K,
  // which replace the attention's row-statistics pass over K.
  const size_t qkv_bytes = ((size_t)M * 3 * C * 2 + 255) / 256 * 256;
  const int k_parts = norm ? sanala::qkv_gemm_k_parts((int)C, sanala::gemm_wide(M, 3 * (int)C)) : 0;
  const size_t ssq_bytes = ((size_t)M * k_parts * 4 + 255) / 256 * 256;
  const size_t xb_bytes = ((size_t)M * C * 2 + 255) / 256 * 256;  // x K-blocked for the GEMM
  ScratchLease lease;
  if (lease.acquire(dev, stream, qkv_bytes + ssq_bytes + std::max(xb_bytes, plan.ws_bytes)) != hipSuccess)
    return SANA_ERR_HIP;
  char* ws = static_cast<char*>(lease.ptr());
  uint16_t* qkv = reinterpret_cast<uint16_t*>(ws);
  float* k_ssq = norm ? reinterpret_cast<float*>(ws + qkv_bytes) : nullptr;
  // The blocked copy of x and the attention workspace share a region: the GEMM is done with the first
  // before the attention kernels use the second (stream order).
  char* region = ws + qkv_bytes + ssq_bytes;
  hipError_t e = sanala::launch_relayout_k32(static_cast<const uint16_t*>(x), M, (int)C,
                                             reinterpret_cast<uint16_t*>(region), stream);
  if (e == hipSuccess)
    e = sanala::launch_qkv_gemm(reinterpret_cast<const uint16_t*>(region), static_cast<const uint16_t*>(Wqkv), qkv, M,
                                (int)C, stream, k_ssq);
  if (e == hipSuccess)
    e = sanala::launch_attn(plan, qkv, 3 * C, qkv + C, qkv + 2 * C, 3 * C, gq, gk, eps, out, C, region, stream, k_ssq,
                            k_parts);
  return e == hipSuccess ? SANA_OK : SANA_ERR_HIP;
}


extern "C" sana_status_t sana_mix_ffn_fwd(const void* x, const void* W1, const void* Wdw, const void* W2, int B,
                                          int Hg, int Wg, int C, int F, void* out, hipStream_t stream) {
  if (!x || !W1 || !Wdw || !W2 || !out) return SANA_ERR_INVALID_ARG;
  if (B < 1 || Hg < 1 || Wg < 1 || C < 1 || F < 1) return SANA_ERR_INVALID_ARG;
  if (C % 32 != 0 || F % 32 != 0 || Wg > sanala::mix_ffn_max_width() || B > 65535) return SANA_ERR_UNSUPPORTED;
  if (C > (1 << 20) || F > (1 << 20)) return SANA_ERR_UNSUPPORTED;
  const int64_t M = (int64_t)B * Hg * Wg;
  if (M > (int64_t(1) << 30) || (double)M * 2.0 * F >= 1099511627776.0) return SANA_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W2) || !aligned16(out) || (reinterpret_cast<uintptr_t>(Wdw) & 1))
    return SANA_ERR_MISALIGNED;
  const size_t xbytes = (size_t)M * C * 2;
  if (overlaps(out, xbytes, x, xbytes) || overlaps(out, xbytes, W1, (size_t)C * 2 * F * 2) ||
      overlaps(out, xbytes, W2, (size_t)F * C * 2) || overlaps(out, xbytes, Wdw, (size_t)2 * F * 9 * 2))
    return SANA_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SANA_ERR_HIP;
  init_pool(dev);
  g_timing.count = 0;
  ScratchLease lease;
  if (lease.acquire(dev, stream, sanala::mix_ffn_workspace_bytes(M, C, F)) != hipSuccess) return SANA_ERR_HIP;
  const hipError_t e = sanala::launch_mix_ffn(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W1),
                                              static_cast<const uint16_t*>(Wdw), static_cast<const uint16_t*>(W2), B,
                                              Hg, Wg, C, F, static_cast<uint16_t*>(out), lease.ptr(), stream);
  return e == hipSuccess ? SANA_OK : SANA_ERR_HIP;
}

extern "C" sana_status_t sana_cross_attn_fwd(const void* q, const void* k, const void* v, const float* gq,
                                             const float* gk, const int* kv_len, int B, int N, int L, int H, int D,
                                             float eps, void* out, hipStream_t stream, sana_dtype_t dtype) {
  if (!q || !k || !v || !out) return SANA_ERR_INVALID_ARG;
  if (dtype != SANA_F32 && dtype != SANA_BF16 && dtype != SANA_F16) return SANA_ERR_INVALID_ARG;
  if (B <= 0 || N <= 0 || L <= 0 || H <= 0 || D <= 0) return SANA_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.f || (gq == nullptr) != (gk == nullptr)) return SANA_ERR_INVALID_ARG;
  if (dtype != SANA_BF16 || D != sanala::kHeadDim || H > sanala::cross_attn_max_heads() ||
      L > sanala::cross_attn_max_keys() || B > 65535)
    return SANA_ERR_UNSUPPORTED;
  const double qelems = (double)B * N * H * D;
  if (qelems >= 1099511627776.0) return SANA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (gq && !aligned16(gq)) ||
      (gk && !aligned16(gk)) || (reinterpret_cast<uintptr_t>(kv_len) & 3))
    return SANA_ERR_MISALIGNED;
  const size_t qbytes = (size_t)B * N * H * D * 2, kbytes = (size_t)B * L * H * D * 2;
  if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, k, kbytes) || overlaps(out, qbytes, v, kbytes))
    return SANA_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SANA_ERR_HIP;
  init_pool(dev);
  g_timing.count = 0;
  ScratchLease lease;
  if (lease.acquire(dev, stream, sanala::cross_attn_workspace_bytes(B, N, L, H)) != hipSuccess) return SANA_ERR_HIP;
  const hipError_t e = sanala::launch_cross_attn(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                                 static_cast<const uint16_t*>(v), gq, gk, kv_len, B, N, L, H, eps,
                                                 static_cast<uint16_t*>(out), lease.ptr(), stream);
  return e == hipSuccess ? SANA_OK : SANA_ERR_HIP;
}

extern "C" sana_status_t sana_quantize_rows_i8(const void* x, int64_t rows, int C, void* xq, float* x_scale,
                                               hipStream_t stream) {
  if (!x || !xq || !x_scale || rows < 1 || C < 1) return SANA_ERR_INVALID_ARG;
  if (C % 8 != 0 || rows > (int64_t(1) << 32)) return SANA_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(xq)) return SANA_ERR_MISALIGNED;
  if (overlaps(xq, (size_t)rows * C, x, (size_t)rows * C * 2)) return SANA_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SANA_ERR_HIP;
  g_timing.count = 0;
  return sanala::launch_quant_rows(static_cast<const uint16_t*>(x), rows, C, static_cast<int8_t*>(xq), x_scale,
                                   stream) == hipSuccess
             ? SANA_OK
             : SANA_ERR_HIP;
}

extern "C" sana_status_t sana_pack_weight_i8(const void* Wt_q, int64_t rows, int C, void* Wt_p, hipStream_t stream) {
  if (!Wt_q || !Wt_p || rows < 1 || C < 1) return SANA_ERR_INVALID_ARG;
  if (C % 64 != 0 || rows > (int64_t(1) << 30) || rows * C > (int64_t(1) << 40)) return SANA_ERR_UNSUPPORTED;
  if (!aligned16(Wt_q) || !aligned16(Wt_p)) return SANA_ERR_MISALIGNED;
  const size_t bytes = (size_t)rows * C;
  if (overlaps(Wt_p, bytes, Wt_q, bytes)) return SANA_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SANA_ERR_HIP;
  g_timing.count = 0;
  return sanala::launch_pack_k64(static_cast<const int8_t*>(Wt_q), rows, C, static_cast<int8_t*>(Wt_p), stream) ==
                 hipSuccess
             ? SANA_OK
             : SANA_ERR_HIP;
}

extern "C" sana_status_t sana_qkv_w8a8_linear_attn_fwd(const void* x, const void* Wt_p, const float* w_scale,
                                                       const float* gq, const float* gk, int B, int N, int H, int D,
                                                       float eps, void* out, hipStream_t stream) {
  if (!x || !Wt_p || !w_scale || !out) return SANA_ERR_INVALID_ARG;
  sana_status_t st = check_common(B, N, H, D, eps, gq, gk);
  if (st != SANA_OK) return st;
  const int64_t C = (int64_t)H * D;
  if (C % 64 != 0) return SANA_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(Wt_p) || !aligned16(w_scale) || !aligned16(out)) return SANA_ERR_MISALIGNED;
  const int64_t M = (int64_t)B * N;
  const size_t xbytes = (size_t)M * C * 2;
  if (overlaps(out, xbytes, x, xbytes) || overlaps(out, xbytes, Wt_p, (size_t)C * 3 * C) ||
      overlaps(out, xbytes, w_scale, (size_t)C * 3 * 4))
    return SANA_ERR_INVALID_ARG;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SANA_ERR_HIP;
  init_pool(dev);
  g_timing.count = 0;
  const bool norm = gq != nullptr;
  const sanala::AttnPlan plan = sanala::plan_attn(B, N, H, sanala::kDtypeBf16, norm, true);
  // Stream-ordered scratch: int8 x and its row scales, the bf16 qkv, the K row partial sums of squares.
  const size_t xq_bytes = ((size_t)M * C + 255) / 256 * 256;
  const size_t sx_bytes = ((size_t)M * 4 + 255) / 256 * 256;
  const size_t qkv_bytes = ((size_t)M * 3 * C * 2 + 255) / 256 * 256;
  const int k_parts = norm ? sanala::qkv_gemm_k_parts((int)C, false) : 0;  // the int8 GEMM's panels
  const size_t ssq_bytes = ((size_t)M * k_parts * 4 + 255) / 256 * 256;
  ScratchLease lease;
  if (lease.acquire(dev, stream, xq_bytes + sx_bytes + qkv_bytes + ssq_bytes + plan.ws_bytes) != hipSuccess)
    return SANA_ERR_HIP;
  char* base = static_cast<char*>(lease.ptr());
  int8_t* xq = reinterpret_cast<int8_t*>(base);
  float* sx = reinterpret_cast<float*>(base + xq_bytes);
  uint16_t* qkv = reinterpret_cast<uint16_t*>(base + xq_bytes + sx_bytes);
  float* k_ssq = norm ? reinterpret_cast<float*>(base + xq_bytes + sx_bytes + qkv_bytes) : nullptr;
  hipError_t e = sanala::launch_quant_rows(static_cast<const uint16_t*>(x), M, (int)C, xq, sx, stream, true);
  if (e == hipSuccess)
    e = sanala::launch_qkv_gemm_i8(xq, static_cast<const int8_t*>(Wt_p), sx, w_scale, qkv, M, (int)C, stream, k_ssq);
  if (e == hipSuccess)
    e = sanala::launch_attn(plan, qkv, 3 * C, qkv + C, qkv + 2 * C, 3 * C, gq, gk, eps, out, C,
                            base + xq_bytes + sx_bytes + qkv_bytes + ssq_bytes, stream, k_ssq, k_parts);
  return e == hipSuccess ? SANA_OK : SANA_ERR_HIP;
}

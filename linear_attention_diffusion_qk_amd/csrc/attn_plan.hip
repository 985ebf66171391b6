// Launch planning and dtype dispatch of the linear attention.
#include "attn.h"

#include <algorithm>
#include <atomic>
#include <cstdlib>

namespace sanala {

namespace {
constexpr size_t kPartStrideBytes = (kHeadDim * kHeadDim + kHeadDim) * 4;
constexpr size_t kMaxLds = 160 * 1024;  // LDS per CU on gfx950

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  const int v = std::atoi(s);
  return v > 0 ? v : dflt;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int device_cus() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      v > 0)
    return v;
  return 256;
}
}  // namespace

int max_heads() { return 320; }

uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{0};
  uint32_t e = counter.fetch_add(1) + 1;
  while (e == 0) e = counter.fetch_add(1) + 1;  // 0 is what fresh memory holds
  return e;
}

AttnPlan plan_attn(int B, int N, int H, int dtype, bool norm, bool fused) {
  AttnPlan p{};
  p.B = B;
  p.N = N;
  p.H = H;
  p.dtype = dtype;
  p.norm = norm;
  p.num_cus = device_cus();
  const bool bf = dtype != kDtypeF32;  // 16-bit storage: the bf16 / binary16 kernels
  // KV chunking.  fp32: about 1024 blocks, chunks of at least 256 tokens (the partial state costs 33/Tc
  // of the K+V traffic).  16-bit state kernel (block = head pair x chunk, five resident per CU): the
  // chunk length minimising a cost model fitted to MI355X measurements -- a block streams 256 bytes per
  // token at about 12 GB/s, a CU at about 23 GB/s, and a split sequence adds the reduction (a launch of
  // about 6 us plus 0.2 us per chunk, plus 0.0045 us per (sample, head) state beyond 280: the reduction
  // takes 4-5 us up to 4 samples of 70 heads, but 12.8 us for 30 samples in 4 chunks and 14 us for 32 in
  // 2; without that term 16 and 30 samples of 1024 tokens were split into 4 chunks of 256, 77.3 and
  // 137.3 us per call against 68.8 and 124.8 us unsplit).  It picks 14 chunks of 1216 tokens on the 4K
  // workload (73-75 us per call against 75-77 us for 29 of 576, and 77.8 us for 15 of 1152, whose 525
  // blocks leave 13 CUs a third chunk), one chunk per sample for batches of 1024-token samples (no
  // reduction), and 8 chunks of 128 for a single 1024-token sample.
  const int groups = bf ? (H + 1) / 2 : H;
  const int64_t per_chunk = (int64_t)B * groups;
  const int n64 = (N + 63) / 64 * 64;
  int Tc;
  if (bf) {
    // Chunks shorter than 256 tokens only for a single sample of up to 8192 tokens or up to 2048 tokens in
    // all: in larger batches their many partials cost more to reduce than the model's reduction term says
    // (8 x 1024 tokens: 49.5 us per call with the short chunks it chose, 46.5 us with 256; 4 x 1024: 33.6
    // against 32.4 us; 2 x 1024 keeps them: 22.9-23.9 against 24.2 us).
    const int min_chunk = std::min(n64, ((B == 1 && N <= 8192) || (int64_t)B * N <= 2048) ? 64 : 256);
    double best = 1e30;
    Tc = n64;
    for (int t = min_chunk; t <= n64; t += 64) {
      const int64_t nc = (N + t - 1) / t;
      if (t > min_chunk && (N + t - 64 - 1) / (t - 64) == nc) continue;  // same split, shorter chunks
      const int64_t blocks = per_chunk * nc;
      const int64_t per_cu = (blocks + p.num_cus - 1) / p.num_cus;
      const double stream_us = std::max(0.021 * t, 0.0111 * (double)per_cu * t);
      const double heads_beyond = std::max(0.0, (double)B * H - 280.0);
      const double cost = stream_us + (nc > 1 ? 6.0 + 0.2 * (double)nc + 0.0045 * heads_beyond : 0.0);
      if (cost < best) {
        best = cost;
        Tc = t;
      }
    }
  } else {
    const int nc = (int)std::max<int64_t>(1, (1024 + per_chunk - 1) / per_chunk);
    Tc = ((N + nc - 1) / nc + 63) / 64 * 64;
    Tc = std::max(Tc, std::min(256, n64));
  }
  Tc = env_int("SANA_KV_CHUNK", Tc);
  Tc = std::max(Tc, (N + 65535) / 65536);  // at most 65536 chunks: partial offsets stay within 32 bits
  Tc = std::max(64, (Tc + 63) / 64 * 64);
  p.Tc = Tc;
  p.NC = (N + Tc - 1) / Tc;
  // bf16 output kernel: persistent when the sample's operands fit in LDS and there are enough tiles to
  // fill the device (SANA_OUT_KERNEL=2 asks for the tile kernel).
  const int64_t tiles = (int64_t)B * ((N + 15) / 16);
  const int out_env = env_int("SANA_OUT_KERNEL", 0);
  if (bf && H <= 2 * kPersistPPW * kPersistMaxWaves && out_persist_lds_bytes(H) <= kMaxLds && tiles >= 2 * p.num_cus && out_env != kOutTile &&
      out_env != kOutTileGroups)
    p.out_kind = kOutPersist;
  else if (bf && ((tiles < 2 * p.num_cus && out_env != kOutTile) || out_env == kOutTileGroups))
    p.out_kind = kOutTileGroups;  // too few tiles for one per CU: split the heads over blocks
  else
    p.out_kind = kOutTile;
  // Strided tiles once a sample spans at least two tiles per block (so that a block's tiles stay within
  // few samples); SANA_OUT_SCHED=1 asks for contiguous runs.
  {
    const int64_t blocks = std::min<int64_t>(p.num_cus, tiles);
    p.out_strided = p.out_kind == kOutPersist && (N + 15) / 16 >= 2 * blocks && env_int("SANA_OUT_SCHED", 2) != 1;
    // Otherwise, when a sample's tiles split evenly into runs of the per-block count, the blocks of a
    // sample take its tiles interleaved, so that they too sweep the sample together (SANA_OUT_SCHED=1
    // asks for plain contiguous runs).
    const int64_t per = blocks > 0 ? (tiles + blocks - 1) / blocks : 1;
    const int tps = (N + 15) / 16;
    p.out_group = p.out_kind == kOutPersist && !p.out_strided && env_int("SANA_OUT_SCHED", 2) != 1 && tps % per == 0
                      ? (int)(tps / per)
                      : 0;
  }
  // K row statistics inside the state pass (one read of K), for calls whose output kernel forms r_q
  // itself: SANA_STATE_XCHG=1 asks for it (off by default: on MI355X it measures slower than the
  // separate row-statistics pass followed by the plain state pass).  SANA_XCHG_SPIN_US: the wait limit
  // of the cross-block waits (this exchange and the chunk rendezvous) in microseconds (default 200; 0
  // makes every wait that is not met at once take the local route, which gives the same bits).
  {
    const char* s = std::getenv("SANA_STATE_XCHG");
    const bool on = s && s[0] == '1' && s[1] == 0;
    p.state_xchg = bf && norm && p.out_kind != kOutTileGroups && on;
  }
  // A split sequence (16-bit path) is reduced by a launch of its own (kv_reduce).  SANA_STATE_RENDEZVOUS=1
  // asks the state blocks to reduce the chunk partials among themselves instead, where every block of
  // the grid can be resident at once (five per CU) and there are at most 16 chunks.  The two routes sum
  // in the same order and give the same bits; on MI355X the rendezvous saves the launch but its tail
  // costs as much (4K workload 68.5 against 68.2 us per call, 1024 tokens 18.7 against 18.3 us), so it
  // is off by default.
  {
    const char* s = std::getenv("SANA_STATE_RENDEZVOUS");
    const bool on = s && s[0] == '1' && s[1] == 0;
    p.rendezvous = bf && p.NC > 1 && p.NC <= 16 && (int64_t)B * groups * p.NC <= 5 * (int64_t)p.num_cus && on;
  }
  // K and V are read with non-temporal loads (the row-statistics pass and the 16-bit state pass are their
  // last readers, and the output pass then finds more of Q in the caches) when together they exceed the
  // 256 MB Infinity Cache, and behind the fused projection.  Measured on MI355X, per call, ordinary ->
  // non-temporal: 32 x 1024 tokens 139.7 -> 127.9 us, 2 x 16384 129.8 -> 123.5, 4 x 8192 136.1 -> 134.3,
  // the 2K fused front end (4 x 4096) 542.7 -> 537.7 and its W8A8 form 402.0 -> 394.5; below the cache
  // size the other way: 1 x 16384 66.4 -> 67.7, 8 x 2048 73.9 -> 76.6, 2 x 4096 42.5 -> 43.8, and a
  // single 1024-token sample unchanged.  SANA_STATE_NT_V=0 or 1 forces either form.
  {
    const char* s = std::getenv("SANA_STATE_NT_V");
    const bool forced = s && (s[0] == '0' || s[0] == '1') && s[1] == 0;
    const double kv_bytes = 2.0 * (double)B * N * H * kHeadDim * (dtype == kDtypeF32 ? 4 : 2);
    p.nt_v = bf && !p.state_xchg && (forced ? s[0] == '1' : (fused || kv_bytes > 256.0 * 1024 * 1024));
  }
  {
    const char* s = std::getenv("SANA_XCHG_SPIN_US");
    const long us = (s && *s) ? std::atol(s) : 200;
    p.xchg_spin = (uint32_t)(std::min<long>(std::max<long>(us, 0), 10000000) * 100);
  }
  const size_t BH = (size_t)B * H;
  size_t off = 0;
  p.off_rk = off;   off = align_up(off + (norm ? (size_t)B * N * 4 : 0), 256);
  p.off_rq = off;
  off = align_up(off + (norm && (!bf || H > 72 || p.out_kind == kOutTileGroups) ? (size_t)B * N * 4 : 0), 256);
  p.off_part = off; off = align_up(off + (p.NC > 1 || !bf ? BH * p.NC * kPartStrideBytes : 0), 256);
  p.off_S32 = off;  off = align_up(off + (bf ? 0 : BH * kHeadDim * kHeadDim * 4), 256);
  p.off_z = off;    off = align_up(off + (bf ? 0 : BH * kHeadDim * 4), 256);
  p.off_Sop = off;  off = align_up(off + (bf ? bf16_operand_bytes((int64_t)BH, H) : 0), 256);
  p.off_xchg = off; off = align_up(off + (p.state_xchg ? kv_state_x_exchange_bytes((int64_t)B * N, H) : 0), 256);
  // Rendezvous flags, one word per (sample, head pair, chunk).
  p.off_flags = off; off = align_up(off + (p.rendezvous ? (size_t)B * groups * p.NC * 4 : 0), 256);
  p.ws_bytes = off;
  return p;
}

hipError_t launch_attn(const AttnPlan& p, const void* q, int64_t ldq, const void* k, const void* v, int64_t ldkv,
                       const float* gq, const float* gk, float eps, void* out, int64_t ldo, void* ws,
                       hipStream_t stream, const float* k_ssq, int k_parts) {
  if (p.dtype == kDtypeF32)
    return launch_attn_f32(p, static_cast<const float*>(q), ldq, static_cast<const float*>(k),
                           static_cast<const float*>(v), ldkv, gq, gk, eps, static_cast<float*>(out), ldo, ws, stream);
  return launch_attn_bf16(p, static_cast<const uint16_t*>(q), ldq, static_cast<const uint16_t*>(k),
                          static_cast<const uint16_t*>(v), ldkv, gq, gk, eps, static_cast<uint16_t*>(out), ldo, ws,
                          p.num_cus, stream, k_ssq, k_parts);
}

}  // namespace sanala

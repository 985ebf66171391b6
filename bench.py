#!/usr/bin/env python3
"""Throughput of libsanala's ReLU linear attention with QK-RMSNorm on one MI355X.

Prints ONE JSON line: tokens/s of the whole call on the 4K workload (B=1, N=16384 tokens, 70 heads x 32,
bf16 I/O, K with 1% outlier rows), achieved HBM GB/s against the 8 TB/s peak, the dominant kernel's
roofline, the 1024px workload (B=1, N=1024) as a secondary figure, and the fp64 oracle timed on the
host cores as a CPU baseline.

A step is one sana_linear_attn_fwd call over the resident inputs (row statistics, KV state, chunk
reduction and output: the whole path).

  python bench.py [--gpus 1] [--steps 50] [--warmup 1000] [--workload config4|config1|config2|config3|config5|w8a8|mixffn]
                  [--no-cold] [--no-secondary] [--no-cpu-baseline]
  python bench.py --mode copy        # plain device copy of known size (counter calibration under rocprofv3)
  python bench.py --summarize-trace TRACE.db WORKLOAD OUT.txt COMMAND...
                                     # rocprofv3 --kernel-trace database -> per-kernel summary under profiles/
  python bench.py --summarize-counters WORKLOAD OUT.txt "COMMANDS" PMC.db...
                                     # rocprofv3 --pmc databases -> per-kernel counter summary (MFMA busy, waits, ...)
  python bench.py --summarize-traffic KERNEL_FETCH.db KERNEL_WRITE.db COPY_FETCH.db COPY_WRITE.db [OUT [WORKLOAD [ENV]]]
                                     # rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE databases -> profiles/hbm_traffic.txt
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak
MFMA_I8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA peak

WORKLOADS = {
    "config1": dict(cfg=1, desc="512px linear attention, fp32: B=1, N=256 (16x16 latent), H=70, D=32, fp32 I/O, "
                                "QK-RMSNorm on"),
    "config4": dict(cfg=4, desc="4K linear attention: B=1, N=16384 (128x128 latent), H=70, D=32, bf16 I/O, "
                                "K ~ N(0,30^2) with 1% rows x100, QK-RMSNorm on"),
    "config2": dict(cfg=2, desc="1024px linear attention: B=1, N=1024 (32x32 latent), H=70, D=32, bf16 I/O, QK-RMSNorm on"),
    "config3": dict(cfg=3, desc="1024px repeat-sampling batch: B=32, N=1024, H=70, D=32, bf16 I/O, QK-RMSNorm on"),
    "config5": dict(cfg=5, desc="2K fused front end: x[4,4096,2240] bf16 @ Wqkv[2240,6720] -> linear attention H=70, D=32"),
    "w8a8": dict(cfg=5, desc="2K front end in W8A8: x[4,4096,2240] bf16 quantised per token, int8 Wt[6720,2240] "
                             "with column scales -> linear attention H=70, D=32 on bf16 qkv"),
    "mixffn": dict(cfg=5, desc="2K Mix-FFN: x[4, 64x64, 2240] bf16 @ W1[2240,11200] -> 3x3 depthwise conv (zero pad) "
                               "-> GLU -> @ W2[5600,2240]"),
    "cross4k": dict(cfg=6, N=16384, desc="4K cross-attention with QK-RMSNorm: B=1, N=16384 image tokens (128x128 "
                                         "latent), L=300 text tokens, H=70, D=32, bf16"),
    "cross1k": dict(cfg=6, N=1024, desc="1024px cross-attention with QK-RMSNorm: B=1, N=1024 image tokens, L=300 text "
                                        "tokens, H=70, D=32, bf16"),
}
# Cross-attention: the softmax's exp2 runs on the vector ALU at a quarter of the fp32 rate; from the
# fp32 vector peak (157.3 TFLOP/s = 78.6 T fused multiply-adds/s) that is 19.66 T exponentials/s.
EXP2_PEAK_T = 157.3 / 2 / 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_diffusion_qk_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on these sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("source_hash") != source_hash() or rec.get("workload") != workload:
        return None
    val = rec.get(f"{kernel}_bytes_per_launch")
    return float(val) if val else None


class Inputs:
    def __init__(self, name: str):
        import torch
        from synth import gen_config
        self.name = name
        self.spec = WORKLOADS[name]
        t0 = time.time()
        if name == "w8a8":
            from synth import gen_w8a8
            inp = gen_w8a8(self.spec["cfg"], 4, 4096)
            self.kind = "w8a8"
        elif name == "mixffn":
            from synth import gen_mix_ffn
            inp = gen_mix_ffn(self.spec["cfg"], 4, 64, 64)
            self.kind = "mixffn"
        elif name.startswith("cross"):
            from synth import gen_cross
            inp = gen_cross(self.spec["cfg"], 1, self.spec["N"], L=300)
            self.kind = "cross"
        else:
            inp = gen_config(self.spec["cfg"])
            self.kind = "qkv" if self.spec["cfg"] == 5 else "attn"
        self.host = inp
        bf = torch.bfloat16
        g = lambda a: torch.from_numpy(a).to("cuda")  # noqa: E731
        if self.kind in ("attn", "cross"):
            tdt = torch.float32 if inp.dtype == "f32" else bf
            self.q, self.k, self.v = (torch.from_numpy(a).to("cuda").to(tdt) for a in (inp.q, inp.k, inp.v))
            self.out = torch.empty_like(self.q)
            if self.kind == "cross":
                self.kv_len = torch.from_numpy(inp.kv_len).to("cuda")
                self.L = inp.L
        elif self.kind == "qkv":
            self.x = torch.from_numpy(inp.x).to("cuda").to(bf)
            self.w = torch.from_numpy(inp.w).to("cuda").to(bf)
            self.out = torch.empty_like(self.x)
        elif self.kind == "mixffn":
            self.x, self.w1, self.kdw, self.w2 = (torch.from_numpy(a).to("cuda").to(bf)
                                                  for a in (inp.x, inp.w1, inp.kdw, inp.w2))
            self.out = torch.empty_like(self.x)
        else:
            self.x = torch.from_numpy(inp.x).to("cuda").to(bf)
            import linear_attention_diffusion_qk_amd as sanala
            # The int8 weight is laid out once, as at model load; the timed calls take the packed copy.
            self.wt = sanala.pack_weight_i8(torch.from_numpy(inp.wt_q).to("cuda"))
            self.sw = torch.from_numpy(inp.s_w).to("cuda")
            self.out = torch.empty_like(self.x)
        if self.kind == "mixffn":
            self.B, self.N, self.C = inp.x.shape
            self.H, self.D = self.C // 32, 32
        else:
            self.gq, self.gk = g(inp.gq), g(inp.gk)
            self.B, self.N, self.H, self.D = inp.B, inp.N, inp.H, inp.D
            self.C = self.H * self.D
        torch.cuda.synchronize()
        log(f"[bench] {name}: inputs generated and resident in {time.time() - t0:.1f}s")

    def step(self, sanala):
        if self.kind == "attn":
            sanala.sana_linear_attn_fwd(self.q, self.k, self.v, self.gq, self.gk, self.B, self.N, self.H, self.D,
                                        self.host.eps, self.out)
        elif self.kind == "qkv":
            sanala.sana_qkv_linear_attn_fwd(self.x, self.w, self.gq, self.gk, self.B, self.N, self.H, self.D,
                                            self.host.eps, self.out)
        elif self.kind == "mixffn":
            sanala.sana_mix_ffn_fwd(self.x, self.w1, self.kdw, self.w2, self.B, self.host.Hg, self.host.Wg, self.C,
                                    self.host.F, self.out)
        elif self.kind == "cross":
            sanala.sana_cross_attn_fwd(self.q, self.k, self.v, self.gq, self.gk, self.kv_len, self.B, self.N, self.L,
                                       self.H, self.D, self.host.eps, self.out)
        else:
            sanala.sana_qkv_w8a8_linear_attn_fwd(self.x, self.wt, self.sw, self.gq, self.gk, self.B, self.N, self.H,
                                                 self.D, self.host.eps, self.out)

    @property
    def esize(self) -> int:
        return 4 if getattr(self.host, "dtype", "bf16") == "f32" else 2

    def algorithmic_bytes(self) -> int:
        """Read Q, K, V and write O once: 4 * B * N * C * element size bytes (cross-attention: Q and O over
        the N image tokens, K and V over the L text tokens)."""
        if self.kind == "cross":
            return 2 * self.B * (self.N + self.L) * self.C * self.esize
        return 4 * self.B * self.N * self.C * self.esize

    def kernel_bytes(self, kernel: str) -> float:
        tok = self.B * self.N * self.C * self.esize
        if kernel in ("kv_state", "kv_partial"):
            return 2 * tok            # read K and V
        if kernel == "out":
            return 2 * tok            # read Q, write O
        if kernel in ("rowstats_k", "rowstats_q"):
            return tok                # read one tensor
        if kernel == "fused":
            return 4 * tok
        if kernel == "cross_attn":
            return self.algorithmic_bytes()
        return 0.0


def time_steps(inputs: Inputs, sanala, steps: int, warmup: int) -> float:
    import torch
    for _ in range(warmup):
        inputs.step(sanala)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        inputs.step(sanala)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per step


def time_steady(inputs: Inputs, sanala, steps: int, settle_s: float = 0.2) -> float:
    """ms per step of back-to-back calls after at least settle_s seconds of calls: the GPU's clocks rise
    over the first tens of milliseconds of work after idle (on MI355X the first 50 calls of the 4K
    workload ran 8% slower than steady state, those of the 4K cross-attention 22%), which a short
    warm-up leaves partly inside the timed steps."""
    import time
    import torch
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(20):
            inputs.step(sanala)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        inputs.step(sanala)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_graph(inputs: Inputs, sanala, per_graph: int = 20, replays: int = 50) -> float:
    """Per-call time of the allocation-free call replayed from a HIP graph (torch.cuda.CUDAGraph) that holds
    `per_graph` calls back to back: the same kernels with no host work between the calls."""
    import torch
    i = inputs

    def call():
        sanala.sana_linear_attn_fwd_noalloc(i.q, i.k, i.v, i.gq, i.gk, i.B, i.N, i.H, i.D, i.host.eps, i.out)

    call()  # the static scratch's address and the kernels' LDS limits are set up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            call()
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * per_graph)


def pct(xs, q: float) -> float:
    """q-quantile of xs (linear interpolation between order statistics)."""
    v = sorted(xs)
    pos = q * (len(v) - 1)
    lo = int(pos)
    hi = min(lo + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (pos - lo)


def spread(us) -> dict:
    return {"median": round(pct(us, 0.5), 2), "p10": round(pct(us, 0.1), 2), "p90": round(pct(us, 0.9), 2)}


def time_rounds(inputs: Inputs, sanala, rounds: int = 20, per: int = 10) -> list:
    """us per call in each of `rounds` rounds of `per` back-to-back calls (one event pair per round, so no
    event packets sit between the calls; run after time_steady, with settled clocks)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(rounds)]
    for e0, e1 in evs:
        e0.record()
        for _ in range(per):
            inputs.step(sanala)
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) / per * 1e3 for e0, e1 in evs]


class CacheFlush:
    """A read-only pass over 1 GiB between timed calls: evicts the L2s and the 256 MB Infinity Cache and
    leaves only clean lines behind (a write pass would leave dirty lines whose write-back lands on the
    next kernels).  Runs outside the timing events."""

    def __init__(self, nbytes: int = 1 << 30):
        import torch
        self.buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda")

    def __call__(self):
        import torch
        torch.sum(self.buf, dim=0, out=self.sink)


def time_cold(inputs: Inputs, sanala, steps: int, warmup: int, flush: CacheFlush):
    """(mean ms per call, us of each call) with the caches flushed before every call (flush outside the events): the inputs
    come from HBM, as when the call follows unrelated work."""
    import torch
    for _ in range(warmup):
        flush()
        inputs.step(sanala)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        flush()
        e0.record()
        inputs.step(sanala)
        e1.record()
    torch.cuda.synchronize()
    times = [e0.elapsed_time(e1) for e0, e1 in evs]
    return sum(times) / steps, [t * 1e3 for t in times]


def copy_ceiling(reps: int = 20):
    """Measured bandwidth ceilings beside the 8 TB/s spec: a plain device-to-device copy of 256 MiB
    (torch's copy kernel; reads and writes 256 MiB each) and a read-only reduction over 1 GiB."""
    import torch
    n = 256 * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    big = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    out = {}
    for name, fn, nbytes in (("copy", lambda: dst.copy_(src), 2 * n), ("read", lambda: torch.sum(big, dim=0, out=sink), 1 << 30)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"{name}_GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    out["note"] = ("device copy of 256 MiB (bytes read + written) and a read-only sum over 1 GiB, torch kernels, "
                   f"{reps} back-to-back launches each; spec peak {HBM_PEAK_GBPS:.0f} GB/s")
    del src, dst, big
    return out


def point(inputs: Inputs, ms: float) -> dict:
    b = inputs.algorithmic_bytes()
    gbps = b / (ms * 1e-3) / 1e9
    return {"ms_per_step": round(ms, 5), "tokens_per_s": round(inputs.B * inputs.N / (ms * 1e-3), 1),
            "achieved_GBps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def host_cpu() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "usable_cpus": affinity}


def kernel_times(inputs: Inputs, sanala, reps: int = 20, lead: int = 4):
    """Average per-kernel duration from the start/stop events of each kernel's own dispatch (library timing).
    Each timed call is queued behind `lead` untimed ones, so that it runs on a busy GPU as the calls of a
    back-to-back run do (reading a call's events waits for it, which would otherwise leave the GPU idle
    before every timed call)."""
    acc = {}
    try:
        for _ in range(reps):
            sanala.sana_timing_enable(False)
            for _ in range(lead):
                inputs.step(sanala)
            sanala.sana_timing_enable(True)
            inputs.step(sanala)
            for name, ms in sanala.sana_timing_last():
                acc.setdefault(name, []).append(ms)
    finally:
        sanala.sana_timing_enable(False)
    return {k: sum(v) / len(v) for k, v in acc.items()}


def cpu_baseline(inputs: Inputs, min_seconds: float = 12.0, max_reps: int = 200):
    """The fp64 oracle as it stands, on the same host arrays, repeated until >= min_seconds of CPU work
    (about 12-15 s on the 4K workload)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    h = inputs.host
    reps, t0 = 0, time.time()
    while True:
        if inputs.kind == "attn":
            oracle.linear_attn(h.q, h.k, h.v, h.gq, h.gk, h.H, h.D, h.eps)
        elif inputs.kind == "qkv":
            oracle.qkv_linear_attn(h.x, h.w, h.gq, h.gk, h.H, h.D, h.eps)
        elif inputs.kind == "mixffn":
            oracle.mix_ffn(h.x, h.w1, h.kdw, h.w2, h.Hg, h.Wg)
        elif inputs.kind == "cross":
            oracle.cross_attn(h.q, h.k, h.v, h.gq, h.gk, h.H, h.D, h.eps, kv_len=h.kv_len)
        else:
            oracle.qkv_w8a8_linear_attn(h.x, h.wt_q, h.s_w, h.gq, h.gk, h.H, h.D, h.eps)
        reps += 1
        el = time.time() - t0
        if el >= min_seconds or reps >= max_reps:
            break
    tokens = h.B * h.N * reps
    res = {"value": tokens / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{reps} full passes of the {inputs.name} workload ({h.B}x{h.N} tokens each) "
                     f"through the fp64 NumPy oracle in {el:.1f}s; cores = the BLAS threads it ran on"}
    res.update(host_cpu())
    return res


def run_copy_calibration():
    """A plain device-to-device copy of 256 MiB, five times: reads and writes 268,435,456 bytes per launch."""
    import torch
    n = 256 * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy", "bytes_per_launch": n}))


def _pmc_means(db: str, counter: str):
    """Mean counter value per kernel name in a rocprofv3 --pmc database."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, value from counters_collection where counter_name = ?", (counter,)).fetchall()
    acc = {}
    for name, val in rows:
        acc.setdefault(name, []).append(float(val))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_traffic(kfetch: str, kwrite: str, cfetch: str, cwrite: str, workload: str = "config4",
                      env: str = "") -> str:
    """Per-dispatch HBM bytes of each libsanala kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    scaled by what the same counters read for a plain device copy of 268,435,456 bytes.  `env`: the
    environment settings the kernel runs were made with (shown in the commands)."""
    pre = f"{env} " if env else ""
    copy_bytes = 256 * 1024 * 1024
    pick = lambda d: max((v for k, v in d.items() if "copy" in k.lower() or "elementwise" in k.lower()), default=None)  # noqa: E731
    cf, cw = pick(_pmc_means(cfetch, "FETCH_SIZE")), pick(_pmc_means(cwrite, "WRITE_SIZE"))
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    kf, kw = _pmc_means(kfetch, "FETCH_SIZE"), _pmc_means(kwrite, "WRITE_SIZE")
    lines = ["# HBM traffic per dispatch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (separate runs).",
             "# Counter KiB x 1024 x calibration; calibration = 268435456 / (counter bytes of a plain",
             "# device copy of 268435456 bytes, bench.py --mode copy).",
             "# Commands (from /tmp, TMPDIR=/tmp, one pass each):",
             f"#   {pre}rocprofv3 --pmc FETCH_SIZE -d kfetch -o run -- python3 /root/repo/bench.py --steps 2 --warmup 1 "
             f"--no-cpu-baseline --no-secondary --no-cold --workload {workload}",
             f"#   {pre}rocprofv3 --pmc WRITE_SIZE -d kwrite -o run -- (same bench command)",
             "#   rocprofv3 --pmc FETCH_SIZE -d cfetch -o run -- python3 /root/repo/bench.py --mode copy",
             "#   rocprofv3 --pmc WRITE_SIZE -d cwrite -o run -- python3 /root/repo/bench.py --mode copy",
             "#   python3 bench.py --summarize-traffic kfetch/run_results.db kwrite/run_results.db "
             "cfetch/run_results.db cwrite/run_results.db",
             f"workload: {workload}", f"source_hash: {source_hash()}",
             f"fetch_calibration: {f_scale:.4f}", f"write_calibration: {w_scale:.4f}"]
    short = {"rowstats": "rowstats_k", "kv_state_x": "kv_state_x", "kv_state": "kv_state", "kv_reduce": "kv_reduce",
             "out_persist": "out", "out_bf16": "out", "qkv_gemm": "qkv_gemm"}
    for name in sorted(set(kf) | set(kw)):
        tag = next((v for k, v in short.items() if k in name), None)
        if tag is None or "sanala" not in name:
            continue
        fb = kf.get(name, 0.0) * 1024.0 * f_scale
        wb = kw.get(name, 0.0) * 1024.0 * w_scale
        lines.append(f"{tag}_fetch_bytes_per_launch: {fb:.0f}")
        lines.append(f"{tag}_write_bytes_per_launch: {wb:.0f}")
        lines.append(f"{tag}_bytes_per_launch: {fb + wb:.0f}")
    return "\n".join(lines) + "\n"


def summarize_trace(db: str, workload: str, command: str) -> str:
    """Per-kernel duration statistics of a rocprofv3 --kernel-trace database (its `kernels` view)."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels").fetchall()
    acc = {}
    for name, dur in rows:
        acc.setdefault(name, []).append(float(dur) / 1000.0)  # ns -> us
    total = sum(sum(v) for v in acc.values())

    def short(name: str) -> str:
        n = name.split("(")[0]
        return n.replace("void ", "").replace("sanala::", "").replace("at::native::", "torch ")

    lines = [f"# rocprofv3 kernel-trace summary: {WORKLOADS[workload]['desc']}",
             f"# Command (from /tmp, TMPDIR=/tmp): {command}",
             f"# source_hash {source_hash()}",
             "# Calls include warm-up and the per-kernel event-timed repetitions of bench.py.",
             "#",
             f"# {'kernel':58s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share%':>7s}"]
    for name, v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"  {short(name)[:58]:58s} {len(v):6d} {sum(v) / len(v):9.2f} {min(v):9.2f} {max(v):9.2f} "
                     f"{100.0 * sum(v) / total:7.2f}")
    return "\n".join(lines) + "\n"


def summarize_counters(dbs, workload: str, command: str) -> str:
    """Per-kernel means of the counters in rocprofv3 --pmc databases (one pass each), with derived
    figures: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE of one XCD x 1024 SIMDs); waves waiting to
    issue = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES, waiting on anything = SQ_WAIT_ANY / SQ_WAVE_CYCLES; LDS
    bank conflicts per LDS-active cycle; L2 hit rate = TCC_HIT / (TCC_HIT + TCC_MISS)."""
    import sqlite3
    per = {}
    for db in dbs:
        con = sqlite3.connect(db)
        rows = con.execute("select kernel_name, counter_name, value from counters_collection").fetchall()
        for name, ctr, val in rows:
            per.setdefault(name, {}).setdefault(ctr, []).append(float(val))
    lines = [f"# rocprofv3 counter summary: {WORKLOADS[workload]['desc']}",
             f"# Commands (from /tmp, TMPDIR=/tmp), one counter pass each: {command}",
             f"# source_hash {source_hash()}",
             "# Values are means per dispatch (GRBM_GUI_ACTIVE as stored: summed over the 8 XCDs).  Derived:",
             "# mfma_busy% = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs); wait_issue% =",
             "# SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; wait_any% = SQ_WAIT_ANY / SQ_WAVE_CYCLES;",
             "# lds_conflict% = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; l2_hit% = TCC_HIT / (TCC_HIT + TCC_MISS)."]
    for name, ctrs in sorted(per.items()):
        if "sanala" not in name:
            continue
        m = {c: sum(v) / len(v) for c, v in ctrs.items()}
        short = name.split("(")[0].replace("void ", "").replace("sanala::", "")
        lines.append(f"kernel: {short}")
        for c in sorted(m):
            lines.append(f"  {c}: {m[c]:.6g}")
        g = m.get("GRBM_GUI_ACTIVE")
        if g and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            # the database holds GRBM_GUI_ACTIVE summed over the 8 XCDs; the busy-cycle ratio wants one XCD's
            lines.append(f"  gpu_active_cycles_per_xcd: {g / 8:.6g}")
            lines.append(f"  mfma_busy%: {100.0 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (g / 8 * 1024):.1f}")
        if m.get("SQ_WAVE_CYCLES"):
            if "SQ_WAIT_INST_ANY" in m:
                lines.append(f"  wait_issue%: {100.0 * m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.1f}")
            if "SQ_WAIT_ANY" in m:
                lines.append(f"  wait_any%: {100.0 * m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.1f}")
        if m.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in m:
            lines.append(f"  lds_conflict%: {100.0 * m['SQ_LDS_BANK_CONFLICT'] / m['SQ_LDS_IDX_ACTIVE']:.2f}")
        hit, miss = m.get("TCC_HIT_sum", m.get("TCC_HIT")), m.get("TCC_MISS_sum", m.get("TCC_MISS"))
        if hit is not None and miss is not None and hit + miss > 0:
            lines.append(f"  l2_hit%: {100.0 * hit / (hit + miss):.1f}")
    return "\n".join(lines) + "\n"


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        # --summarize-counters WORKLOAD OUTFILE "COMMAND" DB...
        text = summarize_counters(sys.argv[5:], sys.argv[2], sys.argv[4])
        with open(sys.argv[3], "w") as f:
            f.write(text)
        print(text)
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        # --summarize-trace DB WORKLOAD OUTFILE COMMAND...
        text = summarize_trace(sys.argv[2], sys.argv[3], " ".join(sys.argv[5:]))
        with open(sys.argv[4], "w") as f:
            f.write(text)
        print(text)
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-traffic":
        # --summarize-traffic KFETCH KWRITE CFETCH CWRITE [OUTFILE [WORKLOAD [ENV]]]
        out = sys.argv[6] if len(sys.argv) > 6 else os.path.join(ROOT, "profiles", "hbm_traffic.txt")
        text = summarize_traffic(*sys.argv[2:6], workload=sys.argv[7] if len(sys.argv) > 7 else "config4",
                                 env=sys.argv[8] if len(sys.argv) > 8 else "")
        with open(out, "w") as f:
            f.write(text)
        print(text)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 1000 untimed calls by default (about 70 ms on the 4K workload): the GPU's clocks settle within the
    # first 20-40 ms of work after idle, so a shorter warm-up leaves part of that ramp in the timed calls.
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="config4", choices=sorted(WORKLOADS))
    ap.add_argument("--mode", default="bench", choices=["bench", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the flushed-cache timings and the copy ceiling")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.mode == "copy":
        run_copy_calibration()
        return

    import linear_attention_diffusion_qk_amd as sanala
    sanala.load_library()

    main_in = Inputs(args.workload)
    ms = time_steps(main_in, sanala, args.steps, args.warmup)
    tokens = main_in.B * main_in.N
    value = tokens / (ms * 1e-3)
    alg_bytes = main_in.algorithmic_bytes()
    call_gbps = alg_bytes / (ms * 1e-3) / 1e9
    log(f"[bench] {args.workload}: {ms * 1e3:.1f} us/step, {value:.4g} tokens/s, {call_gbps:.0f} GB/s algorithmic")
    steady = None
    if main_in.kind in ("attn", "cross"):
        sts = time_steady(main_in, sanala, max(args.steps, 200))
        steady = point(main_in, sts)
        steady["note"] = ("back-to-back calls after 0.2 s of calls, once the clocks have settled; value above: "
                          "the contract's warm-up steps, then the timed steps")
        steady["per_call_us"] = spread(time_rounds(main_in, sanala))
        steady["per_call_us"]["note"] = "over 20 rounds of 10 back-to-back calls (one event pair per round)"
        log(f"[bench] {args.workload} steady state: {sts * 1e3:.1f} us/step")
    cold = None
    flush = None
    if not args.no_cold and main_in.kind in ("attn", "qkv", "w8a8", "cross"):
        flush = CacheFlush()
        cms, cold_us = time_cold(main_in, sanala, args.steps, max(1, args.warmup // 2), flush)
        cold = point(main_in, cms)
        cold["note"] = "1 GiB read-only pass before every call, outside the events"
        cold["per_call_us"] = spread(cold_us)
        log(f"[bench] {args.workload} cold: {cms * 1e3:.1f} us/step")

    kt = kernel_times(main_in, sanala)
    log(f"[bench] per-kernel (events): " + ", ".join(f"{k}={v * 1e3:.1f}us" for k, v in kt.items()))
    if main_in.kind == "mixffn":
        F = main_in.host.F
        gemm_ms = kt.get("gemm_expand", float("nan"))
        flops = 2.0 * tokens * main_in.C * 2 * F
        ach = flops / (gemm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "gemm_expand", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                "avg_launch_us": round(gemm_ms * 1e3, 2), "algorithmic_per_launch": flops}
        cb = tokens * (2 * F + F) * 2
        conv_ms = kt.get("dwconv_glu", float("nan"))
        roof["dwconv_glu"] = {"bound": "hbm", "achieved": round(cb / (conv_ms * 1e-3) / 1e9, 1),
                              "peak": HBM_PEAK_GBPS, "unit": "GB/s", "algorithmic_per_launch": cb,
                              "avg_launch_us": round(conv_ms * 1e3, 2)}
    elif main_in.kind == "cross":
        # The dominant kernel is bound by the softmax's exponentials on the vector ALU: one per (image token,
        # valid text token, head); its HBM rate and MFMA rate are given beside it.
        cms = kt.get("cross_attn", float("nan"))
        exps = float(main_in.N * int(main_in.kv_len.sum().item()) * main_in.H)
        ach = exps / (cms * 1e-3) / 1e12
        flops = 4.0 * main_in.N * int(main_in.kv_len.sum().item()) * main_in.C
        kb = main_in.algorithmic_bytes()
        roof = {"bound": "alu", "kernel": "cross_attn", "achieved": round(ach, 2), "peak": round(EXP2_PEAK_T, 2),
                "unit": "T exp2/s", "frac": round(ach / EXP2_PEAK_T, 4), "traffic": None,
                "avg_launch_us": round(cms * 1e3, 2), "algorithmic_per_launch": exps,
                "hbm": {"achieved": round(kb / (cms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "algorithmic_per_launch": kb},
                "mfma": {"achieved": round(flops / (cms * 1e-3) / 1e12, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "algorithmic_per_launch": flops}}
    elif main_in.kind in ("qkv", "w8a8"):
        gname = "qkv_gemm" if main_in.kind == "qkv" else "qkv_gemm_i8"
        peak = MFMA_BF16_PEAK_TFLOPS if main_in.kind == "qkv" else MFMA_I8_PEAK_TOPS
        gemm_ms = kt.get(gname, float("nan"))
        flops = 2.0 * tokens * main_in.C * 3 * main_in.C
        ach = flops / (gemm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": gname, "achieved": round(ach, 1), "peak": peak,
                "unit": "TFLOP/s" if main_in.kind == "qkv" else "TOP/s", "frac": round(ach / peak, 4),
                "traffic": None, "avg_launch_us": round(gemm_ms * 1e3, 2), "algorithmic_per_launch": flops}
    else:
        dom = max((k for k in kt if main_in.kernel_bytes(k) > 0), key=lambda k: kt[k])
        kb = main_in.kernel_bytes(dom)
        ach = kb / (kt[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": stored_traffic(dom, args.workload),
                "avg_launch_us": round(kt[dom] * 1e3, 2), "algorithmic_per_launch": kb}

    secondary = None
    if not args.no_secondary and args.workload == "config4":
        sec_in = Inputs("config2")
        sms = time_steps(sec_in, sanala, max(args.steps, 200), args.warmup)  # host-bound calls: average over more
        secondary = {"workload": WORKLOADS["config2"]["desc"], "warm": point(sec_in, sms)}
        secondary["warm"]["note"] = ("back-to-back calls: the 18 MB working set stays in the 256 MB Infinity Cache, "
                                     "so this is not an HBM figure")
        log(f"[bench] config2: {sms * 1e3:.1f} us/step warm")
        ssts = time_steady(sec_in, sanala, 500)
        secondary["steady"] = point(sec_in, ssts)
        secondary["steady"]["note"] = "back-to-back calls after 0.2 s of calls (settled clocks)"
        secondary["steady"]["per_call_us"] = spread(time_rounds(sec_in, sanala))
        log(f"[bench] config2: {ssts * 1e3:.1f} us/step steady state")
        if flush is not None:
            scms, scold_us = time_cold(sec_in, sanala, max(args.steps, 50), args.warmup, flush)
            secondary["cold"] = point(sec_in, scms)
            secondary["cold"]["note"] = "1 GiB read-only pass before every call, outside the events: inputs from HBM"
            secondary["cold"]["per_call_us"] = spread(scold_us)
            log(f"[bench] config2: {scms * 1e3:.1f} us/step cold")
        try:
            gms = time_graph(sec_in, sanala)
            secondary["graph"] = point(sec_in, gms)
            secondary["graph"]["note"] = ("the allocation-free call captured 20 times in one HIP graph and replayed: "
                                          "the same kernels with no host work between calls")
            log(f"[bench] config2: {gms * 1e3:.1f} us/step from a HIP graph")
        except Exception as e:  # noqa: BLE001 - a secondary figure must not cost the headline line
            secondary["graph"] = {"error": f"{type(e).__name__}: {e}"}
            log(f"[bench] config2 graph replay failed: {e}")
        secondary["kernels_us"] = {k: round(v * 1e3, 2) for k, v in kernel_times(sec_in, sanala).items()}
        del sec_in
    cross = None
    if not args.no_secondary and args.workload == "config4":
        # The block's cross-attention over the same 4K latent (300 text tokens), warm, with its kernels.
        x_in = Inputs("cross4k")
        xms = time_steps(x_in, sanala, max(args.steps, 200), args.warmup)
        xsts = time_steady(x_in, sanala, 200)
        xkt = kernel_times(x_in, sanala)
        exps = float(x_in.N * int(x_in.kv_len.sum().item()) * x_in.H)
        cms = xkt.get("cross_attn", float("nan"))
        cross = {"workload": WORKLOADS["cross4k"]["desc"], "ms_per_step": round(xms, 5),
                 "tokens_per_s": round(x_in.B * x_in.N / (xms * 1e-3), 1),
                 "steady_ms_per_step": round(xsts, 5), "steady_tokens_per_s": round(x_in.B * x_in.N / (xsts * 1e-3), 1),
                 "kernels_us": {k: round(v * 1e3, 2) for k, v in xkt.items()},
                 "roofline": {"bound": "alu", "kernel": "cross_attn", "unit": "T exp2/s",
                              "achieved": round(exps / (cms * 1e-3) / 1e12, 2), "peak": round(EXP2_PEAK_T, 2),
                              "frac": round(exps / (cms * 1e-3) / 1e12 / EXP2_PEAK_T, 4)}}
        log(f"[bench] cross4k: {xms * 1e3:.1f} us/step warm, {xsts * 1e3:.1f} us/step steady state; kernels " +
            ", ".join(f"{k}={v * 1e3:.1f}us" for k, v in xkt.items()))
        del x_in
    ceiling = None
    if not args.no_cold:
        del flush
        ceiling = copy_ceiling()
        log(f"[bench] copy ceiling: {ceiling}")

    cpu = None if args.no_cpu_baseline else cpu_baseline(main_in)
    if cpu:
        log(f"[bench] cpu baseline: {cpu['value']:.4g} tokens/s on {cpu['cores']} threads")

    line = {
        "metric": "linear-attn tokens/s + achieved HBM GB/s (% of peak) at N=1024 and N=16384",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 projection, bf16 attention" if main_in.kind == "w8a8" else "bf16",
        "data": "synthetic (seeded N(0,1) inputs of SANA shapes; no trained weights)",
        "config": {"workload": WORKLOADS[args.workload]["desc"], "B": main_in.B, "N": main_in.N, "H": main_in.H,
                   "D": main_in.D, "C": main_in.C, "parallelism": "single GPU"},
        "achieved_GBps": round(call_gbps, 1),
        "frac_of_hbm_peak": round(call_gbps / HBM_PEAK_GBPS, 4),
        "timing": ("value: back-to-back calls (warm) after the warm-up steps; steady_state: the same after 0.2 s of "
                   "calls; cold: caches flushed before each call"),
        "steady_state": steady,
        "cold": cold,
        "copy_ceiling": ceiling,
        "kernels_us": {k: round(v * 1e3, 2) for k, v in kt.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "cross_attention": cross,
        "source_hash": source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Throughput of libsanala's ReLU linear attention with QK-RMSNorm on one MI355X.

Prints ONE JSON line: tokens/s of the whole call on the 4K workload (B=1, N=16384 tokens, 70 heads x 32,
bf16 I/O, K with 1% outlier rows), achieved HBM GB/s against the 8 TB/s peak, the dominant kernel's
roofline, the 1024px workload (B=1, N=1024) as a secondary figure, and the fp64 oracle timed on the
host cores as a CPU baseline.

A step is one sana_linear_attn_fwd call over the resident inputs (row statistics, KV state, chunk
reduction and output: the whole path).

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload config4|config2|config3|config5|w8a8|mixffn]
  python bench.py --mode copy        # plain device copy of known size (counter calibration under rocprofv3)
  python bench.py --summarize-traffic KERNEL_FETCH.db KERNEL_WRITE.db COPY_FETCH.db COPY_WRITE.db
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
    "config4": dict(cfg=4, desc="4K linear attention: B=1, N=16384 (128x128 latent), H=70, D=32, bf16 I/O, "
                                "K ~ N(0,30^2) with 1% rows x100, QK-RMSNorm on"),
    "config2": dict(cfg=2, desc="1024px linear attention: B=1, N=1024 (32x32 latent), H=70, D=32, bf16 I/O, QK-RMSNorm on"),
    "config3": dict(cfg=3, desc="1024px repeat-sampling batch: B=32, N=1024, H=70, D=32, bf16 I/O, QK-RMSNorm on"),
    "config5": dict(cfg=5, desc="2K fused front end: x[4,4096,2240] bf16 @ Wqkv[2240,6720] -> linear attention H=70, D=32"),
    "w8a8": dict(cfg=5, desc="2K front end in W8A8: x[4,4096,2240] bf16 quantised per token, int8 Wt[6720,2240] "
                             "with column scales -> linear attention H=70, D=32 on bf16 qkv"),
    "mixffn": dict(cfg=5, desc="2K Mix-FFN: x[4, 64x64, 2240] bf16 @ W1[2240,11200] -> 3x3 depthwise conv (zero pad) "
                               "-> GLU -> @ W2[5600,2240]"),
}


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
        else:
            inp = gen_config(self.spec["cfg"])
            self.kind = "qkv" if self.spec["cfg"] == 5 else "attn"
        self.host = inp
        bf = torch.bfloat16
        g = lambda a: torch.from_numpy(a).to("cuda")  # noqa: E731
        if self.kind == "attn":
            self.q, self.k, self.v = (torch.from_numpy(a).to("cuda").to(bf) for a in (inp.q, inp.k, inp.v))
            self.out = torch.empty_like(self.q)
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
        else:
            sanala.sana_qkv_w8a8_linear_attn_fwd(self.x, self.wt, self.sw, self.gq, self.gk, self.B, self.N, self.H,
                                                 self.D, self.host.eps, self.out)

    def algorithmic_bytes(self) -> int:
        """Read Q, K, V and write O once: 4 * B * N * C * 2 bytes (bf16)."""
        return 4 * self.B * self.N * self.C * 2

    def kernel_bytes(self, kernel: str) -> float:
        tok = self.B * self.N * self.C * 2
        if kernel in ("kv_state", "kv_partial"):
            return 2 * tok            # read K and V
        if kernel == "out":
            return 2 * tok            # read Q, write O
        if kernel in ("rowstats_k", "rowstats_q"):
            return tok                # read one tensor
        if kernel == "fused":
            return 4 * tok
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


def kernel_times(inputs: Inputs, sanala, reps: int = 20):
    """Average per-kernel duration from the start/stop events of each kernel's own dispatch (library timing)."""
    sanala.sana_timing_enable(True)
    acc = {}
    try:
        for _ in range(reps):
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
        else:
            oracle.qkv_w8a8_linear_attn(h.x, h.wt_q, h.s_w, h.gq, h.gk, h.H, h.D, h.eps)
        reps += 1
        el = time.time() - t0
        if el >= min_seconds or reps >= max_reps:
            break
    tokens = h.B * h.N * reps
    return {"value": tokens / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} full passes of the {inputs.name} workload ({h.B}x{h.N} tokens each) "
                      f"through the fp64 NumPy oracle in {el:.1f}s"}


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


def summarize_traffic(kfetch: str, kwrite: str, cfetch: str, cwrite: str, workload: str = "config4") -> str:
    """Per-dispatch HBM bytes of each libsanala kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    scaled by what the same counters read for a plain device copy of 268,435,456 bytes."""
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
             "#   rocprofv3 --pmc FETCH_SIZE -d kfetch -o run -- python3 /root/repo/bench.py --steps 3 --warmup 1 "
             "--no-cpu-baseline --no-secondary",
             "#   rocprofv3 --pmc WRITE_SIZE -d kwrite -o run -- (same bench command)",
             "#   rocprofv3 --pmc FETCH_SIZE -d cfetch -o run -- python3 /root/repo/bench.py --mode copy",
             "#   rocprofv3 --pmc WRITE_SIZE -d cwrite -o run -- python3 /root/repo/bench.py --mode copy",
             "#   python3 bench.py --summarize-traffic kfetch/run_results.db kwrite/run_results.db "
             "cfetch/run_results.db cwrite/run_results.db",
             f"workload: {workload}", f"source_hash: {source_hash()}",
             f"fetch_calibration: {f_scale:.4f}", f"write_calibration: {w_scale:.4f}"]
    short = {"rowstats": "rowstats_k", "kv_state": "kv_state", "kv_reduce": "kv_reduce", "out_persist": "out",
             "out_bf16": "out", "qkv_gemm": "qkv_gemm"}
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


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-traffic":
        text = summarize_traffic(*sys.argv[2:6])
        with open(os.path.join(ROOT, "profiles", "hbm_traffic.txt"), "w") as f:
            f.write(text)
        print(text)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="config4", choices=sorted(WORKLOADS))
    ap.add_argument("--mode", default="bench", choices=["bench", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
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
        sms = time_steps(sec_in, sanala, max(args.steps, 50), args.warmup)
        sb = sec_in.algorithmic_bytes()
        secondary = {"workload": WORKLOADS["config2"]["desc"], "tokens_per_s": round(sec_in.B * sec_in.N / (sms * 1e-3)),
                     "ms_per_step": round(sms, 5), "achieved_GBps": round(sb / (sms * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(sb / (sms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "note": "18 MB working set: stays in the 256 MB Infinity Cache across back-to-back steps"}
        log(f"[bench] config2: {sms * 1e3:.1f} us/step")
        del sec_in

    cpu = None if args.no_cpu_baseline else cpu_baseline(main_in)
    if cpu:
        log(f"[bench] cpu baseline: {cpu['value']:.4g} tokens/s on {cpu['cores']} threads")

    line = {
        "metric": "linear-attn tokens/s (+ achieved HBM GB/s, % of peak) at N=16384; N=1024 in 'secondary'",
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
        "kernels_us": {k: round(v * 1e3, 2) for k, v in kt.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "source_hash": source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Shared helpers of the GPU parity tests: upload seeded inputs, run the HIP path, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

# Gates on max |O_gpu - O_oracle| relative to max |V| for each storage type.
GATE = {"f32": 1e-5, "bf16": 2e-2, "f16": 2e-2}
# Scale-aware bounds relative to max |O_oracle|, derived from the arithmetic: fp32 I/O keeps every step
# in fp32 (error a few ulp of the fp32 sums); bf16 I/O rounds phi(Q) to bf16 as an MFMA operand and the
# output to bf16, 2^-9 relative each, so a few parts in 1e3 of the output scale.  binary16 I/O keeps
# the same bf16 operands in the output contraction (its state values can exceed the binary16 range) and
# rounds the output to binary16 (2^-11), so it takes the bf16 bounds.
SCALE_BOUND = {"f32": 1e-5, "bf16": 1e-2, "f16": 1e-2}


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(TORCH_DT[dtype]).contiguous()


def gains_dev(g):
    return None if g is None else torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).to("cuda")


def run_attn(sanala, inp, out=None):
    q, k, v = dev(inp.q, inp.dtype), dev(inp.k, inp.dtype), dev(inp.v, inp.dtype)
    o = sanala.linear_attn(q, k, v, gains_dev(inp.gq), gains_dev(inp.gk), inp.H, inp.D, inp.eps, out=out)
    torch.cuda.synchronize()
    return o


def metrics(o_gpu: np.ndarray, o_ref: np.ndarray, v_ref: np.ndarray) -> dict:
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    return dict(max_err=float(err.max()), rms_err=float(np.sqrt(np.mean(err * err))),
                max_v=float(np.abs(v_ref).max()), max_o=float(np.abs(o_ref).max()),
                nan=int(np.isnan(o_gpu).sum()))


def check(o_gpu: torch.Tensor, o_ref: np.ndarray, v_ref: np.ndarray, dtype: str, label: str = "") -> dict:
    og = o_gpu.float().cpu().numpy()
    m = metrics(og, o_ref, v_ref)
    print(f"[parity] {label} dtype={dtype} max_err={m['max_err']:.3e} rms={m['rms_err']:.3e} "
          f"max|V|={m['max_v']:.3f} max|O|={m['max_o']:.3e} err/max|O|={m['max_err'] / max(m['max_o'], 1e-30):.3e}",
          flush=True)
    assert m["nan"] == 0, f"{label}: {m['nan']} NaN outputs"
    assert m["max_err"] <= GATE[dtype] * m["max_v"], f"{label}: gate failed {m}"
    assert m["max_err"] <= SCALE_BOUND[dtype] * m["max_o"], f"{label}: scale-aware bound failed {m}"
    return m


def oracle_out(inp):
    return oracle.linear_attn(inp.q, inp.k, inp.v, inp.gq, inp.gk, inp.H, inp.D, inp.eps)

"""GPU parity on the edges of the output kernels and of the eps reading (the Sana notes, section 2.1,
Eq. (1), with one eps inside the QK-Norm square root and one after the denominator's dot product).

* The persistent output kernel (one block per CU, all heads' operands in LDS) at head counts other than
  70: a single head, an odd count (the last wave clamps its second head and masks its stores) and
  72 heads (the most whose operands fit: 162,816 of 163,840 bytes of LDS).  B = 1, N = 8200 gives 513
  tiles, enough for that kernel to be chosen.  The output buffer is NaN-poisoned, so every element
  must be written.
* A large eps (0.5) with small queries and keys, so that eps dominates both mean squares and the
  denominator: the output kernels' eps / r_q = eps * sqrt(ms + eps) rewrite and the state's r_k are
  then far from their small-eps values.
* eps = 0 with an all-zero phi(q) row: 0/0, NaN on both sides, at the same positions.
* The widest head count the library takes (H = 320) on the fp32 path (80 head groups of 4 in its output
  kernel's grid) and on the 16-bit path.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from synth import gen_attn
from synth.gen import bf16_round
from tests.parity_util import GATE, SCALE_BOUND, check, dev, gains_dev, oracle_out

pytestmark = pytest.mark.gpu


def _with_env(name, value, fn):
    old = os.environ.get(name)
    os.environ[name] = value
    try:
        return fn()
    finally:
        if old is None:
            del os.environ[name]
        else:
            os.environ[name] = old


def _run_poisoned(sanala, inp):
    q, k, v = dev(inp.q, inp.dtype), dev(inp.k, inp.dtype), dev(inp.v, inp.dtype)
    tdt = q.dtype
    out = torch.full(q.shape, float("nan"), device="cuda", dtype=tdt)
    o = sanala.linear_attn(q, k, v, gains_dev(inp.gq), gains_dev(inp.gk), inp.H, inp.D, inp.eps, out=out)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("H", [1, 3, 71, 72])
def test_persistent_output_kernel_head_counts(gpu_lib, H, dtype):
    inp = gen_attn(5000 + H, 1, 8200, H=H, dtype=dtype)
    print(f"[edge] persistent H={H} {dtype}", flush=True)
    o = _run_poisoned(gpu_lib, inp)
    assert not torch.isnan(o).any(), "an output element was not written"
    check(o, oracle_out(inp), inp.v, dtype, f"persistent H={H}")


def _small_queries(inp, scale):
    inp.q[:] = inp.q * np.float32(scale)
    if inp.dtype == "bf16":
        inp.q[:] = bf16_round(inp.q)
    elif inp.dtype == "f16":
        inp.q[:] = inp.q.astype(np.float16).astype(np.float32)
    return inp


@pytest.mark.parametrize("dtype,B,N,kind", [("bf16", 1, 8200, "1"), ("bf16", 2, 1000, "1"), ("bf16", 2, 1000, "2"),
                                            ("f16", 1, 8200, "1"), ("f32", 2, 300, "1")])
def test_large_eps(gpu_lib, dtype, B, N, kind):
    # queries at 1e-3 and keys at 0.03 of unit scale: eps = 0.5 dominates both mean squares, and the
    # denominator phi(q).z is then comparable to eps
    inp = _small_queries(gen_attn(5100 + N, B, N, dtype=dtype, eps=0.5, k_scale=0.03), 1e-3)
    print(f"[edge] eps=0.5 {dtype} B={B} N={N} out kernel {kind}", flush=True)
    o = _with_env("SANA_OUT_KERNEL", kind, lambda: _run_poisoned(gpu_lib, inp))
    ref = oracle_out(inp)
    # the eps terms are not negligible here: the same inputs with eps = 1e-6 give a far-away output
    tiny = oracle.linear_attn(inp.q, inp.k, inp.v, inp.gq, inp.gk, inp.H, inp.D, 1e-6)
    assert np.abs(ref - tiny).max() > 10 * SCALE_BOUND[dtype] * np.abs(ref).max()
    check(o, ref, inp.v, dtype, f"eps=0.5 {dtype} N={N} kind={kind}")


@pytest.mark.parametrize("dtype,B,N,kind", [("bf16", 1, 8200, "1"), ("bf16", 2, 700, "1"), ("bf16", 2, 700, "2"),
                                            ("f32", 1, 200, "1")])
def test_eps_zero_with_zero_phi_rows_gives_nan_where_the_oracle_does(gpu_lib, dtype, B, N, kind):
    inp = gen_attn(5200 + N, B, N, dtype=dtype, eps=0.0)
    assert (inp.gq > 0).all()
    rows = [(0, 0), (0, N // 2), (B - 1, N - 1)]
    for b, n in rows:
        inp.q[b, n] = -np.abs(inp.q[b, n])            # phi(q) = 0 for the whole row: 0 / 0
    print(f"[edge] eps=0 {dtype} B={B} N={N} out kernel {kind}", flush=True)
    o = _with_env("SANA_OUT_KERNEL", kind, lambda: _run_poisoned(gpu_lib, inp)).float().cpu().numpy()
    ref = oracle_out(inp)
    nan_ref, nan_gpu = np.isnan(ref), np.isnan(o)
    assert nan_ref.any()
    assert np.array_equal(nan_ref, nan_gpu), "NaN positions differ from the oracle's"
    for b, n in rows:
        assert nan_gpu[b, n].all()
    ok = ~nan_ref
    err = np.abs(o[ok].astype(np.float64) - ref[ok])
    assert err.max() <= GATE[dtype] * np.abs(inp.v).max()
    assert err.max() <= SCALE_BOUND[dtype] * np.abs(ref[ok]).max()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_widest_head_count(gpu_lib, dtype):
    inp = gen_attn(5300, 2, 37, H=320, dtype=dtype)
    print(f"[edge] H=320 {dtype}", flush=True)
    o = _run_poisoned(gpu_lib, inp)
    assert not torch.isnan(o).any()
    check(o, oracle_out(inp), inp.v, dtype, f"H=320 {dtype}")

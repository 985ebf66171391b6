"""GPU parity: the HIP path through the C-ABI against the fp64 oracle on the same seeded inputs.

Gates: max |O_gpu - O_oracle| <= 1e-5 max|V| (fp32 I/O) and <= 2e-2 max|V| (bf16 and binary16 I/O), plus the
scale-aware bound relative to max |O_oracle| in parity_util.SCALE_BOUND.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from synth import gen_attn, gen_config, gen_qkv
from tests.parity_util import check, dev, gains_dev, oracle_out, run_attn

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("B,N", [(1, 1), (2, 17), (1, 64), (3, 100), (1, 333), (2, 1037)])
def test_small_shapes_span_tiles_and_tails(gpu_lib, dtype, B, N):
    inp = gen_attn(1000 + N, B, N, dtype=dtype)
    o = run_attn(gpu_lib, inp)
    check(o, oracle_out(inp), inp.v, dtype, f"B={B} N={N}")


@pytest.mark.parametrize("H", [1, 3, 70, 71, 80])
def test_head_counts(gpu_lib, H):
    """Odd head counts (a half-filled head pair) and H above one output block's register budget."""
    for dtype in ("f32", "bf16"):
        inp = gen_attn(2000 + H, 2, 150, H=H, dtype=dtype)
        check(run_attn(gpu_lib, inp), oracle_out(inp), inp.v, dtype, f"H={H}")


@pytest.mark.parametrize("N,chunk", [(5000, None), (3000, "1024")], ids=["planner", "chunk1024"])
def test_fp32_state_over_long_chunks(gpu_lib, N, chunk):
    """The fp32 state kernel keeps four 64-token sub-blocks' loads in flight in a ring of register sets;
    chunks of more than four sub-blocks reuse its slots (5000 tokens: the planner's chunks of 384, six
    sub-blocks; SANA_KV_CHUNK=1024: sixteen)."""
    import os
    inp = gen_attn(2100 + N, 1, N, dtype="f32")
    old = os.environ.get("SANA_KV_CHUNK")
    if chunk is not None:
        os.environ["SANA_KV_CHUNK"] = chunk
    try:
        o = run_attn(gpu_lib, inp)
    finally:
        if chunk is not None:
            if old is None:
                del os.environ["SANA_KV_CHUNK"]
            else:
                os.environ["SANA_KV_CHUNK"] = old
    check(o, oracle_out(inp), inp.v, "f32", f"fp32 N={N} chunk={chunk}")


def test_config1_fp32_full(gpu_lib):
    inp = gen_config(1)
    check(run_attn(gpu_lib, inp), oracle_out(inp), inp.v, "f32", "config1")


def test_config2_bf16_full(gpu_lib):
    inp = gen_config(2)
    check(run_attn(gpu_lib, inp), oracle_out(inp), inp.v, "bf16", "config2")


def test_config3_bf16_full(gpu_lib):
    inp = gen_config(3)
    check(run_attn(gpu_lib, inp), oracle_out(inp), inp.v, "bf16", "config3")


def test_config4_bf16_full(gpu_lib):
    inp = gen_config(4)
    o = run_attn(gpu_lib, inp)
    check(o, oracle_out(inp), inp.v, "bf16", "config4")


def test_config5_qkv_full(gpu_lib):
    inp = gen_qkv(5, 4, 4096)
    o_ref, parts = oracle.qkv_linear_attn(inp.x, inp.w, inp.gq, inp.gk, inp.H, inp.D, inp.eps, return_parts=True)
    x, w = dev(inp.x, "bf16"), dev(inp.w, "bf16")
    o = gpu_lib.qkv_linear_attn(x, w, gains_dev(inp.gq), gains_dev(inp.gk), inp.H, inp.D, inp.eps)
    torch.cuda.synchronize()
    check(o, o_ref, parts["v"], "bf16", "config5")


def test_qkv_small_ragged(gpu_lib):
    """GEMM tiles with ragged M and an odd head count (3C not a multiple of the 192-column tile)."""
    for B, N, H in [(1, 37, 70), (2, 300, 3), (1, 129, 5)]:
        inp = gen_qkv(77 + N, B, N, H=H)
        o_ref, parts = oracle.qkv_linear_attn(inp.x, inp.w, inp.gq, inp.gk, H, 32, inp.eps, return_parts=True)
        o = gpu_lib.qkv_linear_attn(dev(inp.x, "bf16"), dev(inp.w, "bf16"), gains_dev(inp.gq), gains_dev(inp.gk), H)
        torch.cuda.synchronize()
        check(o, o_ref, parts["v"], "bf16", f"qkv B={B} N={N} H={H}")


def test_structured_v(gpu_lib):
    """V = N(0,1) + 3 makes every output O(1), so the bound relative to max|O| is a tight one."""
    for dtype in ("f32", "bf16"):
        inp = gen_attn(31, 1, 1024, dtype=dtype, v_shift=3.0)
        check(run_attn(gpu_lib, inp), oracle_out(inp), inp.v, dtype, "structured V")


def test_norm_off(gpu_lib):
    """QK-Norm off (both gains NULL): phi = ReLU, the SANA-1.0 form of Eq. (1)."""
    for dtype in ("f32", "bf16", "f16"):
        inp = gen_attn(32, 2, 500, dtype=dtype, norm=False)
        check(run_attn(gpu_lib, inp), oracle_out(inp), inp.v, dtype, "norm off")


def test_outlier_keys_norm_off_fp32_state(gpu_lib):
    """Config-4 style K (sd 30, 1% rows x100) without QK-Norm: z reaches ~1e5-1e6, beyond fp16."""
    inp = gen_attn(4, 1, 4096, dtype="bf16", k_scale=30.0, outlier_frac=0.01, norm=False)
    o_ref, parts = oracle.linear_attn(inp.q, inp.k, inp.v, None, None, inp.H, inp.D, inp.eps, return_parts=True)
    assert parts["z"].max() > 65504.0
    check(run_attn(gpu_lib, inp), o_ref, inp.v, "bf16", "outlier K, norm off")


def test_outlier_keys_norm_off_f16_io(gpu_lib):
    """The same keys stored as IEEE binary16 (largest finite value 65504): z exceeds the binary16 range,
    yet the state stays in fp32 and the output is finite and within the gates."""
    inp = gen_attn(4, 1, 4096, dtype="f16", k_scale=30.0, outlier_frac=0.01, norm=False)
    o_ref, parts = oracle.linear_attn(inp.q, inp.k, inp.v, None, None, inp.H, inp.D, inp.eps, return_parts=True)
    assert parts["z"].max() > 65504.0
    o = run_attn(gpu_lib, inp)
    assert o.dtype == torch.float16 and torch.isfinite(o).all()
    check(o, o_ref, inp.v, "f16", "outlier K, norm off, f16")


@pytest.mark.parametrize("kind", ["1", "2"])
def test_f16_io_output_kernels(gpu_lib, kind):
    """binary16 I/O with the QK-Norm on, through both output kernels, several tiles and a ragged tail,
    NaN-poisoned output buffer, two calls bit-identical."""
    inp = gen_attn(43, 2, 2100, dtype="f16")
    q, k, v = dev(inp.q, "f16"), dev(inp.k, "f16"), dev(inp.v, "f16")
    gq, gk = gains_dev(inp.gq), gains_dev(inp.gk)

    def run():
        out = torch.full(q.shape, float("nan"), device="cuda", dtype=torch.float16)
        o = gpu_lib.linear_attn(q, k, v, gq, gk, inp.H, inp.D, inp.eps, out=out)
        torch.cuda.synchronize()
        return o

    o1 = _with_env("SANA_OUT_KERNEL", kind, run)
    o2 = _with_env("SANA_OUT_KERNEL", kind, run)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    check(o1, oracle_out(inp), inp.v, "f16", f"f16 out kernel {kind}")


def test_f16_head_counts_and_chunked_state(gpu_lib):
    """Odd and large head counts, and a token count split over several state chunks (the reduce)."""
    for H, N in ((3, 150), (71, 150), (80, 150), (70, 16384)):
        inp = gen_attn(3000 + H, 1, N, H=H, dtype="f16")
        check(run_attn(gpu_lib, inp), oracle_out(inp), inp.v, "f16", f"f16 H={H} N={N}")


def test_deterministic_bitwise(gpu_lib):
    inp = gen_config(2)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    gq, gk = gains_dev(inp.gq), gains_dev(inp.gk)
    o1 = gpu_lib.linear_attn(q, k, v, gq, gk, 70)
    o2 = gpu_lib.linear_attn(q, k, v, gq, gk, 70)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_nan_poisoned_output_fully_written(gpu_lib):
    for dtype in ("f32", "bf16"):
        inp = gen_attn(33, 2, 777, dtype=dtype)
        out = torch.full(inp.q.shape, float("nan"), device="cuda", dtype=torch.float32 if dtype == "f32" else torch.bfloat16)
        o = run_attn(gpu_lib, inp, out=out)
        assert not torch.isnan(o).any()
        check(o, oracle_out(inp), inp.v, dtype, "poisoned out")


def test_zero_phi_rows_give_exact_zero(gpu_lib):
    for dtype in ("f32", "bf16"):
        inp = gen_attn(34, 1, 200, dtype=dtype)
        inp.q[0, 5] = -np.abs(inp.q[0, 5])          # all of phi(q) for token 5 is zero
        o = run_attn(gpu_lib, inp)
        assert torch.count_nonzero(o[0, 5]).item() == 0
        inp.k[:] = -np.abs(inp.k)                   # all phi(k) zero: S = 0, z = 0, O = 0 through eps
        o2 = run_attn(gpu_lib, inp)
        assert torch.count_nonzero(o2).item() == 0


def test_batch_samples_independent(gpu_lib):
    inp = gen_attn(35, 3, 300, dtype="bf16")
    o = run_attn(gpu_lib, inp)
    inp.v[1] *= -2.0
    o2 = run_attn(gpu_lib, inp)
    assert torch.equal(o[0].view(torch.int16), o2[0].view(torch.int16))
    assert torch.equal(o[2].view(torch.int16), o2[2].view(torch.int16))
    assert not torch.equal(o[1].view(torch.int16), o2[1].view(torch.int16))


def test_rejects_bad_arguments_without_enqueueing(gpu_lib):
    inp = gen_attn(36, 1, 8, dtype="bf16")
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    gq, gk = gains_dev(inp.gq), gains_dev(inp.gk)
    out = torch.empty_like(q)
    with pytest.raises(gpu_lib.SanaError) as e:
        gpu_lib.sana_linear_attn_fwd(q, k, v, gq, None, 1, 8, 70, 32, 1e-6, out)
    assert e.value.status == 1
    with pytest.raises(gpu_lib.SanaError) as e:
        gpu_lib.sana_linear_attn_fwd(q, k, v, gq, gk, 1, 8, 140, 16, 1e-6, out)
    assert e.value.status == 2
    with pytest.raises(gpu_lib.SanaError) as e:
        gpu_lib.sana_linear_attn_fwd(q, k, v, gq, gk, 1, 8, 70, 32, 1e-6, q)  # out aliases q
    assert e.value.status == 1


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


def _mixed_scale_rows(seed, B, N, H, rows):
    """bf16 inputs where some query rows carry tiny values (1e-12) on the first ten heads only: for those
    heads the eps / r_q term dominates the denominator, and r_q comes from the other heads' channels."""
    inp = gen_attn(seed, B, N, H=H, dtype="bf16")
    for b, n in rows:
        inp.q[b, n, : 10 * 32] *= np.float32(1e-12)
    from synth.gen import bf16_round
    inp.q[:] = bf16_round(inp.q)
    return inp


def _rowwise_check(o, o_ref, rows, H, label):
    """Relative check per (row, head) block: the gates relative to max|V| would not see these rows."""
    og = o.float().cpu().numpy()
    for b, n in rows:
        for h in range(H):
            ref = o_ref[b, n, 32 * h: 32 * h + 32]
            got = og[b, n, 32 * h: 32 * h + 32]
            scale = np.abs(ref).max()
            err = np.abs(got - ref).max()
            assert err <= 1e-2 * scale + 1e-30, f"{label}: row {b},{n} head {h}: err {err:.3e} vs scale {scale:.3e}"


@pytest.mark.parametrize("kind", ["1", "2", "3"])
@pytest.mark.parametrize("N", [2100, 8200])
def test_output_kernels_agree_with_oracle(gpu_lib, kind, N):
    """The output kernels on the same inputs: the default choice (1: persistent at 8200 tokens x 2, head
    groups at 2100 x 2), the tile kernel over all heads (2) and the head-group kernel with r_q from the
    row-statistics launch (3)."""
    inp = gen_attn(41, 2, N, dtype="bf16")
    o = _with_env("SANA_OUT_KERNEL", kind, lambda: run_attn(gpu_lib, inp))
    check(o, oracle_out(inp), inp.v, "bf16", f"out kernel {kind} N={N}")


def test_many_heads_tile_kernel_with_row_statistics_of_q(gpu_lib):
    """H = 80 with many tiles: the operands exceed the LDS, so the tile kernel runs over head groups of
    72 with r_q from a row-statistics pass over Q."""
    inp = gen_attn(46, 1, 8200, H=80, dtype="bf16")
    check(run_attn(gpu_lib, inp), oracle_out(inp), inp.v, "bf16", "H=80 N=8200")


@pytest.mark.parametrize("B,N,norm", [(1, 12345, True), (2, 8200, True), (1, 9000, False), (8, 1024, True),
                                      (9, 1000, False)])
def test_persistent_schedules_agree(gpu_lib, B, N, norm):
    """Persistent output kernel with its default schedule (strided tiles for the long samples; for
    8 x 1024 and 9 x 1000 the blocks of a sample taking its tiles interleaved) and with contiguous runs:
    every tile written (NaN-poisoned output), both bit-identical, within the gates.  Covers a ragged
    last tile, a sample change inside the strided sweep and the norm-off variant."""
    inp = gen_attn(47 + N, B, N, dtype="bf16", norm=norm)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    gq, gk = gains_dev(inp.gq), gains_dev(inp.gk)

    def run():
        out = torch.full(q.shape, float("nan"), device="cuda", dtype=torch.bfloat16)
        o = gpu_lib.linear_attn(q, k, v, gq, gk, inp.H, inp.D, inp.eps, out=out)
        torch.cuda.synchronize()
        return o

    o_strided = _with_env("SANA_OUT_SCHED", "2", run)
    o_runs = _with_env("SANA_OUT_SCHED", "1", run)
    assert not torch.isnan(o_strided).any() and not torch.isnan(o_runs).any()
    assert torch.equal(o_strided.view(torch.int16), o_runs.view(torch.int16))
    check(o_strided, oracle_out(inp), inp.v, "bf16", f"schedules B={B} N={N} norm={norm}")


@pytest.mark.parametrize("kind", ["1", "2", "3"])
def test_mixed_scale_query_rows(gpu_lib, kind):
    rows = [(0, 3), (0, 64), (1, 100), (1, 4000)]
    inp = _mixed_scale_rows(42, 2, 4100, 70, rows)
    o_ref = oracle_out(inp)
    o = _with_env("SANA_OUT_KERNEL", kind, lambda: run_attn(gpu_lib, inp))
    check(o, o_ref, inp.v, "bf16", "mixed-scale rows")
    _rowwise_check(o, o_ref, rows, 70, "mixed-scale rows")


def _sampled_rows_check(o, inp, label, rows_per_sample=96, seed=0):
    """Oracle on sampled output rows (the first and last token always included): the state from all
    tokens, the output for the sampled rows only."""
    rng = np.random.default_rng(seed)
    N = inp.N
    phik = oracle.feature_map(inp.k, inp.gk, inp.eps)
    S, z = oracle.kv_state(phik, inp.v, inp.H, inp.D)
    idx = np.unique(np.concatenate([rng.choice(N, size=min(rows_per_sample, N), replace=False), [0, N - 1]]))
    phiq = oracle.feature_map(inp.q[:, idx], inp.gq, inp.eps)
    o_ref = oracle.attend(phiq, S, z, inp.eps, inp.H, inp.D)
    check(o[:, torch.from_numpy(idx).to(o.device)], o_ref, inp.v, inp.dtype, label)


@pytest.mark.parametrize("B,N", [(1, 65536), (3, 20011)])
def test_long_sequences_sampled_rows(gpu_lib, B, N):
    """Four times the 4K token count (several hundred MB per tensor: 64-bit offsets, many chunks per
    sample) and a ragged batch whose output tiles cross sample boundaries."""
    inp = gen_attn(45 + N, B, N, dtype="bf16")
    o = run_attn(gpu_lib, inp)
    assert not torch.isnan(o).any()
    _sampled_rows_check(o, inp, f"B={B} N={N}")


def test_scratch_reuse_across_streams_and_growth(gpu_lib):
    """The scratch buffer is kept per stream and grows on demand: interleaved calls on two streams with
    different sizes, then a larger call on the first stream, each against its own single-stream result."""
    small = gen_attn(48, 1, 300, dtype="bf16")
    large = gen_attn(49, 2, 5000, dtype="bf16")
    ref_small, ref_large = run_attn(gpu_lib, small), run_attn(gpu_lib, large)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ins = {}
    for name, inp in (("small", small), ("large", large)):
        ins[name] = (dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16"), gains_dev(inp.gq), gains_dev(inp.gk))
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        for name, stream in (("small", s1), ("large", s2), ("large", s1), ("small", s2)):
            q, k, v, gq, gk = ins[name]
            with torch.cuda.stream(stream):
                out = torch.empty_like(q)
                gpu_lib.sana_linear_attn_fwd(q, k, v, gq, gk, q.shape[0], q.shape[1], 70, 32, 1e-6, out,
                                             stream=stream)
            outs.append((name, out))
    torch.cuda.synchronize()
    for name, out in outs:
        ref = ref_small if name == "small" else ref_large
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), name


def test_chunk_reduction_across_consecutive_calls(gpu_lib):
    """A sample's state split over many chunks (partials in the per-stream scratch, then the reduction):
    consecutive calls on one stream with different inputs each match the oracle (nothing of the previous
    call's state survives), and repeating the first input repeats its output bit for bit."""
    def run():
        outs = []
        for inp in (a, b, a):
            outs.append(run_attn(gpu_lib, inp))
        return outs

    for dtype in ("bf16", "f16"):
        a = gen_attn(51, 2, 3000, dtype=dtype)
        b = gen_attn(52, 2, 3000, dtype=dtype)
        o_a, o_b, o_a2 = _with_env("SANA_KV_CHUNK", "256", run)
        check(o_a, oracle_out(a), a.v, dtype, f"{dtype} first call")
        check(o_b, oracle_out(b), b.v, dtype, f"{dtype} second call")
        assert torch.equal(o_a.view(torch.int16), o_a2.view(torch.int16))

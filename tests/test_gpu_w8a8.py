"""GPU parity of the W8A8 front end and of the device quantiser against the oracle.

W8A8 deployment: "Sana: Efficient High-Resolution Image Synthesis with Linear Diffusion
Transformers" (paper notes), section 7 "on-device deployment".  The quantiser's integer codes and
fp32 scales are compared bit for bit (both sides decide them in fp32); the attention output, formed
from the bf16-rounded qkv of the int8 projection, takes the bf16 gates.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import bf16_round, gen_w8a8
from tests.parity_util import check, dev, gains_dev

pytestmark = pytest.mark.gpu


def _run(gpu_lib, inp):
    x = dev(inp.x, "bf16")
    wt = torch.from_numpy(np.ascontiguousarray(inp.wt_q)).to("cuda")
    sw = torch.from_numpy(np.ascontiguousarray(inp.s_w)).to("cuda")
    out = torch.full(x.shape, float("nan"), device="cuda", dtype=torch.bfloat16)
    o = gpu_lib.qkv_w8a8_linear_attn(x, gpu_lib.pack_weight_i8(wt), sw, gains_dev(inp.gq), gains_dev(inp.gk), inp.H,
                                     inp.D, inp.eps, out=out)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("rows,C", [(1, 64), (6720, 2240), (13, 192), (300, 4480)])
def test_pack_weight_layout(gpu_lib, rows, C):
    """The packed weight against the layout written out: byte ((c // 64) * rows + n) * 64 + c % 64 = Wt[n, c]."""
    rng = np.random.default_rng(rows + C)
    wt = rng.integers(-127, 128, size=(rows, C), dtype=np.int8)
    wp = gpu_lib.pack_weight_i8(torch.from_numpy(wt).to("cuda"))
    torch.cuda.synchronize()
    flat = wp.cpu().numpy().reshape(-1)
    n, c = np.meshgrid(np.arange(rows), np.arange(C), indexing="ij")
    assert np.array_equal(flat[((c // 64) * rows + n) * 64 + c % 64], wt)


@pytest.mark.parametrize("rows,C", [(1, 2240), (37, 2240), (1000, 64), (5, 8), (300, 4480)])
def test_quantize_rows_bit_exact(gpu_lib, rows, C):
    rng = np.random.default_rng(rows * 7 + C)
    x = bf16_round((rng.standard_normal((rows, C)) * rng.uniform(0.01, 100.0, (rows, 1))).astype(np.float32))
    x[0, :] = 0.0                                  # all-zero row: codes 0, scale 0
    if rows > 2:
        x[2, :] = 0.0
        x[2, C // 2] = -3.0                        # a single value: it maps to -127, the rest to 0
    xq, sx = gpu_lib.quantize_rows_i8(dev(x, "bf16"))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows(x)
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("B,N,H,norm", [(1, 1, 70, True), (2, 300, 70, True), (1, 1037, 70, False),
                                        (3, 129, 2, True), (1, 513, 10, True)])
def test_w8a8_small_shapes(gpu_lib, B, N, H, norm):
    """Ragged row panels, column panels past 3C (C = 64 and 320) and the norm-off variant."""
    inp = gen_w8a8(600 + N + H, B, N, H=H, norm=norm)
    o_ref, parts = oracle.qkv_w8a8_linear_attn(inp.x, inp.wt_q, inp.s_w, inp.gq, inp.gk, H, 32, inp.eps,
                                               return_parts=True)
    o = _run(gpu_lib, inp)
    assert not torch.isnan(o).any()
    check(o, o_ref, parts["v"], "bf16", f"w8a8 B={B} N={N} H={H} norm={norm}")


def test_w8a8_2k_workload_sampled_rows(gpu_lib):
    """The 2K front-end shape (x [4, 4096, 2240]): the state from all tokens, outputs on sampled rows."""
    inp = gen_w8a8(5, 4, 4096)
    o = _run(gpu_lib, inp)
    assert not torch.isnan(o).any()
    C = inp.H * inp.D
    xq, sx = oracle.quantize_rows(inp.x)
    qkv = oracle.w8a8_project(xq, sx, inp.wt_q, inp.s_w)
    q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    phik = oracle.feature_map(k, inp.gk, inp.eps)
    S, z = oracle.kv_state(phik, v, inp.H, inp.D)
    rng = np.random.default_rng(0)
    idx = np.unique(np.concatenate([rng.choice(inp.N, size=96, replace=False), [0, inp.N - 1]]))
    phiq = oracle.feature_map(q[:, idx], inp.gq, inp.eps)
    o_ref = oracle.attend(phiq, S, z, inp.eps, inp.H, inp.D)
    check(o[:, torch.from_numpy(idx).to(o.device)], o_ref, v, "bf16", "w8a8 2K sampled rows")


def test_w8a8_argument_errors(gpu_lib):
    inp = gen_w8a8(9, 1, 16, H=3)                    # C = 96: not a multiple of 64
    x = dev(inp.x, "bf16")
    wt = torch.from_numpy(np.ascontiguousarray(inp.wt_q)).to("cuda")   # layout never read: the calls are rejected
    sw = torch.from_numpy(np.ascontiguousarray(inp.s_w)).to("cuda")
    out = torch.empty_like(x)
    with pytest.raises(gpu_lib.SanaError) as e:
        gpu_lib.sana_pack_weight_i8(wt, 9 * 32, 96, torch.empty_like(wt))
    assert e.value.status == 2
    with pytest.raises(gpu_lib.SanaError) as e:
        gpu_lib.sana_qkv_w8a8_linear_attn_fwd(x, wt, sw, gains_dev(inp.gq), gains_dev(inp.gk), 1, 16, 3, 32, 1e-6, out)
    assert e.value.status == 2
    with pytest.raises(gpu_lib.SanaError) as e:
        gpu_lib.sana_qkv_w8a8_linear_attn_fwd(x, wt, sw, gains_dev(inp.gq), None, 1, 16, 3, 32, 1e-6, out)
    assert e.value.status == 1

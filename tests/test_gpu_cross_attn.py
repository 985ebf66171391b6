"""GPU parity of the cross-attention with QK-Norm (sana_cross_attn_fwd) against the fp64 oracle
(oracle/cross_attn.py), element by element on seeded inputs.

Gates, derived from the arithmetic: the keys and queries enter the MFMA as bf16 after the norm (2^-9
relative each), so a logit of size s is off by about s * 2^-8; the softmax weights are rounded to bf16
for the value product (2^-9) and the output to bf16 (2^-9).  A weight error e_j moves the output by
sum_j p_j e_j (v_j - o), so the error stays a small multiple of 2^-8 of max|v - o|:
max |o_gpu - o_oracle| <= 2e-2 * max|V| (the bf16 gate of the self-attention) and, over the whole
tensor, RMS error <= 1e-2 * RMS(o_oracle)."""
import numpy as np
import pytest
import torch

import oracle
from synth import gen_cross
from tests.parity_util import dev, gains_dev

pytestmark = pytest.mark.gpu


def _run(sanala, inp, norm=True, kv=True, out=None):
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    gq, gk = (gains_dev(inp.gq), gains_dev(inp.gk)) if norm else (None, None)
    kv_len = torch.from_numpy(inp.kv_len).to("cuda") if kv else None
    if out is None:
        out = torch.full(q.shape, float("nan"), device="cuda", dtype=torch.bfloat16)
    o = sanala.cross_attn(q, k, v, gq, gk, inp.H, inp.D, inp.eps, kv_len=kv_len, out=out)
    torch.cuda.synchronize()
    return o


def _ref(inp, norm=True, kv=True):
    gq, gk = (inp.gq, inp.gk) if norm else (None, None)
    return oracle.cross_attn(inp.q, inp.k, inp.v, gq, gk, inp.H, inp.D, inp.eps, kv_len=inp.kv_len if kv else None)


def _check(o_gpu, ref, inp, label):
    og = o_gpu.float().cpu().numpy().astype(np.float64)
    assert not np.isnan(og).any(), f"{label}: NaN outputs"
    err = np.abs(og - ref)
    max_v = float(np.abs(inp.v).max())
    rms_err, rms_o = float(np.sqrt(np.mean(err * err))), float(np.sqrt(np.mean(ref * ref)))
    print(f"[cross] {label} max_err={err.max():.3e} max|V|={max_v:.3f} rms_err={rms_err:.3e} rms(o)={rms_o:.3e}",
          flush=True)
    assert err.max() <= 2e-2 * max_v, f"{label}: gate failed ({err.max()} vs {max_v})"
    assert rms_err <= 1e-2 * rms_o, f"{label}: RMS bound failed ({rms_err} vs {rms_o})"


@pytest.mark.parametrize("norm", [True, False], ids=["norm", "nonorm"])
@pytest.mark.parametrize("B,N,L,H,ragged", [(1, 1, 1, 1, False), (2, 100, 37, 3, True), (3, 257, 129, 5, True),
                                            (1, 70, 300, 70, False), (2, 33, 1024, 2, True)])
def test_cross_small_and_ragged(gpu_lib, B, N, L, H, ragged, norm):
    inp = gen_cross(31, B, N, L=L, H=H, ragged=ragged, norm=norm)
    print(f"[cross] B={B} N={N} L={L} H={H} ragged={ragged} norm={norm} kv_len={inp.kv_len.tolist()}", flush=True)
    _check(_run(gpu_lib, inp, norm), _ref(inp, norm), inp, f"B{B} N{N} L{L} H{H}")


@pytest.mark.parametrize("N", [1024, 16384])
def test_cross_sana_shapes(gpu_lib, N):
    """SANA widths: 70 heads of 32, 300 text tokens, 1024px (N = 1024) and 4K (N = 16384) latents."""
    inp = gen_cross(32, 1, N, L=300)
    _check(_run(gpu_lib, inp), _ref(inp), inp, f"N{N} L300 H70")


def test_cross_all_keys_without_lengths(gpu_lib):
    inp = gen_cross(33, 2, 200, L=77, H=4, ragged=True)
    _check(_run(gpu_lib, inp, kv=False), _ref(inp, kv=False), inp, "kv_len NULL")


def test_cross_one_valid_token_returns_its_value(gpu_lib):
    """One valid text token: every weight is exactly 1, so the output is that token's v (bf16, exact)."""
    inp = gen_cross(34, 2, 90, L=50, H=3)
    inp.kv_len[:] = 1
    o = _run(gpu_lib, inp).float().cpu().numpy()
    for b in range(2):
        np.testing.assert_array_equal(o[b], np.broadcast_to(inp.v[b, 0], o[b].shape))


def test_cross_peaked_logits_norm_off(gpu_lib):
    """Norm off with keys 30x larger: logits in the hundreds, softmax close to one-hot.  The norm bound on
    the logits is too loose here to stand in for the maximum, so the kernel takes the exact-maximum pass."""
    inp = gen_cross(35, 1, 300, L=300, H=4, norm=False, k_scale=30.0)
    _check(_run(gpu_lib, inp, norm=False), _ref(inp, norm=False), inp, "peaked")


def test_cross_loose_bound_norm_on(gpu_lib):
    """Norm on, with query 3 and text token 7 of every sample concentrated on one channel each of head 0
    (channels 0 and 1, so the two are orthogonal): after the norm their head-0 parts have norms near
    sqrt(C), so |q^| max|k^| bounds head 0's logits too loosely (2m > 64 in exponent units) and the
    wave takes the exact-maximum pass, whose maximum then enters the MFMA as the subtracted constant,
    while the logits themselves stay moderate."""
    inp = gen_cross(40, 2, 300, L=120, H=8, ragged=True)
    inp.q[:, 3, :32] = 0.0
    inp.q[:, 3, 0] = 60.0
    inp.k[:, 7, :32] = 0.0
    inp.k[:, 7, 1] = 60.0
    assert (inp.kv_len > 7).all()
    _check(_run(gpu_lib, inp), _ref(inp), inp, "loose bound, norm on")


def test_cross_zero_valid_tokens_gives_zeros(gpu_lib):
    """kv_len 0 (not defined by the oracle, which requires >= 1): the library writes zeros."""
    inp = gen_cross(36, 2, 64, L=20, H=2)
    inp.kv_len[:] = [0, 20]
    o = _run(gpu_lib, inp).float().cpu().numpy()
    assert (o[0] == 0).all()
    ref = oracle.cross_attn(inp.q[1:], inp.k[1:], inp.v[1:], inp.gq, inp.gk, inp.H, inp.D, inp.eps)
    err = np.abs(o[1:] - ref).max()
    assert err <= 2e-2 * np.abs(inp.v).max()


def test_cross_bitwise_repeatable(gpu_lib):
    inp = gen_cross(37, 2, 513, L=300, H=6, ragged=True)
    a, b = _run(gpu_lib, inp), _run(gpu_lib, inp)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_cross_argument_errors(gpu_lib):
    inp = gen_cross(38, 1, 8, L=4, H=2)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    out = torch.empty_like(q)
    with pytest.raises(gpu_lib.SanaError):  # 1025 text tokens: beyond the staged-key limit
        kk = torch.zeros(1, 1025, 64, device="cuda", dtype=torch.bfloat16)
        gpu_lib.sana_cross_attn_fwd(q, kk, kk, None, None, None, 1, 8, 1025, 2, 32, 1e-6, out)
    with pytest.raises(gpu_lib.SanaError):  # fp32 storage is not provided
        qf = q.float()
        gpu_lib.sana_cross_attn_fwd(qf, k.float(), v.float(), None, None, None, 1, 8, 4, 2, 32, 1e-6, qf.clone(),
                                    dtype=0)
    with pytest.raises(gpu_lib.SanaError):  # out overlapping q
        gpu_lib.sana_cross_attn_fwd(q, k, v, None, None, None, 1, 8, 4, 2, 32, 1e-6, q)
    with pytest.raises(ValueError):  # wrong kv_len dtype (binding check)
        gpu_lib.sana_cross_attn_fwd(q, k, v, None, None, torch.ones(1, device="cuda"), 1, 8, 4, 2, 32, 1e-6, out)


def test_cross_long_sequence_many_tiles_per_wave(gpu_lib):
    """40000 image tokens over 4 heads: few blocks per head, each wave taking many query tiles (and a
    ragged last tile)."""
    inp = gen_cross(39, 1, 40000, L=300, H=4, ragged=True)
    _check(_run(gpu_lib, inp), _ref(inp), inp, "N40000 H4")

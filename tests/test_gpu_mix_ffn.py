"""GPU parity of Mix-FFN against the oracle.

Mix-FFN: "Sana: Efficient High-Resolution Image Synthesis with Linear Diffusion Transformers" (paper
notes), sections 2.2 and 2.3; width 5600 at 2240 channels (SANA 1.5 research notes, architecture).
The device rounds h = x W1, the gated g and the output to bf16 and sums in fp32.  Each rounding has
a relative RMS error of about 2^-8 / sqrt(12) = 1.1e-3, and the three of them (h passing through the
convolution and the gate) leave about 3e-3 of the output's RMS; the gates below are twice that, RMS
err <= 6e-3 RMS y, and max |err| <= 1e-2 max |y|.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import gen_mix_ffn
from tests.parity_util import dev

pytestmark = pytest.mark.gpu

MAX_GATE, RMS_GATE = 1e-2, 6e-3


def _run(gpu_lib, inp):
    x, w1, kdw, w2 = (dev(a, "bf16") for a in (inp.x, inp.w1, inp.kdw, inp.w2))
    out = torch.full(x.shape, float("nan"), device="cuda", dtype=torch.bfloat16)
    o = gpu_lib.mix_ffn(x, w1, kdw, w2, inp.Hg, inp.Wg, out=out)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


def _check(got, ref, label):
    assert not np.isnan(got).any(), f"{label}: NaN outputs"
    err = np.abs(got.astype(np.float64) - ref)
    rms_err, rms_ref = np.sqrt(np.mean(err ** 2)), np.sqrt(np.mean(ref ** 2))
    print(f"[parity] {label} max_err={err.max():.3e} max|y|={np.abs(ref).max():.3e} rms_err/rms_y={rms_err / rms_ref:.3e}",
          flush=True)
    assert err.max() <= MAX_GATE * np.abs(ref).max(), label
    assert rms_err <= RMS_GATE * rms_ref, label


@pytest.mark.parametrize("B,Hg,Wg,C,F", [(1, 1, 1, 64, 64), (2, 3, 5, 64, 96), (1, 8, 8, 2240, 5600),
                                         (2, 17, 13, 96, 160), (1, 5, 128, 64, 32)])
def test_mix_ffn_small_grids(gpu_lib, B, Hg, Wg, C, F):
    """Single token, ragged grids, a half-filled 64-channel chunk (F = 96, 160), the widest row."""
    inp = gen_mix_ffn(700 + Hg * Wg + F, B, Hg, Wg, C=C, F=F)
    ref = oracle.mix_ffn(inp.x, inp.w1, inp.kdw, inp.w2, Hg, Wg)
    _check(_run(gpu_lib, inp), ref, f"mix-ffn B={B} {Hg}x{Wg} C={C} F={F}")


def test_mix_ffn_2k_grid_sampled_tokens(gpu_lib):
    """x [4, 64x64, 2240], F = 5600: the oracle on sampled tokens from their 3x3 neighbourhoods
    (zero outside the grid), grid corners and edges included."""
    inp = gen_mix_ffn(5, 4, 64, 64)
    got = _run(gpu_lib, inp)
    rng = np.random.default_rng(0)
    picks = [(b, i, j) for b in range(4) for (i, j) in [(0, 0), (0, 63), (63, 0), (63, 63), (0, 17), (40, 63)]]
    picks += [(int(rng.integers(4)), int(rng.integers(64)), int(rng.integers(64))) for _ in range(40)]
    ref, out = [], []
    for b, i, j in picks:
        patch = np.zeros((1, 9, inp.x.shape[2]))
        for p in range(3):
            for q in range(3):
                ii, jj = i + p - 1, j + q - 1
                if 0 <= ii < 64 and 0 <= jj < 64:
                    patch[0, 3 * p + q] = inp.x[b, ii * 64 + jj]
        y = oracle.mix_ffn(patch, inp.w1, inp.kdw, inp.w2, 3, 3)  # zero rows stand for the padding
        ref.append(y[0, 4])
        out.append(got[b, i * 64 + j])
    _check(np.array(out), np.array(ref), "mix-ffn 2K sampled tokens")


def test_mix_ffn_argument_errors(gpu_lib):
    inp = gen_mix_ffn(9, 1, 2, 2, C=64, F=48)      # F not a multiple of 32
    x, w1, kdw, w2 = (dev(a, "bf16") for a in (inp.x, inp.w1, inp.kdw, inp.w2))
    out = torch.empty_like(x)
    with pytest.raises(gpu_lib.SanaError) as e:
        gpu_lib.sana_mix_ffn_fwd(x, w1, kdw, w2, 1, 2, 2, 64, 48, out)
    assert e.value.status == 2
    wide = gen_mix_ffn(10, 1, 1, 300, C=64, F=64)   # Wg > 128 (checked before any use)
    x, w1, kdw, w2 = (dev(a, "bf16") for a in (wide.x, wide.w1, wide.kdw, wide.w2))
    with pytest.raises(gpu_lib.SanaError) as e:
        gpu_lib.sana_mix_ffn_fwd(x, w1, kdw, w2, 1, 1, 300, 64, 64, torch.empty_like(x))
    assert e.value.status == 2

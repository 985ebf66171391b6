"""The bf16 GEMMs at both block widths (192 and 256 output columns per block; SANA_GEMM_WIDE forces one).
Each output element is summed over K in the same order at either width, so the Mix-FFN's output is the
same bit for bit; the fused projection's K row statistics are summed over column panels that differ
with the width, so there both widths are held to the oracle's gates.  Shapes are ragged in rows
(several 256-row panels, the last partial) and in columns at both widths, and the K block of the
fused projection spans two 256-column panels or three 192-column ones."""
import os

import numpy as np
import pytest
import torch

import oracle
from synth import gen_mix_ffn, gen_qkv
from tests.parity_util import check, dev, gains_dev
from tests.test_gpu_mix_ffn import _check as check_mix

pytestmark = pytest.mark.gpu


def _at_width(wide, fn):
    old = os.environ.get("SANA_GEMM_WIDE")
    os.environ["SANA_GEMM_WIDE"] = "1" if wide else "0"
    try:
        return fn()
    finally:
        if old is None:
            del os.environ["SANA_GEMM_WIDE"]
        else:
            os.environ["SANA_GEMM_WIDE"] = old


def test_mix_ffn_both_widths(gpu_lib):
    """C = 320, F = 224: 2F = 448 columns (panels 256 + 192 or 192 + 192 + 64), C = 320 (256 + 64 or
    192 + 128); 2 x 17 x 31 = 1054 rows (five 256-row panels)."""
    inp = gen_mix_ffn(7301, 2, 17, 31, C=320, F=224)
    x, w1, kdw, w2 = (dev(a, "bf16") for a in (inp.x, inp.w1, inp.kdw, inp.w2))
    ref = oracle.mix_ffn(inp.x, inp.w1, inp.kdw, inp.w2, inp.Hg, inp.Wg)
    outs = []
    for wide in (False, True):
        print(f"[widths] mix-ffn wide={wide}", flush=True)
        o = _at_width(wide, lambda: gpu_lib.mix_ffn(x, w1, kdw, w2, inp.Hg, inp.Wg))
        torch.cuda.synchronize()
        check_mix(o.float().cpu().numpy(), ref, f"mix-ffn wide={wide}")
        outs.append(o)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_fused_projection_both_widths(gpu_lib):
    """H = 11 (C = 352, 3C = 1056 columns: panels 4 x 256 + 32 or 5 x 192 + 96), 2 x 300 rows."""
    inp = gen_qkv(7302, 2, 300, H=11)
    o_ref, parts = oracle.qkv_linear_attn(inp.x, inp.w, inp.gq, inp.gk, inp.H, inp.D, inp.eps, return_parts=True)
    x, w = dev(inp.x, "bf16"), dev(inp.w, "bf16")
    gq, gk = gains_dev(inp.gq), gains_dev(inp.gk)
    for wide in (False, True):
        print(f"[widths] fused projection wide={wide}", flush=True)
        o = _at_width(wide, lambda: gpu_lib.qkv_linear_attn(x, w, gq, gk, inp.H))
        torch.cuda.synchronize()
        check(o, o_ref, parts["v"], "bf16", f"fused projection wide={wide}")

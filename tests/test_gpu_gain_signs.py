"""QK-Norm gains of either sign.  The gains are learned and may be negative; phi(x) = ReLU(x * r * g)
then keeps the entries where x and g have opposite signs ("Sana" paper notes, section 2.1, Eq. (1); the
QK Norm bullet of the SANA 1.5 notes).  The 16-bit kernels fold the sign of each gain into the bf16
operands (ReLU(sign(g) * x), exact in bf16) and its magnitude into the reduced state, and the
cross-attention folds the gains into its normalised operands, so every route is checked against the fp64
oracle with about 30% of the gain signs flipped, at the usual gates."""
import os

import numpy as np
import pytest
import torch

import oracle
from synth import gen_attn, gen_cross, gen_qkv, gen_w8a8
from tests.parity_util import check, dev, gains_dev, oracle_out, run_attn

pytestmark = pytest.mark.gpu


def _flip(g, seed):
    rng = np.random.default_rng(seed)
    signs = np.where(rng.random(g.shape[0]) < 0.3, -1.0, 1.0)
    return (g * signs).astype(np.float32)


def _with_env(env, fn):
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        return fn()
    finally:
        for k, v in old.items():
            if v is None:
                del os.environ[k]
            else:
                os.environ[k] = v


# (dtype, B, N, H): the fp32 path; the persistent output kernel (8200 tokens), also at odd H; the
# head-group tile kernel (few tiles); binary16; H = 80 (tile kernel with its own r_q pass).
CASES = [("f32", 2, 300, 70), ("bf16", 1, 8200, 70), ("bf16", 1, 8200, 71), ("bf16", 1, 1000, 70),
         ("f16", 2, 600, 70), ("bf16", 2, 150, 80)]


@pytest.mark.parametrize("dtype,B,N,H", CASES)
def test_linear_attn_gain_signs(gpu_lib, dtype, B, N, H):
    inp = gen_attn(4100 + N + H, B, N, H=H, dtype=dtype)
    inp.gq, inp.gk = _flip(inp.gq, 1), _flip(inp.gk, 2)
    print(f"[signs] {dtype} B={B} N={N} H={H}", flush=True)
    check(run_attn(gpu_lib, inp), oracle_out(inp), inp.v, dtype, f"signs {dtype} B={B} N={N} H={H}")


@pytest.mark.parametrize("env", [{"SANA_STATE_XCHG": "1"}, {"SANA_STATE_RENDEZVOUS": "1"}],
                         ids=["state_exchange", "rendezvous"])
def test_optional_routes_gain_signs(gpu_lib, env):
    """The optional state routes with flipped gains: the rendezvous sums the chunks in the reduction
    launch's order (same bits); the exchange forms r_k by another order of the same sum (a few bf16 ulps
    from the default route); both meet the oracle's gates."""
    inp = gen_attn(4200, 1, 8200, dtype="bf16")
    inp.gq, inp.gk = _flip(inp.gq, 3), _flip(inp.gk, 4)
    o_route = _with_env(env, lambda: run_attn(gpu_lib, inp))
    o_default = run_attn(gpu_lib, inp)
    check(o_route, oracle_out(inp), inp.v, "bf16", f"signs {env}")
    if "SANA_STATE_RENDEZVOUS" in env:
        assert torch.equal(o_route.view(torch.int16), o_default.view(torch.int16))
    else:
        diff = (o_route.float() - o_default.float()).abs().max().item()
        assert diff <= 2e-2 * o_route.float().abs().max().item(), diff


def test_fused_projection_gain_signs(gpu_lib):
    """The K statistics come from the projection's epilogue on this path."""
    inp = gen_qkv(4300, 2, 300, H=70)
    gq, gk = _flip(inp.gq, 5), _flip(inp.gk, 6)
    o_ref, parts = oracle.qkv_linear_attn(inp.x, inp.w, gq, gk, inp.H, inp.D, inp.eps, return_parts=True)
    o = gpu_lib.qkv_linear_attn(dev(inp.x, "bf16"), dev(inp.w, "bf16"), gains_dev(gq), gains_dev(gk), inp.H)
    torch.cuda.synchronize()
    check(o, o_ref, parts["v"], "bf16", "signs fused projection")


def test_w8a8_gain_signs(gpu_lib):
    inp = gen_w8a8(4400, 1, 300)
    gq, gk = _flip(inp.gq, 7), _flip(inp.gk, 8)
    o_ref, parts = oracle.qkv_w8a8_linear_attn(inp.x, inp.wt_q, inp.s_w, gq, gk, inp.H, 32, inp.eps,
                                               return_parts=True)
    x = dev(inp.x, "bf16")
    wt = torch.from_numpy(np.ascontiguousarray(inp.wt_q)).to("cuda")
    sw = torch.from_numpy(np.ascontiguousarray(inp.s_w)).to("cuda")
    o = gpu_lib.qkv_w8a8_linear_attn(x, gpu_lib.pack_weight_i8(wt), sw, gains_dev(gq), gains_dev(gk), inp.H, inp.D,
                                     inp.eps)
    torch.cuda.synchronize()
    check(o, o_ref, parts["v"], "bf16", "signs w8a8")


def test_cross_attn_gain_signs(gpu_lib):
    """Cross-attention gates: max error <= 2e-2 max|V|, RMS error <= 1e-2 RMS(o)."""
    inp = gen_cross(4500, 2, 500, L=300, H=70, ragged=True)
    inp.gq, inp.gk = _flip(inp.gq, 9), _flip(inp.gk, 10)
    q, k, v = dev(inp.q, "bf16"), dev(inp.k, "bf16"), dev(inp.v, "bf16")
    kv_len = torch.from_numpy(inp.kv_len).to("cuda")
    o = gpu_lib.cross_attn(q, k, v, gains_dev(inp.gq), gains_dev(inp.gk), inp.H, inp.D, inp.eps, kv_len=kv_len)
    torch.cuda.synchronize()
    ref = oracle.cross_attn(inp.q, inp.k, inp.v, inp.gq, inp.gk, inp.H, inp.D, inp.eps, kv_len=inp.kv_len)
    og = o.float().cpu().numpy().astype(np.float64)
    err = np.abs(og - ref)
    rms_err, rms_o = float(np.sqrt(np.mean(err * err))), float(np.sqrt(np.mean(ref * ref)))
    print(f"[signs] cross max_err={err.max():.3e} rms_err={rms_err:.3e} rms(o)={rms_o:.3e}", flush=True)
    assert not np.isnan(og).any()
    assert err.max() <= 2e-2 * np.abs(inp.v).max()
    assert rms_err <= 1e-2 * rms_o

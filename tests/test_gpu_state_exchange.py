"""The state pass that forms r_k itself (one read of K; the blocks of a token chunk exchange per-head-pair
sums of squares as epoch-tagged values), selected with SANA_STATE_XCHG=1.  Its waits are bounded; past the limit a block forms the
missing values from the full K rows with the same arithmetic in the same order.  A wait limit of 0
(set from the host) sends most waits down that route: the output must not change by a single bit.
Both routes, and the separate row-statistics pass, against the fp64 oracle."""
import os

import pytest
import torch

from synth import gen_attn, gen_config
from tests.parity_util import check, dev, gains_dev, oracle_out

pytestmark = pytest.mark.gpu


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


def _run(sanala, inp):
    q, k, v = dev(inp.q, inp.dtype), dev(inp.k, inp.dtype), dev(inp.v, inp.dtype)
    out = torch.full(q.shape, float("nan"), device="cuda", dtype=q.dtype)
    o = sanala.linear_attn(q, k, v, gains_dev(inp.gq), gains_dev(inp.gk), inp.H, inp.D, inp.eps, out=out)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("case", ["config4", "b2_n8200_h71", "b3_n3000_f16", "b1_n70000", "b4_n1024"])
def test_exchange_routes_agree_bitwise(gpu_lib, case):
    inp = {"config4": lambda: gen_config(4),
           "b2_n8200_h71": lambda: gen_attn(81, 2, 8200, H=71, dtype="bf16"),
           "b3_n3000_f16": lambda: gen_attn(82, 3, 3000, dtype="f16"),
           "b1_n70000": lambda: gen_attn(83, 1, 70000, dtype="bf16"),
           "b4_n1024": lambda: gen_attn(84, 4, 1024, dtype="bf16")}[case]()
    print(f"[xchg] {case}", flush=True)
    o_x = _with_env({"SANA_STATE_XCHG": "1"}, lambda: _run(gpu_lib, inp))
    o_late = _with_env({"SANA_STATE_XCHG": "1", "SANA_XCHG_SPIN_US": "0"}, lambda: _run(gpu_lib, inp))
    o_sep = _with_env({"SANA_STATE_XCHG": "0"}, lambda: _run(gpu_lib, inp))
    assert not torch.isnan(o_x).any()
    assert torch.equal(o_x.view(torch.int16), o_late.view(torch.int16)), "local route differs from the exchange"
    if inp.N <= 20000:
        ref = oracle_out(inp)
        check(o_x, ref, inp.v, inp.dtype, f"exchange {case}")
        check(o_sep, ref, inp.v, inp.dtype, f"separate statistics {case}")
    # the two ways of forming r_k differ only in the order of a sum: outputs within a few bf16 ulps
    diff = (o_x.float() - o_sep.float()).abs().max().item()
    assert diff <= 2e-2 * o_x.float().abs().max().item(), diff


def test_exchange_repeats_bitwise_across_calls(gpu_lib):
    inp = gen_attn(85, 1, 16384, dtype="bf16")
    outs = [_with_env({"SANA_STATE_XCHG": "1"}, lambda: _run(gpu_lib, inp)) for _ in range(3)]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


@pytest.mark.parametrize("case", ["b32_n1024", "b4_n1000_f16", "b2_n777_norm_off", "b1_n4096"])
def test_kv_load_forms_agree_bitwise(gpu_lib, case):
    """Non-temporal K and V loads in the row-statistics and state passes (the planner's choice when K and
    V together exceed the Infinity Cache, and behind the fused projection; SANA_STATE_NT_V forces either
    form) change only the loads' cache policy: the output must be the same bit for bit, and within the
    oracle's gates.  Cases: the 32-sample batch (non-temporal by default), a binary16 batch, a batch with
    the norm off, a single sample (ordinary by default)."""
    inp = {"b32_n1024": lambda: gen_config(3),
           "b4_n1000_f16": lambda: gen_attn(7401, 4, 1000, dtype="f16"),
           "b2_n777_norm_off": lambda: gen_attn(7402, 2, 777, dtype="bf16", norm=False),
           "b1_n4096": lambda: gen_attn(7403, 1, 4096, dtype="bf16")}[case]()
    print(f"[nt-v] {case}", flush=True)
    outs = [_with_env({"SANA_STATE_NT_V": f}, lambda: _run(gpu_lib, inp)) for f in ("0", "1")]
    bits = torch.int16
    assert torch.equal(outs[0].view(bits), outs[1].view(bits)), case
    if case != "b32_n1024":  # the 32-sample batch is checked against the oracle elsewhere
        check(outs[1], oracle_out(inp), inp.v, inp.dtype, f"nt-v {case}")

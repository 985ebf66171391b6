"""Chunk reduction inside the state pass (the rendezvous, SANA_STATE_RENDEZVOUS=1): when a sequence is
split into several token chunks, the state blocks of a head pair publish their chunk partials and each
sums one slice of the pair's state over all chunks, instead of the separate reduction launch (the
default).  Its waits are bounded; a chunk whose partial has not appeared by the limit is formed by the
waiting block itself.  Every route sums the chunks in the same order, so the reduction launch, the
rendezvous, and the rendezvous with a wait limit of 0 (most waits then take the local route) must agree
bit for bit; each is also checked against the fp64 oracle."""
import os

import pytest
import torch

from synth import gen_attn, gen_config
import oracle
from tests.parity_util import check, dev, gains_dev

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


def _run(sanala, inp, norm=True):
    q, k, v = dev(inp.q, inp.dtype), dev(inp.k, inp.dtype), dev(inp.v, inp.dtype)
    out = torch.full(q.shape, float("nan"), device="cuda", dtype=q.dtype)
    gq, gk = (gains_dev(inp.gq), gains_dev(inp.gk)) if norm else (None, None)
    o = sanala.linear_attn(q, k, v, gq, gk, inp.H, inp.D, inp.eps, out=out)
    torch.cuda.synchronize()
    return o


CASES = {
    "config4": lambda: gen_config(4),                              # 14 chunks of 1216 tokens
    "config2": lambda: gen_config(2),                              # 8 chunks of 128 tokens
    "b2_n8200_h71": lambda: gen_attn(91, 2, 8200, H=71, dtype="bf16"),  # odd H: the last pair has one head
    "b3_n3000_f16": lambda: gen_attn(92, 3, 3000, dtype="f16"),
    "b1_n700_h3": lambda: gen_attn(93, 1, 700, H=3, dtype="bf16"),  # few pairs, ragged last chunk
    "b1_n70000": lambda: gen_attn(94, 1, 70000, dtype="bf16"),     # beyond 16 chunks: reduction launch
}


@pytest.mark.parametrize("norm", [True, False], ids=["norm", "nonorm"])
@pytest.mark.parametrize("case", list(CASES))
def test_rendezvous_routes_agree_bitwise(gpu_lib, case, norm):
    inp = CASES[case]()
    print(f"[rendezvous] {case} norm={norm}", flush=True)
    o_r = _with_env({"SANA_STATE_RENDEZVOUS": "1"}, lambda: _run(gpu_lib, inp, norm))
    o_late = _with_env({"SANA_STATE_RENDEZVOUS": "1", "SANA_XCHG_SPIN_US": "0"}, lambda: _run(gpu_lib, inp, norm))
    o_launch = _run(gpu_lib, inp, norm)
    assert not torch.isnan(o_r).any()
    assert torch.equal(o_r.view(torch.int16), o_launch.view(torch.int16)), "rendezvous differs from the reduction launch"
    assert torch.equal(o_r.view(torch.int16), o_late.view(torch.int16)), "local route differs from the rendezvous"
    if inp.N * inp.B <= 20000:
        gq, gk = (inp.gq, inp.gk) if norm else (None, None)
        ref = oracle.linear_attn(inp.q, inp.k, inp.v, gq, gk, inp.H, inp.D, inp.eps)
        check(o_r, ref, inp.v, inp.dtype, f"rendezvous {case}")


def test_rendezvous_repeats_bitwise_across_calls(gpu_lib):
    inp = gen_config(2)
    outs = [_with_env({"SANA_STATE_RENDEZVOUS": "1"}, lambda: _run(gpu_lib, inp)) for _ in range(4)]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))

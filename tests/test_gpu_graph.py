"""The allocation-free entry point inside a HIP graph (torch.cuda.CUDAGraph): for callers that replay a
fixed sequence of launches (a sampler's steps) without host work per call.  The call is captured once
and replayed several times with eager work on the same device in between; every replay must give the
bits of the eager allocating call on the same inputs, and a replay after new values have been copied
into the captured inputs must give the eager result for those values.  The cases cover one chunk per
head pair, several chunks with the reduction launch, the head-group output kernel and the fp32 path."""
import pytest
import torch

from synth import gen_attn
from tests.parity_util import dev, gains_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)


@pytest.mark.parametrize("seed,B,N,dtype", [(81, 1, 1024, "bf16"), (82, 2, 777, "bf16"), (83, 1, 64, "bf16"),
                                            (84, 1, 300, "f32")])
def test_graph_replays_give_the_eager_bits(gpu_lib, seed, B, N, dtype):
    print(f"[graph] B={B} N={N} {dtype}", flush=True)
    inp = gen_attn(seed, B, N, dtype=dtype)
    q, k, v = dev(inp.q, dtype), dev(inp.k, dtype), dev(inp.v, dtype)
    gq, gk = gains_dev(inp.gq), gains_dev(inp.gk)
    H, D, eps = inp.H, inp.D, inp.eps
    out = torch.empty_like(q)

    def call():
        gpu_lib.sana_linear_attn_fwd_noalloc(q, k, v, gq, gk, B, N, H, D, eps, out)

    call()  # the static scratch's address and the kernels' LDS limits are set up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()

    def eager():
        ref = torch.empty_like(q)
        gpu_lib.sana_linear_attn_fwd(q, k, v, gq, gk, B, N, H, D, eps, ref)
        return ref

    ref = eager()
    for r in range(3):
        out.fill_(float("nan"))
        other = dev(gen_attn(seed + 1000 + r, 1, 200, dtype=dtype).q, dtype)  # eager work between replays
        junk = torch.empty_like(other)
        gpu_lib.sana_linear_attn_fwd(other, other, other, None, None, 1, 200, H, D, eps, junk)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), f"replay {r}"
    new = gen_attn(seed + 2000, B, N, dtype=dtype)
    for t, a in ((q, new.q), (k, new.k), (v, new.v)):
        t.copy_(dev(a, dtype))
    g.replay()
    ref2 = eager()
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref2)), "replay on new inputs"
    assert not torch.equal(_bits(ref2), _bits(ref))

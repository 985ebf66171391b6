"""The allocation-free entry point (static per-device scratch) against sana_linear_attn_fwd: the same
kernels on the same inputs, so the outputs must agree bit for bit; each is also within the gates of
the fp64 oracle.  Two calls in a row, the second on a smaller input (the static buffer keeps the first
call's contents), then a third of another dtype."""
import pytest
import torch

from synth import gen_attn, gen_config
from tests.parity_util import check, dev, gains_dev, oracle_out

pytestmark = pytest.mark.gpu


def _both(sanala, inp):
    q, k, v = dev(inp.q, inp.dtype), dev(inp.k, inp.dtype), dev(inp.v, inp.dtype)
    gq, gk = gains_dev(inp.gq), gains_dev(inp.gk)
    B, N = q.shape[0], q.shape[1]
    ref = torch.empty_like(q)
    sanala.sana_linear_attn_fwd(q, k, v, gq, gk, B, N, inp.H, inp.D, inp.eps, ref)
    out = torch.full_like(q, float("nan"))
    sanala.sana_linear_attn_fwd_noalloc(q, k, v, gq, gk, B, N, inp.H, inp.D, inp.eps, out)
    torch.cuda.synchronize()
    return out, ref


def test_no_alloc_entry_point_matches_the_allocating_one(gpu_lib):
    cases = [(gen_config(4), "16384 tokens"), (gen_attn(71, 2, 1000, dtype="bf16"), "2 x 1000 tokens"),
             (gen_attn(72, 1, 300, dtype="f32"), "fp32 300 tokens")]
    for inp, label in cases:
        print(f"[no-alloc] {label}", flush=True)
        out, ref = _both(gpu_lib, inp)
        bits = torch.int32 if out.dtype == torch.float32 else torch.int16
        assert torch.equal(out.view(bits), ref.view(bits)), label
        check(out, oracle_out(inp), inp.v, inp.dtype, f"no-alloc {label}")


def test_no_alloc_entry_point_rejects_calls_beyond_its_scratch(gpu_lib):
    # 512 samples of 1024 tokens need about 80 MB of scratch: rejected before anything is enqueued
    with pytest.raises(gpu_lib.SanaError) as e:
        lib = gpu_lib.load_library()
        T = 1 << 40  # fake, far-apart device addresses: the call must return before touching any
        st = lib.sana_linear_attn_fwd_noalloc(T, 2 * T, 3 * T, 4 * T, 4 * T + 16384, 512, 1024, 70, 32, 1e-6,
                                              5 * T, 0, 1)
        raise gpu_lib.SanaError(st, "sana_linear_attn_fwd_noalloc")
    assert e.value.status == 5

"""Calls that overlap on the GPU.  Four streams each queue a different workload many times without
synchronising: the bf16 attention over split chunks (with its reduction launch), the fp32 attention,
the fused projection and the cross-attention over ragged text lengths.  Each stream's calls hold that
stream's scratch, so calls on different streams may run at the same time without sharing memory, and
every kernel sums in a fixed order: each output must equal the single-stream result bit for bit."""
import numpy as np
import pytest
import torch

from synth import gen_attn, gen_cross, gen_qkv
from tests.parity_util import dev, gains_dev

pytestmark = pytest.mark.gpu

REPS = 24


def _workloads(gpu_lib):
    """[(name, call(out) -> None, out template)]: each call writes into the output it is given."""
    a = gen_attn(7101, 1, 8200, dtype="bf16")
    aq, ak, av = dev(a.q, "bf16"), dev(a.k, "bf16"), dev(a.v, "bf16")
    agq, agk = gains_dev(a.gq), gains_dev(a.gk)
    f = gen_attn(7102, 2, 300, dtype="f32")
    fq, fk, fv = dev(f.q, "f32"), dev(f.k, "f32"), dev(f.v, "f32")
    fgq, fgk = gains_dev(f.gq), gains_dev(f.gk)
    p = gen_qkv(7103, 1, 600, H=70)
    px, pw = dev(p.x, "bf16"), dev(p.w, "bf16")
    pgq, pgk = gains_dev(p.gq), gains_dev(p.gk)
    c = gen_cross(7104, 2, 500, L=300, H=70, ragged=True)
    cq, ck, cv = dev(c.q, "bf16"), dev(c.k, "bf16"), dev(c.v, "bf16")
    cgq, cgk = gains_dev(c.gq), gains_dev(c.gk)
    kv_len = torch.from_numpy(np.ascontiguousarray(c.kv_len)).to("cuda")
    return [
        ("attn bf16 8200", lambda out: gpu_lib.linear_attn(aq, ak, av, agq, agk, a.H, out=out), aq),
        ("attn f32 2x300", lambda out: gpu_lib.linear_attn(fq, fk, fv, fgq, fgk, f.H, out=out), fq),
        ("fused projection 600", lambda out: gpu_lib.qkv_linear_attn(px, pw, pgq, pgk, p.H, out=out), px),
        ("cross 2x500 L=300", lambda out: gpu_lib.cross_attn(cq, ck, cv, cgq, cgk, c.H, kv_len=kv_len, out=out), cq),
    ]


def test_overlapping_calls_on_four_streams(gpu_lib):
    work = _workloads(gpu_lib)
    refs = []
    for name, call, like in work:
        ref = torch.empty_like(like)
        call(ref)
        refs.append(ref)
    outs = [[torch.full_like(like, float("nan")) for _ in range(REPS)] for _, _, like in work]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in work]
    print(f"[concurrent] {len(work)} streams x {REPS} calls", flush=True)
    for r in range(REPS):  # the streams' queues interleave call by call
        for (name, call, _), s, o in zip(work, streams, outs):
            with torch.cuda.stream(s):
                call(o[r])
    torch.cuda.synchronize()
    for (name, _, _), ref, o in zip(work, refs, outs):
        bits = torch.int32 if ref.dtype == torch.float32 else torch.int16
        for r in range(REPS):
            assert torch.equal(o[r].view(bits), ref.view(bits)), f"{name}: call {r}"
    for s in streams:
        gpu_lib.sana_release_scratch(stream=s.cuda_stream)

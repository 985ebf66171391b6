"""Measurement support: per-kernel durations from the start/stop events of each kernel's own dispatch
(sana_timing_enable / sana_timing_last).  Timing must not change results, and must record nothing once
switched off."""
import pytest
import torch

from synth import gen_config
from tests.parity_util import run_attn

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N", [4096, 16384])
def test_timing_records_each_kernel_and_leaves_results_unchanged(gpu_lib, N):
    inp = gen_config(4, N=N)
    o_plain = run_attn(gpu_lib, inp)
    gpu_lib.sana_timing_enable(True)
    try:
        o_timed = run_attn(gpu_lib, inp)
        rec = gpu_lib.sana_timing_last()
    finally:
        gpu_lib.sana_timing_enable(False)
    names = [n for n, _ in rec]
    assert "kv_state" in names and names[-1] == "out", names
    assert all(ms > 0.0 for _, ms in rec), rec
    assert torch.equal(o_plain.view(torch.int16), o_timed.view(torch.int16))
    run_attn(gpu_lib, inp)
    assert gpu_lib.sana_timing_last() == []

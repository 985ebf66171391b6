"""Input generators: bf16 rounding, determinism and the workload shapes (no GPU needed)."""
import hashlib

import numpy as np
import pytest
import torch

from synth import CONFIGS, bf16_bits, bf16_round, gen_attn, gen_config, gen_qkv


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.4e38, 1e-45, np.inf, -np.inf], np.float32),
    ]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_bits(x), want)


def test_bf16_ties_to_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to the even mantissa (1)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], np.float32)
    np.testing.assert_array_equal(bf16_round(x), np.array([1.0, 1 + 2 ** -6, -1.0], np.float32))
    nan = bf16_bits(np.array([np.nan], np.float32))
    assert (int(nan[0]) & 0x7F80) == 0x7F80 and (int(nan[0]) & 0x7F) != 0


def _digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_generator_deterministic_and_per_sample():
    a = gen_attn(9, 2, 16, H=2, D=4)
    b = gen_attn(9, 2, 16, H=2, D=4)
    assert _digest(a.q, a.k, a.v, a.gq, a.gk) == _digest(b.q, b.k, b.v, b.gq, b.gk)
    assert not np.array_equal(a.q[0], a.q[1])  # independent stream per sample
    # a batch is the concatenation of its samples: sample 1 does not depend on B
    c = gen_attn(9, 3, 16, H=2, D=4)
    np.testing.assert_array_equal(a.k[1], c.k[1])


def test_bf16_values_are_exact():
    a = gen_attn(3, 1, 32, H=2, D=32, dtype="bf16")
    for t in (a.q, a.k, a.v):
        np.testing.assert_array_equal(bf16_round(t), t)
    x = torch.from_numpy(a.q).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(x, a.q)


def test_outlier_rows():
    N = 1000
    a = gen_attn(4, 1, N, H=1, D=32, dtype="f32", k_scale=30.0, outlier_frac=0.01)
    row_rms = np.sqrt(np.mean(a.k[0].astype(np.float64) ** 2, axis=1))
    big = row_rms > 600  # 30 * 100 = 3000 vs 30
    assert big.sum() == 10


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_config_shapes_small(cfg):
    c = CONFIGS[cfg]
    inp = gen_config(cfg, N=64)
    assert inp.q.shape == (c["B"], 64, 2240)
    assert inp.gq.shape == (2240,) and inp.gq.dtype == np.float32
    assert inp.dtype == c["dtype"]


def test_qkv_config_shapes_small():
    inp = gen_qkv(5, 2, 8)
    assert inp.x.shape == (2, 8, 2240) and inp.w.shape == (2240, 6720)
    np.testing.assert_array_equal(bf16_round(inp.w), inp.w)
    assert abs(float(inp.w.std()) - 0.02) < 1e-3


def test_cross_inputs_shapes_lengths_and_determinism():
    from synth import gen_cross
    a = gen_cross(21, 3, 40, L=50, H=4, ragged=True)
    b = gen_cross(21, 3, 40, L=50, H=4, ragged=True)
    assert a.q.shape == (3, 40, 128) and a.k.shape == (3, 50, 128) and a.v.shape == (3, 50, 128)
    assert a.kv_len.dtype == np.int32 and ((a.kv_len >= 1) & (a.kv_len <= 50)).all()
    assert all(np.array_equal(x, y) for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.kv_len, b.kv_len)))
    full = gen_cross(21, 2, 8, L=50, H=4)
    assert (full.kv_len == 50).all() and full.gq is not None
    assert gen_cross(21, 1, 8, L=5, H=4, norm=False).gq is None

"""Pins of the W8A8 oracle (no GPU needed).

The projection in 8-bit weights and activations: "Sana: Efficient High-Resolution Image Synthesis
with Linear Diffusion Transformers" (paper notes), section 7 "on-device deployment".  Pinned by a
hand-worked quantisation example (tests/golden/w8a8_quant_rows.txt), the rounding error bound of a
symmetric uniform quantiser, power-of-two scale invariance, exact integer brute force of the
projection, a closed-form bound against the unquantised fp64 projection, and the transposed weight
layout on a hand example.
"""
import os
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows():
    xs, qs, ss = [], [], []
    with open(os.path.join(GOLDEN, "w8a8_quant_rows.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "x":
                xs.append([float(v) for v in vals])
            elif key == "q":
                qs.append([int(v) for v in vals])
            elif key == "s":
                ss.append(np.array(int(vals[0], 16), dtype=np.uint32).view(np.float32))
    return np.array(xs, np.float32), np.array(qs, np.int8), np.array(ss, np.float32)


def test_golden_quant_rows_bit_exact():
    x, q_ref, s_ref = _golden_rows()
    q, s = oracle.quantize_rows(x)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))


def _bf16_rows(rng, rows, C, scale=1.0):
    x = (scale * rng.standard_normal((rows, C))).astype(np.float32)
    b = x.view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32).view(np.float32)


def test_quant_error_bound_and_extremes():
    """|x - q s| <= s/2 (up to the fp32 rounding of 127/amax), the largest |x| maps to +-127."""
    rng = np.random.default_rng(1)
    x = _bf16_rows(rng, 64, 2240, scale=3.0)
    x[5, 17] = 0.0
    q, s = oracle.quantize_rows(x)
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= 0.5 * s[:, None] * (1 + 1e-5) + 1e-30)
    amax_idx = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(q[np.arange(64), amax_idx].astype(int)) == 127)
    assert np.all(np.abs(q.astype(int)) <= 127)
    assert q[5, 17] == 0


def test_quant_power_of_two_invariance_and_row_independence():
    """Scaling a row by 2^k scales its s by 2^k and keeps its codes; other rows are untouched."""
    rng = np.random.default_rng(2)
    x = _bf16_rows(rng, 8, 448)
    q0, s0 = oracle.quantize_rows(x)
    y = x.copy()
    y[3] *= np.float32(2.0 ** 7)
    q1, s1 = oracle.quantize_rows(y)
    assert np.array_equal(q0, q1)
    assert s1[3] == s0[3] * np.float32(2.0 ** 7)
    assert np.array_equal(np.delete(s0, 3), np.delete(s1, 3))


def test_projection_exact_against_integer_brute_force():
    """w8a8_project = (sum_c xq*wq) * sx * sw with the integer sum exact (Python ints, Fractions)."""
    rng = np.random.default_rng(3)
    M, C, NO = 3, 64, 12
    xq = rng.integers(-127, 128, size=(M, C)).astype(np.int8)
    wq = rng.integers(-127, 128, size=(NO, C)).astype(np.int8)
    sx = rng.uniform(0.01, 0.1, size=M).astype(np.float32)
    sw = rng.uniform(0.001, 0.01, size=NO).astype(np.float32)
    got = oracle.w8a8_project(xq, sx, wq, sw)
    for m in range(M):
        for n in range(NO):
            acc = sum(int(xq[m, c]) * int(wq[n, c]) for c in range(C))
            exact = Fraction(acc) * Fraction(float(sx[m])) * Fraction(float(sw[n]))
            assert abs(Fraction(got[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def test_weight_quant_is_per_output_column_and_transposed():
    """W [C=2, 3] by hand: column n has amax a_n; row n of Wt_q holds that column's codes."""
    w = np.array([[1.0, -2.0, 0.5],
                  [-0.5, 1.0, 0.25]], np.float32)
    wt_q, sw = oracle.quantize_weight(w)
    assert wt_q.shape == (3, 2)
    assert np.array_equal(wt_q, np.array([[127, -64], [-127, 64], [127, 64]], np.int8))
    assert np.array_equal(sw, np.array([1.0, 2.0, 0.5], np.float32) / np.float32(127))


def test_w8a8_qkv_within_quantisation_bound_of_fp64_projection():
    """|xW - W8A8(x, W)| <= sum_c |x_c| dW + |W_c| dx + dx dW with dx = s_x/2, dW = s_w/2 per element."""
    rng = np.random.default_rng(4)
    M, C = 16, 320
    x = _bf16_rows(rng, M, C)
    w = (0.02 * rng.standard_normal((C, 3 * C))).astype(np.float32)
    wt_q, sw = oracle.quantize_weight(w)
    xq, sx = oracle.quantize_rows(x)
    got = oracle.w8a8_project(xq, sx, wt_q, sw)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    dx = 0.5 * sx.astype(np.float64)[:, None] * (1 + 1e-5)
    dw = 0.5 * sw.astype(np.float64)[None, :] * (1 + 1e-5)
    bound = (np.abs(x).astype(np.float64).sum(1, keepdims=True) * dw
             + dx * np.abs(w).astype(np.float64).sum(0, keepdims=True) + C * dx * dw)
    err = np.abs(got - ref)
    assert np.all(err <= bound)
    assert err.max() > 0  # the quantisation is not a no-op


def _identity_quant_case(seed, B, N, H, D):
    """x with integer entries in [-127, 127] and row maximum 127, so the per-token quantiser is exactly
    the identity (s_x = 127/127 = 1, codes = x).  Wt_q holds 64 * (a permutation matrix) in each of the
    q, k and v row blocks, with column scales 1/64, 2/64, 3/64 (powers of two times small integers, so
    every product below is exact in fp32 and fp64).  The W8A8 projection is then exactly
    q = x, k = 2 x[:, pk], v = 3 x[:, pv]."""
    rng = np.random.default_rng(seed)
    C = H * D
    x = rng.integers(-127, 128, size=(B, N, C)).astype(np.float32)
    rows = x.reshape(-1, C)
    at = rng.integers(0, C, size=rows.shape[0])
    rows[np.arange(rows.shape[0]), at] = np.where(rng.random(rows.shape[0]) < 0.5, 127.0, -127.0)
    perms = [np.arange(C), rng.permutation(C), rng.permutation(C)]
    wt_q = np.zeros((3 * C, C), np.int8)
    for blk, p in enumerate(perms):
        wt_q[blk * C + np.arange(C), p] = 64
    sw = np.concatenate([np.full(C, (blk + 1) / 64.0, np.float32) for blk in range(3)])
    return x, wt_q, sw, perms


def test_w8a8_composition_matches_linear_attn_of_exact_projection():
    """qkv_w8a8_linear_attn = linear_attn of the dequantised projection's q | k | v blocks, in that order
    (the Sana notes, section 7: W8A8 projection, linear attention in full precision).  With the
    identity quantisation above, the expected q, k, v are known in closed form; a k|v or q|k slice swap,
    raw x in place of the projection, or a projection left without its scales each move the output by
    far more than rounding."""
    H, D, eps = 2, 32, 1e-6
    x, wt_q, sw, (pq, pk, pv) = _identity_quant_case(5, 2, 7, H, D)
    xq, sx = oracle.quantize_rows(x)
    assert np.array_equal(xq.astype(np.float32), x) and np.all(sx == 1.0)
    rng = np.random.default_rng(6)
    C = H * D
    for gq, gk in ((1 + 0.1 * rng.standard_normal(C), 1 + 0.1 * rng.standard_normal(C)), (None, None)):
        gq = None if gq is None else gq.astype(np.float32)
        gk = None if gk is None else gk.astype(np.float32)
        got = oracle.qkv_w8a8_linear_attn(x, wt_q, sw, gq, gk, H, D, eps)
        q, k, v = x[..., pq], 2.0 * x[..., pk], 3.0 * x[..., pv]
        want = oracle.linear_attn(q, k, v, gq, gk, H, D, eps)
        assert np.max(np.abs(got - want)) <= 1e-14 * np.max(np.abs(want))
        scale = np.max(np.abs(want))
        wrong = {
            "k|v swapped": oracle.linear_attn(q, v, k, gq, gk, H, D, eps),
            "q|k swapped": oracle.linear_attn(k, q, v, gq, gk, H, D, eps),
            "raw x": oracle.linear_attn(x, x, x, gq, gk, H, D, eps),
            "no dequantisation": oracle.linear_attn(64 * q, 64 * x[..., pk], 64 * x[..., pv], gq, gk, H, D, eps),
        }
        for name, o in wrong.items():
            assert np.max(np.abs(o - got)) > 1e-3 * scale, name

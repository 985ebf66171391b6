"""Pins of the Mix-FFN oracle (no GPU needed).

Mix-FFN: "Sana: Efficient High-Resolution Image Synthesis with Linear Diffusion Transformers"
(paper notes), section 2.2 (inverted residual, 3x3 depthwise convolution, GLU) and section 2.3 (zero
padding of the 3x3 convolution); width 5600 at 2240 channels from the SANA 1.5 research notes.
Pinned by delta and shift kernels (identity, orientation and zero fill), SciPy's correlate2d per
channel, the closed forms of the GLU gate, and a pure-Python loop brute force of the whole FFN on a
tiny grid.
"""
import math

import numpy as np
import pytest
from scipy.signal import correlate2d

import oracle


def test_delta_kernel_is_identity():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((2, 12, 5))
    k = np.zeros((5, 3, 3))
    k[:, 1, 1] = 1.0
    assert np.array_equal(oracle.depthwise_conv3x3(h, k, 3, 4), h)


@pytest.mark.parametrize("p,q", [(0, 1), (2, 1), (1, 0), (1, 2), (0, 0), (2, 2)])
def test_shift_kernel_moves_the_grid_with_zero_fill(p, q):
    """A one-hot tap (p, q) reads h[i + p - 1, j + q - 1]: rows/columns past the edge read zeros."""
    rng = np.random.default_rng(2)
    Hg, Wg, Ch = 4, 5, 3
    h = rng.standard_normal((1, Hg * Wg, Ch))
    k = np.zeros((Ch, 3, 3))
    k[:, p, q] = 1.0
    out = oracle.depthwise_conv3x3(h, k, Hg, Wg).reshape(Hg, Wg, Ch)
    grid = h.reshape(Hg, Wg, Ch)
    for i in range(Hg):
        for j in range(Wg):
            si, sj = i + p - 1, j + q - 1
            want = grid[si, sj] if 0 <= si < Hg and 0 <= sj < Wg else np.zeros(Ch)
            assert np.array_equal(out[i, j], want)


def test_conv_matches_scipy_correlate2d_per_channel():
    rng = np.random.default_rng(3)
    B, Hg, Wg, Ch = 2, 6, 7, 4
    h = rng.standard_normal((B, Hg * Wg, Ch))
    k = rng.standard_normal((Ch, 3, 3))
    out = oracle.depthwise_conv3x3(h, k, Hg, Wg).reshape(B, Hg, Wg, Ch)
    for b in range(B):
        for c in range(Ch):
            ref = correlate2d(h[b, :, c].reshape(Hg, Wg), k[c], mode="same", boundary="fill", fillvalue=0.0)
            np.testing.assert_allclose(out[b, :, :, c], ref, rtol=1e-13, atol=1e-13)


def test_glu_closed_forms():
    a = np.array([2.0, -3.0, 0.5, 7.0])
    u = np.concatenate([a, [0.0, 0.0, 0.0, 0.0]])[None]
    np.testing.assert_allclose(oracle.glu(u, 4)[0], a / 2, rtol=0, atol=0)        # sigmoid(0) = 1/2
    big = np.concatenate([a, [40.0, 40.0, -40.0, -40.0]])[None]
    g = oracle.glu(big, 4)[0]
    np.testing.assert_allclose(g[:2], a[:2], rtol=1e-15)                           # open gate
    assert np.all(np.abs(g[2:]) < 1e-16 * np.abs(a[2:]) * 1e2)                     # closed gate
    rng = np.random.default_rng(4)
    av, bv = rng.standard_normal(9), rng.standard_normal(9)
    s = oracle.glu(np.concatenate([av, bv]), 9) + oracle.glu(np.concatenate([av, -bv]), 9)
    np.testing.assert_allclose(s, av, rtol=1e-14, atol=1e-15)                      # sigma(b) + sigma(-b) = 1


def test_mix_ffn_against_loop_brute_force():
    """Expansion, padded 3x3 depthwise correlation, value * sigmoid(gate), projection, as plain loops."""
    rng = np.random.default_rng(5)
    B, Hg, Wg, C, F = 1, 3, 3, 2, 3
    x = rng.standard_normal((B, Hg * Wg, C))
    w1 = rng.standard_normal((C, 2 * F))
    kdw = rng.standard_normal((2 * F, 3, 3))
    w2 = rng.standard_normal((F, C))
    y = oracle.mix_ffn(x, w1, kdw, w2, Hg, Wg)
    h = [[sum(x[0, n, c] * w1[c, e] for c in range(C)) for e in range(2 * F)] for n in range(Hg * Wg)]
    for i in range(Hg):
        for j in range(Wg):
            u = []
            for e in range(2 * F):
                acc = 0.0
                for p in range(3):
                    for q in range(3):
                        ii, jj = i + p - 1, j + q - 1
                        if 0 <= ii < Hg and 0 <= jj < Wg:
                            acc += kdw[e, p, q] * h[ii * Wg + jj][e]
                u.append(acc)
            g = [u[f] / (1.0 + math.exp(-u[F + f])) for f in range(F)]
            for c in range(C):
                want = sum(g[f] * w2[f, c] for f in range(F))
                assert abs(y[0, i * Wg + j, c] - want) <= 1e-12 * (1 + abs(want))

"""Oracle of Mix-FFN, the feed-forward half of SANA's Linear DiT block.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Sources (web pages, cited by title and section):
  [Sana]    "Sana: Efficient High-Resolution Image Synthesis with Linear
            Diffusion Transformers" (paper notes), section 2.2 "Mix-FFN": the
            MLP feed-forward is replaced by an inverted residual block, a 3x3
            depthwise convolution and a GLU, which adds the local aggregation
            that linear attention lacks; section 2.3 "NoPE": the 3x3
            convolution with zero padding carries the position information.
  [SANA1.5] "SANA 1.5: ..." (research notes), model architecture bullet on
            scale: 2240 channels per block and an FFN width of 5600.

Readings where the pages leave a step open:
  * Tokens form an Hg x Wg grid in raster order, token n = i * Wg + j (square
    latents: Hg = Wg = sqrt(N)).
  * The inverted residual block expands with a pointwise (1x1) projection
    x @ W1, W1 [C, 2F] for FFN width F, without bias or activation, so that
    the GLU after the convolution returns F channels.
  * The depthwise convolution is per channel over the grid, 3x3, stride 1,
    zero padding 1, no bias, in the cross-correlation form used by deep
    learning frameworks: u[i, j, c] = sum_{p, q in 0..2} kdw[c, p, q] *
    h[i + p - 1, j + q - 1, c], with h = 0 outside the grid.
  * GLU (the gated linear unit in its original form): the first F convolved
    channels are the values a, the last F the gates b, g = a * sigmoid(b).
  * A pointwise projection g @ W2, W2 [F, C], without bias, closes the FFN; the
    block's residual connection lies outside it.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def expand(x, w1) -> np.ndarray:
    """Pointwise expansion x [B, N, C] @ W1 [C, 2F] -> [B, N, 2F] (fp64, no rounding)."""
    return np.matmul(_f64(x), _f64(w1))


def depthwise_conv3x3(h, kdw, Hg: int, Wg: int) -> np.ndarray:
    """3x3 depthwise cross-correlation with zero padding over the Hg x Wg token grid.

    h: [B, N, Ch] with N = Hg * Wg; kdw: [Ch, 3, 3].  Returns [B, N, Ch].
    """
    h = _f64(h)
    B, N, Ch = h.shape
    assert N == Hg * Wg
    grid = h.reshape(B, Hg, Wg, Ch)
    pad = np.zeros((B, Hg + 2, Wg + 2, Ch))
    pad[:, 1:-1, 1:-1, :] = grid
    k = _f64(kdw)
    out = np.zeros_like(grid)
    for p in range(3):
        for q in range(3):
            out += k[:, p, q] * pad[:, p:p + Hg, q:q + Wg, :]
    return out.reshape(B, N, Ch)


def glu(u, F: int) -> np.ndarray:
    """g = a * sigmoid(b) with a = u[..., :F] and b = u[..., F:2F]."""
    u = _f64(u)
    a, b = u[..., :F], u[..., F:2 * F]
    return a / (1.0 + np.exp(-b))


def mix_ffn(x, w1, kdw, w2, Hg: int, Wg: int, return_parts: bool = False):
    """Expansion, depthwise 3x3 convolution, GLU, projection: [B, N, C] -> [B, N, C]."""
    F = _f64(w2).shape[0]
    h = expand(x, w1)
    u = depthwise_conv3x3(h, kdw, Hg, Wg)
    g = glu(u, F)
    y = np.matmul(g, _f64(w2))
    if return_parts:
        return y, dict(h=h, u=u, g=g)
    return y

"""Oracle of the W8A8 QKV projection: 8-bit weights and activations for deployment.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: [Sana] "Sana: Efficient High-Resolution Image Synthesis with Linear
Diffusion Transformers" (paper notes), section 7 "on-device deployment": the
model is deployed with INT8 weights and INT8 activations (W8A8), while the
normalisation layers, the linear attention and the cross-attention KV stay in
full precision.

Readings where the page names only "W8A8":
  * Symmetric int8 with codes in [-127, 127] and no zero point.
  * Activations are quantised per token (row of x) with a scale taken from the
    row itself at run time; weights per output column, offline.
  * Scale s = amax / 127, code q = clamp(round_half_even(x * (127 / amax)),
    -127, 127).  These decisions produce integers from floating point, so they
    are taken here in fp32, exactly as the device takes them (IEEE fp32
    division and product, both correctly rounded); an all-zero row gets s = 0
    and q = 0.
  * The integer products are summed exactly and the sum is dequantised with
    both scales; here that is done in fp64 (every partial sum is an integer
    below 2^53, so an fp64 matmul of the codes is exact).
"""
from __future__ import annotations

import numpy as np

from .linear_attn import linear_attn


def quantize_rows(x):
    """Per-row symmetric int8 codes and fp32 scales of x [..., C] (fp32 arithmetic, see the header)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    nz = amax > 0
    inv = np.zeros_like(amax)
    np.divide(np.float32(127.0), amax, out=inv, where=nz)
    prod = (x32 * inv[..., None]).astype(np.float32)  # one fp32 product per element
    q = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    s = np.zeros_like(amax)
    np.divide(amax, np.float32(127.0), out=s, where=nz)
    return q, s.astype(np.float32)


def quantize_weight(w):
    """W [C, 3C] -> (Wt_q [3C, C] int8, s_w [3C] fp32): the same rule per output column, stored
    transposed (row n holds the C input weights of output column n)."""
    return quantize_rows(np.asarray(w, dtype=np.float32).T)


def w8a8_project(xq, sx, wt_q, sw) -> np.ndarray:
    """sum_c xq[..., c] * wt_q[n, c], exact, times sx[...] * sw[n] in fp64.  Returns [..., 3C]."""
    acc = np.matmul(np.asarray(xq, dtype=np.float64), np.asarray(wt_q, dtype=np.float64).T)
    return acc * np.asarray(sx, dtype=np.float64)[..., None] * np.asarray(sw, dtype=np.float64)


def qkv_w8a8_linear_attn(x, wt_q, sw, gq, gk, H: int, D: int, eps: float, return_parts: bool = False):
    """Quantise x per token, W8A8 projection, then the full-precision linear attention on q | k | v."""
    C = H * D
    xq, sx = quantize_rows(x)
    qkv = w8a8_project(xq, sx, wt_q, sw)
    q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    res = linear_attn(q, k, v, gq, gk, H, D, eps, return_parts=return_parts)
    if not return_parts:
        return res
    o, parts = res
    parts.update(q=q, k=k, v=v, xq=xq, sx=sx)
    return o, parts

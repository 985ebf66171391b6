"""fp64 oracle: ReLU linear self-attention with RMSNorm on Q and K (QK-Norm).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Nothing here is
blocked, fused or reordered beyond what the definitions state; a library
matmul is the only primitive used for the contractions.

Sources (web pages, cited by title and section):
  [Sana]    "Sana: Efficient High-Resolution Image Synthesis with Linear
            Diffusion Transformers" (paper notes), section 2.1 "linear
            attention", Eq. (1), and the sentence after it on precomputing
            the sum of ReLU(K_j)^T V_j so each token costs O(D^2); section 7
            "on-device deployment" (QKV projection).
  [SANA1.5] "SANA 1.5: Efficient Scaling of Training-Time and Inference-Time
            Compute in Linear Diffusion Transformer" (research notes),
            section "model architecture", bullet "QK Norm": RMSNorm on the
            queries and keys of the linear self-attention.

Readings where the pages leave a step open:
  * RMSNorm spans all C = H*D channels of a token (before the head split),
    has a gain vector over C and no bias or mean subtraction; it is applied
    before ReLU: phi(x) = ReLU(x / sqrt(mean_c x_c^2 + eps) * g).
  * One eps serves both the RMSNorm and the attention denominator, where it
    is added after the dot product.  Eq. (1) itself has no eps.
  * Eq. (1) holds per head; head h owns channels [h*D, (h+1)*D).
  * The sum over j runs over all N tokens (non-causal); no 1/sqrt(D) scale;
    no positional encoding (the Sana notes' NoPE section).
  * With gains None the QK-Norm is off and phi(x) = ReLU(x) (SANA-1.0 style).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def rms_inverse(x, eps: float) -> np.ndarray:
    """[SANA1.5] QK Norm.  For every token row, 1 / sqrt(mean over ALL channels of x^2 + eps).

    x: [..., C]  ->  [...]
    """
    x = _f64(x)
    mean_sq = np.mean(x * x, axis=-1)
    return 1.0 / np.sqrt(mean_sq + eps)


def feature_map(x, g: Optional[np.ndarray], eps: float) -> np.ndarray:
    """phi(x) = ReLU(RMSNorm(x) * g); [SANA1.5] QK Norm feeding [Sana] Eq. (1)'s ReLU.

    g None: QK-Norm off, phi(x) = ReLU(x).
    """
    x = _f64(x)
    if g is None:
        return np.maximum(x, 0.0)
    r = rms_inverse(x, eps)
    return np.maximum(x * r[..., None] * _f64(g), 0.0)


def split_heads(x, H: int, D: int) -> np.ndarray:
    """[B, N, H*D] -> [B, N, H, D]; head h owns channels h*D .. h*D + D - 1."""
    x = _f64(x)
    B, N, C = x.shape
    if C != H * D:
        raise ValueError(f"channel count {C} != H*D = {H}*{D}")
    return x.reshape(B, N, H, D)


def kv_state(phik, v, H: int, D: int):
    """[Sana] Eq. (1), the sums over j, precomputed once as the sentence after Eq. (1) says:

    S[b, h] = sum_j phi(K_j,h)^T V_j,h   (D x D, row index = key dim, column = value dim)
    z[b, h] = sum_j phi(K_j,h)           (D)
    """
    pk = split_heads(phik, H, D)            # [B, N, H, D]
    vv = split_heads(v, H, D)               # [B, N, H, D]
    pk_t = np.transpose(pk, (0, 2, 3, 1))   # [B, H, D, N]
    vv_h = np.transpose(vv, (0, 2, 1, 3))   # [B, H, N, D]
    S = np.matmul(pk_t, vv_h)               # [B, H, D, D]
    z = pk.sum(axis=1)                      # [B, H, D]
    return S, z


def attend(phiq, S, z, eps: float, H: int, D: int) -> np.ndarray:
    """[Sana] Eq. (1) per token i and head h, with eps added to the denominator:

    O_i,h = phi(Q_i,h) S_h / (phi(Q_i,h) . z_h + eps)
    """
    pq = split_heads(phiq, H, D)            # [B, N, H, D]
    pq_h = np.transpose(pq, (0, 2, 1, 3))   # [B, H, N, D]
    num = np.matmul(pq_h, S)                # [B, H, N, D]
    den = np.matmul(pq_h, z[..., None])     # [B, H, N, 1]
    with np.errstate(invalid="ignore", divide="ignore"):
        o = num / (den + eps)               # eps = 0 with a zero row: 0/0, left undefined (NaN)
    B, _, N, _ = o.shape
    return np.transpose(o, (0, 2, 1, 3)).reshape(B, N, H * D)


def linear_attn(q, k, v, gq, gk, H: int, D: int, eps: float, return_parts: bool = False):
    """Whole path: QK-RMSNorm -> ReLU -> KV state -> output.  Inputs [B, N, H*D], gains [H*D]."""
    phiq = feature_map(q, gq, eps)
    phik = feature_map(k, gk, eps)
    S, z = kv_state(phik, v, H, D)
    o = attend(phiq, S, z, eps, H, D)
    if not return_parts:
        return o
    parts = dict(S=S, z=z, phiq=phiq, phik=phik)
    if gq is not None:
        parts["r_q"] = rms_inverse(q, eps)
        parts["r_k"] = rms_inverse(k, eps)
    return o, parts


def qkv_project(x, w) -> np.ndarray:
    """[Sana] section 7: the QKV projection x @ Wqkv, no bias, in fp64 without rounding.

    x: [B, N, C]; w: [C, 3C] with column blocks q | k | v.  Returns [B, N, 3C].
    """
    return np.matmul(_f64(x), _f64(w))


def qkv_linear_attn(x, w, gq, gk, H: int, D: int, eps: float, return_parts: bool = False):
    """QKV projection followed by the linear attention on the q | k | v column blocks."""
    C = H * D
    qkv = qkv_project(x, w)
    q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    res = linear_attn(q, k, v, gq, gk, H, D, eps, return_parts=return_parts)
    if not return_parts:
        return res
    o, parts = res
    parts.update(q=q, k=k, v=v)
    return o, parts

"""fp64 oracle: softmax cross-attention over text tokens with RMSNorm on Q and K (QK-Norm).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Nothing here is blocked, fused or reordered
beyond what the definitions state; a library matmul is the only primitive used for the contractions.

Source (web page, cited by title and section):
  [SANA1.5] "SANA 1.5: Efficient Scaling of Training-Time and Inference-Time Compute in Linear
            Diffusion Transformer" (research notes), section "model architecture": a Linear DiT block
            is ReLU linear self-attention, then vanilla cross-attention that injects the text
            condition, then Mix-FFN (bullet on the block's composition); RMSNorm is added on the
            queries and keys of both the linear self-attention and the cross-attention (bullet
            "QK Norm"); the text condition comes from a decoder-only language model's embeddings
            (bullets on the text encoder and on condition injection).

Readings where the page leaves a step open:
  * "Vanilla cross-attention" is multi-head scaled dot-product attention: per head,
    o_i = sum_j softmax_j(q_i . k_j / sqrt(D)) v_j, with the queries from the image tokens, keys and
    values from the text tokens, and the softmax over the text tokens of the same sample.
  * QK Norm as for the self-attention: RMSNorm over all C = H*D channels of a token with a gain vector
    over C and no bias, applied to q and to k before the head split and before the 1/sqrt(D) scale;
    v is not normalised.  With gains None the norm is off.
  * Prompts have different lengths: kv_len[b] (1 <= kv_len[b] <= L) text tokens of sample b take
    part, the others are padding and are left out of the softmax; kv_len None means all L.
  * Head h owns channels [h*D, (h+1)*D) of q, k and v alike.
  * The projections that produce q from the image tokens and k, v from the text embeddings, and the
    output projection, are outside this function, as for the self-attention.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .linear_attn import rms_inverse


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def rms_normalize(x, g, eps: float) -> np.ndarray:
    """[SANA1.5] QK Norm: x / sqrt(mean over all channels of x^2 + eps) * g, per token row."""
    x = _f64(x)
    return x * rms_inverse(x, eps)[..., None] * _f64(g)


def cross_attn(q, k, v, gq: Optional[np.ndarray], gk: Optional[np.ndarray], H: int, D: int = 32,
               eps: float = 1e-6, kv_len: Optional[Sequence[int]] = None) -> np.ndarray:
    """[SANA1.5] model architecture: the block's cross-attention with QK Norm.

    q: [B, N, C] image-token queries; k, v: [B, L, C] text-token keys and values; C = H * D.
    gq, gk: [C] RMSNorm gains (both None: the norm is off).  kv_len: [B] valid text tokens per sample.
    Returns o: [B, N, C] with o[b, i, head h] = sum_j softmax_j(qn_i . kn_j / sqrt(D)) v_j over the
    first kv_len[b] text tokens, qn and kn the normalised queries and keys.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, C = q.shape
    L = k.shape[1]
    assert C == H * D and k.shape == (B, L, C) and v.shape == (B, L, C)
    if (gq is None) != (gk is None):
        raise ValueError("gq and gk go together")
    if gq is not None:
        q = rms_normalize(q, gq, eps)
        k = rms_normalize(k, gk, eps)
    lens = [L] * B if kv_len is None else [int(x) for x in kv_len]
    if any(not 1 <= n <= L for n in lens):
        raise ValueError("every kv_len must lie in [1, L]")
    out = np.empty((B, N, C), dtype=np.float64)
    for b in range(B):
        n_kv = lens[b]
        for h in range(H):
            cols = slice(h * D, (h + 1) * D)
            logits = q[b, :, cols] @ k[b, :n_kv, cols].T / np.sqrt(D)  # [N, n_kv]
            # softmax over the text tokens; subtracting the row maximum leaves it unchanged
            w = np.exp(logits - logits.max(axis=1, keepdims=True))
            w /= w.sum(axis=1, keepdims=True)
            out[b, :, cols] = w @ v[b, :n_kv, cols]
    return out

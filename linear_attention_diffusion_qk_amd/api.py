"""Python binding of libsanala: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C-ABI (include/sanala.h).
torch is used for device memory and the current stream; nothing here computes.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import SanaError

_DTYPES = {torch.float32: _lib.SANA_F32, torch.bfloat16: _lib.SANA_BF16, torch.float16: _lib.SANA_F16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


# The current stream's raw handle without building a torch Stream object (that costs about 3 us a
# call, which is a sixth of a 1024-token call); the public route is the fallback.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream, like: Optional[torch.Tensor] = None) -> int:
    if stream is None:
        if _raw_current_stream is not None and like is not None and like.device.index is not None:
            return int(_raw_current_stream(like.device.index))
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check_dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libsanala takes device tensors")
        if not t.is_contiguous():
            raise ValueError("libsanala takes contiguous tensors")


def sana_linear_attn_fwd(q, k, v, gq, gk, B: int, N: int, H: int, D: int, eps: float, out,
                         stream=None, dtype: Optional[int] = None) -> None:
    """Same arguments as the C entry point; tensors stand in for the device pointers."""
    _check_dev(q, k, v, gq, gk, out)
    if dtype is None:
        dtype = _DTYPES[q.dtype]
    lib = _lib.load_library()
    st = lib.sana_linear_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gq), _ptr(gk), int(B), int(N), int(H), int(D),
                                  float(eps), _ptr(out), _stream_handle(stream, q), int(dtype))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_linear_attn_fwd")


def sana_qkv_linear_attn_fwd(x, Wqkv, gq, gk, B: int, N: int, H: int, D: int, eps: float, out,
                             stream=None) -> None:
    _check_dev(x, Wqkv, gq, gk, out)
    lib = _lib.load_library()
    st = lib.sana_qkv_linear_attn_fwd(_ptr(x), _ptr(Wqkv), _ptr(gq), _ptr(gk), int(B), int(N), int(H), int(D),
                                      float(eps), _ptr(out), _stream_handle(stream, x))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_qkv_linear_attn_fwd")


def sana_pack_weight_i8(Wt_q, rows: int, C: int, Wt_p, stream=None) -> None:
    _check_dev(Wt_q, Wt_p)
    lib = _lib.load_library()
    st = lib.sana_pack_weight_i8(_ptr(Wt_q), int(rows), int(C), _ptr(Wt_p), _stream_handle(stream, Wt_q))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_pack_weight_i8")


def sana_qkv_w8a8_linear_attn_fwd(x, Wt_p, w_scale, gq, gk, B: int, N: int, H: int, D: int, eps: float, out,
                                  stream=None) -> None:
    _check_dev(x, Wt_p, w_scale, gq, gk, out)
    lib = _lib.load_library()
    st = lib.sana_qkv_w8a8_linear_attn_fwd(_ptr(x), _ptr(Wt_p), _ptr(w_scale), _ptr(gq), _ptr(gk), int(B), int(N),
                                           int(H), int(D), float(eps), _ptr(out), _stream_handle(stream, x))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_qkv_w8a8_linear_attn_fwd")


def sana_quantize_rows_i8(x, rows: int, C: int, xq, x_scale, stream=None) -> None:
    _check_dev(x, xq, x_scale)
    lib = _lib.load_library()
    st = lib.sana_quantize_rows_i8(_ptr(x), int(rows), int(C), _ptr(xq), _ptr(x_scale), _stream_handle(stream, x))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_quantize_rows_i8")


def sana_mix_ffn_fwd(x, W1, Wdw, W2, B: int, Hg: int, Wg: int, C: int, F: int, out, stream=None) -> None:
    _check_dev(x, W1, Wdw, W2, out)
    lib = _lib.load_library()
    st = lib.sana_mix_ffn_fwd(_ptr(x), _ptr(W1), _ptr(Wdw), _ptr(W2), int(B), int(Hg), int(Wg), int(C), int(F),
                              _ptr(out), _stream_handle(stream, x))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_mix_ffn_fwd")


def linear_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gq: Optional[torch.Tensor],
                gk: Optional[torch.Tensor], H: int, D: int = 32, eps: float = 1e-6,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """O = phi(Q) S / (phi(Q).z + eps) for q, k, v of shape [B, N, H*D] (fp32, bf16 or binary16)."""
    if q.dim() != 3 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, N, H*D] shape")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be float32, all bfloat16 or all float16")
    B, N, C = q.shape
    if C != H * D:
        raise ValueError(f"last dim {C} != H*D = {H}*{D}")
    for g in (gq, gk):
        if g is not None and (g.dtype != torch.float32 or g.numel() != C):
            raise ValueError("gains must be float32 of length H*D")
    if out is None:
        out = torch.empty_like(q)
    sana_linear_attn_fwd(q, k, v, gq, gk, B, N, H, D, eps, out)
    return out


def qkv_linear_attn(x: torch.Tensor, Wqkv: torch.Tensor, gq: Optional[torch.Tensor], gk: Optional[torch.Tensor],
                    H: int, D: int = 32, eps: float = 1e-6, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [B, N, C] bf16, Wqkv [C, 3C] bf16 -> linear attention of x @ Wqkv's q | k | v blocks."""
    if x.dim() != 3 or x.dtype != torch.bfloat16 or Wqkv.dtype != torch.bfloat16:
        raise ValueError("x must be bf16 [B, N, C] and Wqkv bf16 [C, 3C]")
    B, N, C = x.shape
    if C != H * D or tuple(Wqkv.shape) != (C, 3 * C):
        raise ValueError("shape mismatch between x, Wqkv and H*D")
    if out is None:
        out = torch.empty_like(x)
    sana_qkv_linear_attn_fwd(x, Wqkv, gq, gk, B, N, H, D, eps, out)
    return out


def pack_weight_i8(Wt_q: torch.Tensor) -> torch.Tensor:
    """int8 Wt_q [rows, C] (C a multiple of 64) -> its K-blocked copy [C/64, rows, 64], the weight layout
    qkv_w8a8_linear_attn takes (packed once per weight)."""
    if Wt_q.dim() != 2 or Wt_q.dtype != torch.int8 or Wt_q.shape[1] % 64 != 0 or not Wt_q.is_contiguous():
        raise ValueError("Wt_q must be a contiguous int8 [rows, C] tensor with C a multiple of 64")
    rows, C = Wt_q.shape
    Wt_p = torch.empty((C // 64, rows, 64), dtype=torch.int8, device=Wt_q.device)
    sana_pack_weight_i8(Wt_q, rows, C, Wt_p)
    return Wt_p


def qkv_w8a8_linear_attn(x: torch.Tensor, Wt_p: torch.Tensor, w_scale: torch.Tensor, gq: Optional[torch.Tensor],
                         gk: Optional[torch.Tensor], H: int, D: int = 32, eps: float = 1e-6,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [B, N, C] bf16, Wt_p = pack_weight_i8(Wt_q) [C/64, 3C, 64] int8 (Wt_q [3C, C]: W transposed, quantised
    per output column), w_scale [3C] fp32 -> linear attention of the W8A8 projection's q | k | v blocks
    (x quantised per token inside)."""
    if x.dim() != 3 or x.dtype != torch.bfloat16 or Wt_p.dtype != torch.int8 or w_scale.dtype != torch.float32:
        raise ValueError("x must be bf16 [B, N, C], Wt_p int8 [C/64, 3C, 64] and w_scale float32 [3C]")
    B, N, C = x.shape
    if C != H * D or C % 64 != 0 or tuple(Wt_p.shape) != (C // 64, 3 * C, 64) or w_scale.numel() != 3 * C:
        raise ValueError("shape mismatch between x, Wt_p, w_scale and H*D")
    if out is None:
        out = torch.empty_like(x)
    sana_qkv_w8a8_linear_attn_fwd(x, Wt_p, w_scale, gq, gk, B, N, H, D, eps, out)
    return out


def mix_ffn(x: torch.Tensor, W1: torch.Tensor, Wdw: torch.Tensor, W2: torch.Tensor, Hg: int, Wg: int,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [B, Hg*Wg, C] bf16, W1 [C, 2F], Wdw [2F, 3, 3], W2 [F, C] (all bf16) -> Mix-FFN output [B, Hg*Wg, C]."""
    if x.dim() != 3 or any(t.dtype != torch.bfloat16 for t in (x, W1, Wdw, W2)):
        raise ValueError("x, W1, Wdw and W2 must be bf16")
    B, N, C = x.shape
    F = W2.shape[0]
    if N != Hg * Wg or tuple(W1.shape) != (C, 2 * F) or tuple(Wdw.shape) != (2 * F, 3, 3) or tuple(W2.shape) != (F, C):
        raise ValueError("shape mismatch between x, W1, Wdw, W2 and the grid")
    if out is None:
        out = torch.empty_like(x)
    sana_mix_ffn_fwd(x, W1, Wdw, W2, B, Hg, Wg, C, F, out)
    return out


def quantize_rows_i8(x: torch.Tensor):
    """bf16 [..., C] -> (int8 codes of the same shape, fp32 per-row scales [...]): the device quantiser."""
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    C = x.shape[-1]
    rows = x.numel() // C
    xq = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    sx = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    sana_quantize_rows_i8(x, rows, C, xq, sx)
    return xq, sx


def sana_timing_enable(enable: bool) -> None:
    """Time every kernel of later calls from this thread by its dispatch's start/stop events (measurement only)."""
    _lib.load_library().sana_timing_enable(1 if enable else 0)


def sana_timing_last(capacity: int = 32):
    """[(kernel name, ms)] of the most recent call on this thread, in launch order (waits for it)."""
    import ctypes
    lib = _lib.load_library()
    names = (ctypes.c_char_p * capacity)()
    ms = (ctypes.c_float * capacity)()
    n = lib.sana_timing_last(names, ms, capacity)
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, capacity))]

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
# call, which is a sixth of a 1024-token call).  The accessor is private to torch, so it is used on a
# device only after a first call has checked that it returns what the public route returns there; if
# it is missing, raises, or disagrees, the public route is used from then on.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_raw_agrees: dict = {}  # device index -> whether the private accessor matched the public one


def _raw_matches_public(dev: int) -> bool:
    if _raw_current_stream is None:
        return False
    try:
        return int(_raw_current_stream(dev)) == int(torch.cuda.current_stream(dev).cuda_stream)
    except Exception:  # noqa: BLE001 - any failure means: do not use it
        return False


def _stream_handle(stream, like: Optional[torch.Tensor] = None) -> int:
    if stream is None:
        if like is not None and like.device.index is not None:
            dev = like.device.index
            ok = _raw_agrees.get(dev)
            if ok is None:
                ok = _raw_agrees[dev] = _raw_matches_public(dev)
            if ok:
                return int(_raw_current_stream(dev))
        stream = torch.cuda.current_stream(like.device if like is not None and like.is_cuda else None)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


_NAMES_OF_DTYPE = {v: k for k, v in _DTYPES.items()}


def _need(specs, device_of=None):
    """Checks (name, tensor, numel, dtype) tuples before anything reaches the C-ABI: the kernels read and
    write exactly `numel` elements of `dtype` behind each pointer, so a short, mistyped, strided or
    foreign-device tensor would be read or written out of bounds.  Shape and dtype are checked first,
    then contiguity, then that every tensor is a device tensor on one device.  A tensor of None is
    skipped (optional gains)."""
    present = [(n, t, k, d) for n, t, k, d in specs if t is not None]
    for name, t, numel, dtype in present:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch.Tensor")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if t.numel() != numel:
            raise ValueError(f"{name} must hold {numel} elements, got {t.numel()} (shape {tuple(t.shape)})")
    for name, t, _, _ in present:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    ref = device_of if device_of is not None else (present[0][1] if present else None)
    for name, t, _, _ in present:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor (libsanala takes device pointers)")
        if ref is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _need_sizes(**sizes):
    for name, v in sizes.items():
        if int(v) < 1:
            raise ValueError(f"{name} must be >= 1, got {v}")


def _same_as(name, t, like):
    if not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(like.shape) or t.dtype != like.dtype:
        raise ValueError(f"{name} must be a {like.dtype} tensor of shape {tuple(like.shape)}")


def sana_linear_attn_fwd(q, k, v, gq, gk, B: int, N: int, H: int, D: int, eps: float, out,
                         stream=None, dtype: Optional[int] = None) -> None:
    """Same arguments as the C entry point; tensors stand in for the device pointers."""
    if dtype is None:
        if not isinstance(q, torch.Tensor) or q.dtype not in _DTYPES:
            raise ValueError("q must be a float32, bfloat16 or float16 tensor")
        dtype = _DTYPES[q.dtype]
    if int(dtype) not in _NAMES_OF_DTYPE:
        raise ValueError(f"unknown dtype code {dtype}")
    _need_sizes(B=B, N=N, H=H, D=D)
    tdt, n, C = _NAMES_OF_DTYPE[int(dtype)], int(B) * int(N) * int(H) * int(D), int(H) * int(D)
    _need([("q", q, n, tdt), ("k", k, n, tdt), ("v", v, n, tdt), ("out", out, n, tdt),
           ("gq", gq, C, torch.float32), ("gk", gk, C, torch.float32)])
    lib = _lib.load_library()
    st = lib.sana_linear_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gq), _ptr(gk), int(B), int(N), int(H), int(D),
                                  float(eps), _ptr(out), _stream_handle(stream, q), int(dtype))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_linear_attn_fwd")


def sana_linear_attn_fwd_noalloc(q, k, v, gq, gk, B: int, N: int, H: int, D: int, eps: float, out,
                                 stream=None, dtype: Optional[int] = None) -> None:
    """sana_linear_attn_fwd on the library's static per-device scratch: the call allocates no device memory."""
    if dtype is None:
        if not isinstance(q, torch.Tensor) or q.dtype not in _DTYPES:
            raise ValueError("q must be a float32, bfloat16 or float16 tensor")
        dtype = _DTYPES[q.dtype]
    if int(dtype) not in _NAMES_OF_DTYPE:
        raise ValueError(f"unknown dtype code {dtype}")
    _need_sizes(B=B, N=N, H=H, D=D)
    tdt, n, C = _NAMES_OF_DTYPE[int(dtype)], int(B) * int(N) * int(H) * int(D), int(H) * int(D)
    _need([("q", q, n, tdt), ("k", k, n, tdt), ("v", v, n, tdt), ("out", out, n, tdt),
           ("gq", gq, C, torch.float32), ("gk", gk, C, torch.float32)])
    lib = _lib.load_library()
    st = lib.sana_linear_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(gq), _ptr(gk), int(B), int(N), int(H),
                                          int(D), float(eps), _ptr(out), _stream_handle(stream, q), int(dtype))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_linear_attn_fwd_noalloc")


def sana_qkv_linear_attn_fwd(x, Wqkv, gq, gk, B: int, N: int, H: int, D: int, eps: float, out,
                             stream=None) -> None:
    _need_sizes(B=B, N=N, H=H, D=D)
    C = int(H) * int(D)
    n = int(B) * int(N) * C
    bf = torch.bfloat16
    _need([("x", x, n, bf), ("Wqkv", Wqkv, C * 3 * C, bf), ("out", out, n, bf), ("gq", gq, C, torch.float32),
           ("gk", gk, C, torch.float32)])
    lib = _lib.load_library()
    st = lib.sana_qkv_linear_attn_fwd(_ptr(x), _ptr(Wqkv), _ptr(gq), _ptr(gk), int(B), int(N), int(H), int(D),
                                      float(eps), _ptr(out), _stream_handle(stream, x))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_qkv_linear_attn_fwd")


def sana_pack_weight_i8(Wt_q, rows: int, C: int, Wt_p, stream=None) -> None:
    _need_sizes(rows=rows, C=C)
    _need([("Wt_q", Wt_q, int(rows) * int(C), torch.int8), ("Wt_p", Wt_p, int(rows) * int(C), torch.int8)])
    lib = _lib.load_library()
    st = lib.sana_pack_weight_i8(_ptr(Wt_q), int(rows), int(C), _ptr(Wt_p), _stream_handle(stream, Wt_q))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_pack_weight_i8")


def sana_qkv_w8a8_linear_attn_fwd(x, Wt_p, w_scale, gq, gk, B: int, N: int, H: int, D: int, eps: float, out,
                                  stream=None) -> None:
    _need_sizes(B=B, N=N, H=H, D=D)
    C = int(H) * int(D)
    n = int(B) * int(N) * C
    bf = torch.bfloat16
    _need([("x", x, n, bf), ("Wt_p", Wt_p, 3 * C * C, torch.int8), ("w_scale", w_scale, 3 * C, torch.float32),
           ("out", out, n, bf), ("gq", gq, C, torch.float32), ("gk", gk, C, torch.float32)])
    lib = _lib.load_library()
    st = lib.sana_qkv_w8a8_linear_attn_fwd(_ptr(x), _ptr(Wt_p), _ptr(w_scale), _ptr(gq), _ptr(gk), int(B), int(N),
                                           int(H), int(D), float(eps), _ptr(out), _stream_handle(stream, x))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_qkv_w8a8_linear_attn_fwd")


def sana_quantize_rows_i8(x, rows: int, C: int, xq, x_scale, stream=None) -> None:
    _need_sizes(rows=rows, C=C)
    _need([("x", x, int(rows) * int(C), torch.bfloat16), ("xq", xq, int(rows) * int(C), torch.int8),
           ("x_scale", x_scale, int(rows), torch.float32)])
    lib = _lib.load_library()
    st = lib.sana_quantize_rows_i8(_ptr(x), int(rows), int(C), _ptr(xq), _ptr(x_scale), _stream_handle(stream, x))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_quantize_rows_i8")


def sana_mix_ffn_fwd(x, W1, Wdw, W2, B: int, Hg: int, Wg: int, C: int, F: int, out, stream=None) -> None:
    _need_sizes(B=B, Hg=Hg, Wg=Wg, C=C, F=F)
    n = int(B) * int(Hg) * int(Wg) * int(C)
    bf = torch.bfloat16
    _need([("x", x, n, bf), ("W1", W1, int(C) * 2 * int(F), bf), ("Wdw", Wdw, 2 * int(F) * 9, bf),
           ("W2", W2, int(F) * int(C), bf), ("out", out, n, bf)])
    lib = _lib.load_library()
    st = lib.sana_mix_ffn_fwd(_ptr(x), _ptr(W1), _ptr(Wdw), _ptr(W2), int(B), int(Hg), int(Wg), int(C), int(F),
                              _ptr(out), _stream_handle(stream, x))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_mix_ffn_fwd")


def sana_cross_attn_fwd(q, k, v, gq, gk, kv_len, B: int, N: int, L: int, H: int, D: int, eps: float, out,
                        stream=None, dtype: Optional[int] = None) -> None:
    """Same arguments as the C entry point; tensors stand in for the device pointers (kv_len: an int32
    device tensor of B lengths, or None)."""
    if dtype is None:
        dtype = _lib.SANA_BF16
    _need_sizes(B=B, N=N, L=L, H=H, D=D)
    nq, nk, C = int(B) * int(N) * int(H) * int(D), int(B) * int(L) * int(H) * int(D), int(H) * int(D)
    tdt = _NAMES_OF_DTYPE.get(int(dtype), torch.bfloat16)
    _need([("q", q, nq, tdt), ("k", k, nk, tdt), ("v", v, nk, tdt), ("out", out, nq, tdt),
           ("gq", gq, C, torch.float32), ("gk", gk, C, torch.float32), ("kv_len", kv_len, int(B), torch.int32)])
    lib = _lib.load_library()
    st = lib.sana_cross_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gq), _ptr(gk), _ptr(kv_len), int(B), int(N), int(L),
                                 int(H), int(D), float(eps), _ptr(out), _stream_handle(stream, q), int(dtype))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_cross_attn_fwd")


def sana_release_scratch(stream=None) -> None:
    """Frees the library's scratch buffer of `stream` (default: the current stream) on the current device,
    stream-ordered; call it before destroying a stream the library has used."""
    st = _lib.load_library().sana_release_scratch(_stream_handle(stream))
    if st != _lib.SANA_OK:
        raise SanaError(st, "sana_release_scratch")


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
    _same_as("out", out, q)
    sana_linear_attn_fwd(q, k, v, gq, gk, B, N, H, D, eps, out)
    return out


def cross_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gq: Optional[torch.Tensor],
               gk: Optional[torch.Tensor], H: int, D: int = 32, eps: float = 1e-6,
               kv_len: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Softmax cross-attention with QK-Norm: q [B, N, H*D] image tokens, k, v [B, L, H*D] text tokens,
    all bfloat16; kv_len: int32 [B] valid text tokens per sample (None: all L)."""
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2]:
        raise ValueError("q must be [B, N, C] and k, v [B, L, C] with the same B and C")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must be bfloat16")
    B, N, C = q.shape
    L = k.shape[1]
    if C != H * D:
        raise ValueError(f"last dim {C} != H*D = {H}*{D}")
    if out is None:
        out = torch.empty_like(q)
    _same_as("out", out, q)
    sana_cross_attn_fwd(q, k, v, gq, gk, kv_len, B, N, L, H, D, eps, out)
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
    _same_as("out", out, x)
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
    _same_as("out", out, x)
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
    _same_as("out", out, x)
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

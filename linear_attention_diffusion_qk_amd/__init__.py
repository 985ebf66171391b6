"""libsanala: ReLU linear self-attention with QK-RMSNorm (SANA's Linear DiT block) on MI355X.

The compute lives in hand-written HIP kernels for gfx950 behind a C-ABI (include/sanala.h);
this package only loads that library and marshals torch tensors into it.
"""
from ._lib import EXPORTS, SanaError, library_path, load_library, status_string  # noqa: F401
from .api import (  # noqa: F401
    cross_attn,
    linear_attn,
    mix_ffn,
    pack_weight_i8,
    qkv_linear_attn,
    qkv_w8a8_linear_attn,
    quantize_rows_i8,
    sana_cross_attn_fwd,
    sana_linear_attn_fwd,
    sana_linear_attn_fwd_noalloc,
    sana_mix_ffn_fwd,
    sana_pack_weight_i8,
    sana_qkv_linear_attn_fwd,
    sana_qkv_w8a8_linear_attn_fwd,
    sana_quantize_rows_i8,
    sana_release_scratch,
    sana_timing_enable,
    sana_timing_last,
)

"""The C-ABI library loads without a GPU, exports every declared symbol, and rejects bad arguments on
the host before any HIP call (no compute is launched here)."""
import ctypes
import os
import re

import pytest

import linear_attention_diffusion_qk_amd as sanala

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "sanala.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sana_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert _declared_symbols() == sorted(sanala.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = sanala.load_library()
    for name in _declared_symbols():
        assert hasattr(lib, name), name
    # the binding exposes the same names
    for name in ("sana_linear_attn_fwd", "sana_qkv_linear_attn_fwd"):
        assert callable(getattr(sanala, name))


def test_status_strings():
    for s in range(5):
        assert sanala.status_string(s)
    assert sanala.status_string(99) == "unknown status"


# fake, 16-byte aligned "device" addresses: every call below must be rejected before it is used
A, B_, C_, G1, G2, O = 0x1000, 0x2000000, 0x4000000, 0x6000000, 0x6001000, 0x8000000


@pytest.mark.parametrize("args,status", [
    ((0, B_, C_, G1, G2, 1, 8, 70, 32, 1e-6, O, 0, 1), 1),           # null q
    ((A, B_, C_, G1, 0, 1, 8, 70, 32, 1e-6, O, 0, 1), 1),             # only one gain NULL
    ((A, B_, C_, G1, G2, 0, 8, 70, 32, 1e-6, O, 0, 1), 1),            # B = 0
    ((A, B_, C_, G1, G2, 1, -3, 70, 32, 1e-6, O, 0, 1), 1),           # N < 0
    ((A, B_, C_, G1, G2, 1, 8, 70, 32, float("nan"), O, 0, 1), 1),    # eps NaN
    ((A, B_, C_, G1, G2, 1, 8, 70, 32, -1.0, O, 0, 1), 1),            # eps < 0
    ((A, B_, C_, G1, G2, 1, 8, 70, 32, 1e-6, O, 0, 7), 1),            # unknown dtype
    ((A, B_, C_, G1, G2, 1, 8, 140, 16, 1e-6, O, 0, 1), 2),           # D != 32
    ((A, B_, C_, G1, G2, 1, 8, 400, 32, 1e-6, O, 0, 1), 2),           # H too large
    ((A, B_, C_, G1, G2, 70000, 8, 70, 32, 1e-6, O, 0, 1), 2),        # B too large
    ((A + 2, B_, C_, G1, G2, 1, 8, 70, 32, 1e-6, O, 0, 1), 3),        # misaligned q
    ((A, B_, C_, G1 + 4, G2, 1, 8, 70, 32, 1e-6, O, 0, 1), 3),        # misaligned gain
    ((A, B_, C_, G1, G2, 1, 8, 70, 32, 1e-6, A + 16, 0, 1), 1),       # out overlaps q
])
def test_linear_attn_rejects(args, status):
    lib = sanala.load_library()
    assert lib.sana_linear_attn_fwd(*args) == status


@pytest.mark.parametrize("args,status", [
    ((0, B_, G1, G2, 1, 8, 70, 32, 1e-6, O, 0), 1),
    ((A, B_, G1, 0, 1, 8, 70, 32, 1e-6, O, 0), 1),
    ((A, B_, G1, G2, 1, 8, 70, 30, 1e-6, O, 0), 2),
    ((A, B_ + 8, G1, G2, 1, 8, 70, 32, 1e-6, O, 0), 3),
    ((A, B_, G1, G2, 1, 8, 70, 32, 1e-6, B_ + 64, 0), 1),            # out overlaps W
])
def test_qkv_rejects(args, status):
    lib = sanala.load_library()
    assert lib.sana_qkv_linear_attn_fwd(*args) == status


S_ = 0xA000000  # fake w_scale address


@pytest.mark.parametrize("args,status", [
    ((0, B_, S_, G1, G2, 1, 8, 70, 32, 1e-6, O, 0), 1),              # null x
    ((A, B_, 0, G1, G2, 1, 8, 70, 32, 1e-6, O, 0), 1),               # null w_scale
    ((A, B_, S_, G1, 0, 1, 8, 70, 32, 1e-6, O, 0), 1),               # one gain NULL
    ((A, B_, S_, G1, G2, 1, 8, 3, 32, 1e-6, O, 0), 2),               # C = 96 not a multiple of 64
    ((A, B_, S_ + 4, G1, G2, 1, 8, 70, 32, 1e-6, O, 0), 3),          # misaligned w_scale
    ((A, B_, S_, G1, G2, 1, 8, 70, 32, 1e-6, B_ + 64, 0), 1),        # out overlaps Wt_p
])
def test_w8a8_rejects(args, status):
    lib = sanala.load_library()
    assert lib.sana_qkv_w8a8_linear_attn_fwd(*args) == status


@pytest.mark.parametrize("args,status", [
    ((0, 4, 64, B_, S_, 0), 1),                                       # null x
    ((A, 0, 64, B_, S_, 0), 1),                                       # no rows
    ((A, 4, 60, B_, S_, 0), 2),                                       # C not a multiple of 8
    ((A + 8, 4, 64, B_, S_, 0), 3),                                   # misaligned x
    ((A, 4, 64, A + 32, S_, 0), 1),                                   # xq overlaps x
])
def test_quantize_rows_rejects(args, status):
    lib = sanala.load_library()
    assert lib.sana_quantize_rows_i8(*args) == status


@pytest.mark.parametrize("args,status", [
    ((0, 4, 64, B_, 0), 1),                                           # null Wt_q
    ((A, 0, 64, B_, 0), 1),                                           # no rows
    ((A, 4, 96, B_, 0), 2),                                           # C not a multiple of 64
    ((A, (1 << 30) + 1, 64, B_, 0), 2),                               # too many rows
    ((A, 1 << 30, 1 << 11, B_, 0), 2),                                # rows * C > 2^40
    ((A + 8, 4, 64, B_, 0), 3),                                       # misaligned Wt_q
    ((A, 4, 64, A + 64, 0), 1),                                       # Wt_p overlaps Wt_q
])
def test_pack_weight_rejects(args, status):
    lib = sanala.load_library()
    assert lib.sana_pack_weight_i8(*args) == status


@pytest.mark.parametrize("args,status", [
    ((0, B_, C_, G1, 1, 8, 8, 2240, 5600, O, 0), 1),                 # null x
    ((A, B_, C_, G1, 0, 8, 8, 2240, 5600, O, 0), 1),                 # B = 0
    ((A, B_, C_, G1, 1, 8, 8, 2240, 5000, O, 0), 2),                 # F not a multiple of 32
    ((A, B_, C_, G1, 1, 8, 200, 2240, 5600, O, 0), 2),               # Wg > 128
    ((A + 2, B_, C_, G1, 1, 8, 8, 2240, 5600, O, 0), 3),             # misaligned x
    ((A, B_, C_, G1, 1, 8, 8, 2240, 5600, A + 64, 0), 1),            # out overlaps x
])
def test_mix_ffn_rejects(args, status):
    lib = sanala.load_library()
    assert lib.sana_mix_ffn_fwd(*args) == status


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from linear_attention_diffusion_qk_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.load_library()

"""The Python binding rejects tensors the kernels would read or write out of bounds (wrong element
count, dtype, layout or device) with ValueError before it touches the C-ABI.  Host only: every call
below fails in the checks, so nothing is launched and no GPU is needed."""
import pytest
import torch

import linear_attention_diffusion_qk_amd as sanala

B, N, H, D = 1, 8, 2, 32
C = H * D


def _attn(dtype=torch.bfloat16, **over):
    t = dict(q=torch.zeros(B, N, C, dtype=dtype), k=torch.zeros(B, N, C, dtype=dtype),
             v=torch.zeros(B, N, C, dtype=dtype), gq=torch.ones(C), gk=torch.ones(C),
             out=torch.zeros(B, N, C, dtype=dtype))
    t.update(over)
    return t


@pytest.mark.parametrize("over,match", [
    (dict(out=torch.zeros(B, N, C, dtype=torch.float32)), "out must be torch.bfloat16"),   # 2x past the end
    (dict(out=torch.zeros(B, N, C // 2, dtype=torch.bfloat16)), "out must hold"),
    (dict(v=torch.zeros(B, N - 1, C, dtype=torch.bfloat16)), "v must hold"),
    (dict(gq=torch.ones(C, dtype=torch.bfloat16)), "gq must be torch.float32"),
    (dict(gk=torch.ones(C - 1)), "gk must hold"),
    (dict(k=torch.zeros(B, C, N, dtype=torch.bfloat16).transpose(1, 2)), "k must be contiguous"),
    (dict(), "must be a device tensor"),                                                   # host tensors
])
def test_low_level_attention_checks(over, match):
    t = _attn(**over)
    with pytest.raises(ValueError, match=match):
        sanala.sana_linear_attn_fwd(t["q"], t["k"], t["v"], t["gq"], t["gk"], B, N, H, D, 1e-6, t["out"])


def test_low_level_attention_checks_sizes_and_dtype_code():
    t = _attn()
    with pytest.raises(ValueError, match="N must be >= 1"):
        sanala.sana_linear_attn_fwd(t["q"], t["k"], t["v"], t["gq"], t["gk"], B, 0, H, D, 1e-6, t["out"])
    with pytest.raises(ValueError, match="unknown dtype"):
        sanala.sana_linear_attn_fwd(t["q"], t["k"], t["v"], t["gq"], t["gk"], B, N, H, D, 1e-6, t["out"], dtype=9)
    # dtype code f32 with bf16 tensors: the kernels would read twice the bytes
    with pytest.raises(ValueError, match="q must be torch.float32"):
        sanala.sana_linear_attn_fwd(t["q"], t["k"], t["v"], t["gq"], t["gk"], B, N, H, D, 1e-6, t["out"], dtype=0)


@pytest.mark.parametrize("out,match", [
    (torch.zeros(B, N, C, dtype=torch.float32), "out must be a torch.bfloat16 tensor"),
    (torch.zeros(B, N * C, dtype=torch.bfloat16), "out must be a torch.bfloat16 tensor of shape"),
])
def test_high_level_out_checks(out, match):
    t = _attn()
    with pytest.raises(ValueError, match=match):
        sanala.linear_attn(t["q"], t["k"], t["v"], t["gq"], t["gk"], H, D, out=out)
    x = torch.zeros(B, N, C, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=match):
        sanala.qkv_linear_attn(x, torch.zeros(C, 3 * C, dtype=torch.bfloat16), t["gq"], t["gk"], H, D, out=out)


def test_fused_front_end_checks():
    x = torch.zeros(B, N, C, dtype=torch.bfloat16)
    w = torch.zeros(C, 3 * C, dtype=torch.bfloat16)
    out = torch.zeros_like(x)
    with pytest.raises(ValueError, match="gq must be torch.float32"):
        sanala.sana_qkv_linear_attn_fwd(x, w, torch.ones(C, dtype=torch.float16), torch.ones(C), B, N, H, D, 1e-6, out)
    with pytest.raises(ValueError, match="Wqkv must hold"):
        sanala.sana_qkv_linear_attn_fwd(x, w[:, :C], torch.ones(C), torch.ones(C), B, N, H, D, 1e-6, out)
    wt = torch.zeros(C // 64, 3 * C, 64, dtype=torch.int8)
    with pytest.raises(ValueError, match="w_scale must hold"):
        sanala.sana_qkv_w8a8_linear_attn_fwd(x, wt, torch.ones(C), None, None, B, N, H, D, 1e-6, out)
    with pytest.raises(ValueError, match="out must be torch.bfloat16"):
        sanala.sana_qkv_w8a8_linear_attn_fwd(x, wt, torch.ones(3 * C), None, None, B, N, H, D, 1e-6, out.float())


def test_quantiser_pack_and_mix_ffn_checks():
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="x_scale must hold"):
        sanala.sana_quantize_rows_i8(x, 4, 64, torch.zeros(4, 64, dtype=torch.int8), torch.zeros(3))
    with pytest.raises(ValueError, match="Wt_p must hold"):
        sanala.sana_pack_weight_i8(torch.zeros(4, 64, dtype=torch.int8), 4, 64, torch.zeros(4, 32, dtype=torch.int8))
    F = 64
    xm = torch.zeros(1, 4, C, dtype=torch.bfloat16)
    args = [xm, torch.zeros(C, 2 * F, dtype=torch.bfloat16), torch.zeros(2 * F, 3, 3, dtype=torch.bfloat16),
            torch.zeros(F, C, dtype=torch.bfloat16)]
    with pytest.raises(ValueError, match="Wdw must hold"):
        sanala.sana_mix_ffn_fwd(args[0], args[1], args[2][:F], args[3], 1, 2, 2, C, F, torch.zeros_like(xm))
    with pytest.raises(ValueError, match="out must hold"):
        sanala.sana_mix_ffn_fwd(*args, 1, 2, 2, C, F, torch.zeros(1, 3, C, dtype=torch.bfloat16))


def test_private_stream_accessor_is_not_trusted_when_it_fails(monkeypatch):
    """The binding uses torch's private current-stream accessor only after it agreed with the public
    route; a missing or failing accessor means the public route."""
    from linear_attention_diffusion_qk_amd import api

    def broken(dev):
        raise RuntimeError("no such accessor")

    monkeypatch.setattr(api, "_raw_current_stream", broken)
    assert api._raw_matches_public(0) is False
    monkeypatch.setattr(api, "_raw_current_stream", None)
    assert api._raw_matches_public(0) is False

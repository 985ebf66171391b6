"""Seeded synthetic inputs shaped like SANA's latent-token workloads.

This package only draws random numbers and rounds them to the storage type.
It holds none of the attention arithmetic, so both the fp64 oracle side and
the GPU side can take their inputs from it without sharing any computation.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    AttnInputs,
    CrossInputs,
    MixFfnInputs,
    QkvInputs,
    W8A8Inputs,
    bf16_round,
    bf16_bits,
    gen_attn,
    gen_config,
    gen_cross,
    gen_mix_ffn,
    gen_qkv,
    gen_w8a8,
)

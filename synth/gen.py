"""Seeded input generators for the ReLU linear self-attention workloads.

Shapes follow the SANA pages: the latent token count is (pixels/32)^2 from the
32x deep-compression autoencoder (SANA notes page, section 1 "Deep Compression
Autoencoder", token-count table; SANA-1.5 notes page, architecture section),
and one Linear DiT layer has 2240 channels (SANA-1.5 notes page, architecture
section, scale/resolution bullet), split here as 70 heads of 32.

Every tensor is drawn in float64 from NumPy's PCG64 stream seeded with
SeedSequence([config_id, sample, tensor_id]), cast to float32, and for bf16
storage rounded to the nearest bf16 value (ties to even); for binary16 storage
("f16") rounded to the nearest IEEE half value.  The arrays returned
are float32 whose values are exactly representable in the storage type, so the
GPU side can convert them without further rounding and the oracle can widen
them to float64 exactly.

Tensor ids: q=0, k=1, v=2, gq=3, gk=4, x=5, Wqkv=6, outlier rows=7, int8 weight codes=8,
weight column scales=9, Mix-FFN W1=10, depthwise taps=11, W2=12, text-token keys=13, text-token
values=14, text lengths=15.

Cross-attention inputs stand in for the text encoder's projected embeddings (no encoder is run): the
text-token keys and values are N(0,1) like the image-token queries, with up to 300 text tokens per
sample (SANA's prompt length) and, for ragged batches, a seeded length per sample.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

(TID_Q, TID_K, TID_V, TID_GQ, TID_GK, TID_X, TID_W, TID_OUTLIER, TID_WCODE, TID_WSCALE, TID_W1, TID_KDW,
 TID_W2, TID_TK, TID_TV, TID_TLEN) = range(16)

C_SANA = 2240
H_SANA = 70
D_SANA = 32
EPS_SANA = 1e-6


def _rng(cfg_id: int, sample: int, tid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, sample, tid])))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of x rounded to bf16, round-to-nearest-even; NaN stays NaN (quieted)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    b = x32.view(np.uint32)
    # for every non-NaN pattern b + 0x8000 stays below 2^32, so uint32 arithmetic cannot wrap
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        r[nan] = ((b[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array holding x rounded to the nearest bf16 value (ties to even)."""
    bits = bf16_bits(x).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == "bf16":
        return bf16_round(x32)
    if dtype == "f32":
        return x32
    if dtype == "f16":
        return x32.astype(np.float16).astype(np.float32)  # IEEE binary16, round to nearest even
    raise ValueError(f"unknown storage dtype {dtype!r}")


@dataclass
class AttnInputs:
    """q, k, v: float32 [B, N, H*D]; gq, gk: float32 [H*D]; values exact in `dtype`."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    gq: Optional[np.ndarray]
    gk: Optional[np.ndarray]
    H: int
    D: int
    eps: float
    dtype: str
    name: str = ""

    @property
    def B(self) -> int:
        return self.q.shape[0]

    @property
    def N(self) -> int:
        return self.q.shape[1]


@dataclass
class QkvInputs:
    """x: float32 [B, N, C]; w: float32 [C, 3C] (q | k | v column blocks); values exact in bf16."""
    x: np.ndarray
    w: np.ndarray
    gq: np.ndarray
    gk: np.ndarray
    H: int
    D: int
    eps: float
    dtype: str = "bf16"
    name: str = ""

    @property
    def B(self) -> int:
        return self.x.shape[0]

    @property
    def N(self) -> int:
        return self.x.shape[1]


@dataclass
class W8A8Inputs:
    """x: float32 [B, N, C] exact in bf16; wt_q: int8 [3C, C] (row n = the C weight codes of output
    column n); s_w: float32 [3C] column scales; the effective weight is s_w[n] * wt_q[n, c]."""
    x: np.ndarray
    wt_q: np.ndarray
    s_w: np.ndarray
    gq: Optional[np.ndarray]
    gk: Optional[np.ndarray]
    H: int
    D: int
    eps: float
    name: str = ""

    @property
    def B(self) -> int:
        return self.x.shape[0]

    @property
    def N(self) -> int:
        return self.x.shape[1]


def gains(cfg_id: int, C: int, which: int) -> np.ndarray:
    """RMSNorm gains over all C channels: 1 + 0.1*N(0,1), float32, shared by the batch."""
    return (1.0 + 0.1 * _rng(cfg_id, 0, which).standard_normal(C)).astype(np.float32)


def gen_attn(cfg_id: int, B: int, N: int, H: int = H_SANA, D: int = D_SANA, dtype: str = "bf16",
             eps: float = EPS_SANA, k_scale: float = 1.0, outlier_frac: float = 0.0,
             outlier_mult: float = 100.0, v_shift: float = 0.0, norm: bool = True,
             name: str = "") -> AttnInputs:
    """Q, V ~ N(0,1) (+ v_shift), K ~ k_scale*N(0,1) with floor(outlier_frac*N) seeded rows
    of every sample multiplied by outlier_mult; independent stream per sample."""
    C = H * D
    qs, ks, vs = [], [], []
    for b in range(B):
        q = _rng(cfg_id, b, TID_Q).standard_normal((N, C))
        k = k_scale * _rng(cfg_id, b, TID_K).standard_normal((N, C))
        n_out = int(np.floor(outlier_frac * N))
        if n_out > 0:
            rows = _rng(cfg_id, b, TID_OUTLIER).choice(N, size=n_out, replace=False)
            k[rows, :] *= outlier_mult
        v = _rng(cfg_id, b, TID_V).standard_normal((N, C)) + v_shift
        qs.append(_store(q, dtype))
        ks.append(_store(k, dtype))
        vs.append(_store(v, dtype))
    gq = gains(cfg_id, C, TID_GQ) if norm else None
    gk = gains(cfg_id, C, TID_GK) if norm else None
    return AttnInputs(np.stack(qs), np.stack(ks), np.stack(vs), gq, gk, H, D, eps, dtype, name)


def gen_qkv(cfg_id: int, B: int, N: int, H: int = H_SANA, D: int = D_SANA, eps: float = EPS_SANA,
            w_std: float = 0.02, name: str = "") -> QkvInputs:
    """x ~ N(0,1) [B, N, C] and Wqkv ~ N(0, w_std^2) [C, 3C], both bf16."""
    C = H * D
    xs = [_store(_rng(cfg_id, b, TID_X).standard_normal((N, C)), "bf16") for b in range(B)]
    w = _store(w_std * _rng(cfg_id, 0, TID_W).standard_normal((C, 3 * C)), "bf16")
    return QkvInputs(np.stack(xs), w, gains(cfg_id, C, TID_GQ), gains(cfg_id, C, TID_GK), H, D, eps,
                     "bf16", name)


def gen_w8a8(cfg_id: int, B: int, N: int, H: int = H_SANA, D: int = D_SANA, eps: float = EPS_SANA,
             w_std: float = 0.02, norm: bool = True, name: str = "") -> W8A8Inputs:
    """x ~ N(0,1) bf16 [B, N, C]; int8 weight codes drawn directly as integers, N(0, (127/4)^2)
    rounded and limited to [-127, 127], with column scales w_std * 4/127 * U(0.75, 1.25), so that the
    effective weight has about the spread of an N(0, w_std^2) Wqkv."""
    C = H * D
    xs = [_store(_rng(cfg_id, b, TID_X).standard_normal((N, C)), "bf16") for b in range(B)]
    codes = np.rint(_rng(cfg_id, 0, TID_WCODE).standard_normal((3 * C, C)) * (127.0 / 4.0))
    wt_q = np.clip(codes, -127, 127).astype(np.int8)
    s_w = (w_std * 4.0 / 127.0 * _rng(cfg_id, 0, TID_WSCALE).uniform(0.75, 1.25, 3 * C)).astype(np.float32)
    gq = gains(cfg_id, C, TID_GQ) if norm else None
    gk = gains(cfg_id, C, TID_GK) if norm else None
    return W8A8Inputs(np.stack(xs), wt_q, s_w, gq, gk, H, D, eps, name)


@dataclass
class MixFfnInputs:
    """x: float32 [B, Hg*Wg, C]; w1 [C, 2F]; kdw [2F, 3, 3]; w2 [F, C]; all values exact in bf16."""
    x: np.ndarray
    w1: np.ndarray
    kdw: np.ndarray
    w2: np.ndarray
    Hg: int
    Wg: int
    name: str = ""

    @property
    def B(self) -> int:
        return self.x.shape[0]

    @property
    def F(self) -> int:
        return self.w2.shape[0]


def gen_mix_ffn(cfg_id: int, B: int, Hg: int, Wg: int, C: int = C_SANA, F: int = 5600, w_std: float = 0.02,
                name: str = "") -> MixFfnInputs:
    """x ~ N(0,1); W1, W2 ~ N(0, w_std^2); depthwise taps ~ N(0, 1/9); all rounded to bf16."""
    N = Hg * Wg
    xs = [_store(_rng(cfg_id, b, TID_X).standard_normal((N, C)), "bf16") for b in range(B)]
    w1 = _store(w_std * _rng(cfg_id, 0, TID_W1).standard_normal((C, 2 * F)), "bf16")
    kdw = _store(_rng(cfg_id, 0, TID_KDW).standard_normal((2 * F, 3, 3)) / 3.0, "bf16")
    w2 = _store(w_std * _rng(cfg_id, 0, TID_W2).standard_normal((F, C)), "bf16")
    return MixFfnInputs(np.stack(xs), w1, kdw, w2, Hg, Wg, name)


@dataclass
class CrossInputs:
    q: np.ndarray            # [B, N, C] image-token queries
    k: np.ndarray            # [B, L, C] text-token keys
    v: np.ndarray            # [B, L, C] text-token values
    gq: Optional[np.ndarray]
    gk: Optional[np.ndarray]
    kv_len: np.ndarray       # [B] int32, valid text tokens per sample (1..L)
    H: int
    D: int
    eps: float
    dtype: str
    name: str = ""

    @property
    def B(self) -> int:
        return self.q.shape[0]

    @property
    def N(self) -> int:
        return self.q.shape[1]

    @property
    def L(self) -> int:
        return self.k.shape[1]


def gen_cross(cfg_id: int, B: int, N: int, L: int = 300, H: int = H_SANA, D: int = D_SANA, dtype: str = "bf16",
              eps: float = EPS_SANA, norm: bool = True, ragged: bool = False, k_scale: float = 1.0,
              name: str = "") -> CrossInputs:
    """Queries ~ N(0,1) over N image tokens; text keys ~ k_scale*N(0,1) and values ~ N(0,1) over L text
    tokens; with `ragged`, sample b has a seeded length in [1, L], else all L tokens are valid."""
    C = H * D
    qs, ks, vs, lens = [], [], [], []
    for b in range(B):
        qs.append(_store(_rng(cfg_id, b, TID_Q).standard_normal((N, C)), dtype))
        ks.append(_store(k_scale * _rng(cfg_id, b, TID_TK).standard_normal((L, C)), dtype))
        vs.append(_store(_rng(cfg_id, b, TID_TV).standard_normal((L, C)), dtype))
        lens.append(int(_rng(cfg_id, b, TID_TLEN).integers(1, L + 1)) if ragged else L)
    gq = gains(cfg_id, C, TID_GQ) if norm else None
    gk = gains(cfg_id, C, TID_GK) if norm else None
    return CrossInputs(np.stack(qs), np.stack(ks), np.stack(vs), gq, gk, np.asarray(lens, np.int32), H, D, eps,
                       dtype, name)


# The five SANA-shaped workloads (C = 2240 = 70 heads x 32).
CONFIGS = {
    1: dict(kind="attn", B=1, N=256, dtype="f32",
            desc="512px single layer, fp32 I/O, B=1, N=256"),
    2: dict(kind="attn", B=1, N=1024, dtype="bf16",
            desc="1024px, bf16 I/O, B=1, N=1024"),
    3: dict(kind="attn", B=32, N=1024, dtype="bf16",
            desc="1024px repeat-sampling batch, bf16 I/O, B=32, N=1024"),
    4: dict(kind="attn", B=1, N=16384, dtype="bf16", k_scale=30.0, outlier_frac=0.01,
            outlier_mult=100.0, desc="4K, bf16 I/O, B=1, N=16384, K ~ N(0,30^2) with 1% rows x100"),
    5: dict(kind="qkv", B=4, N=4096, dtype="bf16",
            desc="2K fused front end: x[4,4096,2240] bf16, Wqkv[2240,6720] ~ N(0,0.02^2)"),
}


def gen_config(cfg_id: int, B: Optional[int] = None, N: Optional[int] = None):
    """Inputs of workload `cfg_id`; B and N may be overridden (smaller parity cases)."""
    c = dict(CONFIGS[cfg_id])
    B = c["B"] if B is None else B
    N = c["N"] if N is None else N
    name = f"config{cfg_id}"
    if c["kind"] == "qkv":
        return gen_qkv(cfg_id, B, N, name=name)
    return gen_attn(cfg_id, B, N, dtype=c["dtype"], k_scale=c.get("k_scale", 1.0),
                    outlier_frac=c.get("outlier_frac", 0.0), outlier_mult=c.get("outlier_mult", 100.0),
                    name=name)

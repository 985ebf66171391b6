"""Pins of the fp64 oracle against things other than itself (no GPU needed).

Each test names what the pages or the mathematics fix:
  * hand-worked examples with exact rational answers (tests/golden/);
  * the quadratic (un-factorized) form of Eq. (1) -- sum_j (phi(q_i).phi(k_j)) v_j /
    (sum_j phi(q_i).phi(k_j) + eps) -- by exact rationals, by 40-digit decimals and by
    dense fp64 on tiny inputs;
  * closed forms (N = 1; D = H = 1), invariants (linearity in V, constant shift, hull,
    token permutation, batch independence, positive scaling of phi), zero rows;
  * RMSNorm properties that tell the readings apart (whole-row axis, gain after the
    norm, eps inside the square root, mean rather than sum).
The method: "Sana: Efficient High-Resolution Image Synthesis with Linear Diffusion
Transformers" (paper notes) section 2.1, Eq. (1); QK-Norm: "SANA 1.5: Efficient Scaling of
Training-Time and Inference-Time Compute in Linear Diffusion Transformer" (research notes),
model architecture, QK Norm bullet.
"""
import decimal
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers
def _parse_golden(name):
    rows = {"q": [], "k": [], "v": [], "o": []}
    meta = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key in rows:
                rows[key].append([Fraction(x) for x in vals])
            elif key in ("gq", "gk"):
                meta[key] = [Fraction(x) for x in vals]
            else:
                meta[key] = Fraction(vals[0])
    return meta, rows


def _exact_sqrt(x: Fraction) -> Fraction:
    n, d = x.numerator, x.denominator
    rn, rd = math.isqrt(n), math.isqrt(d)
    assert rn * rn == n and rd * rd == d, f"{x} is not a rational square"
    return Fraction(rn, rd)


def _quadratic_exact(meta, rows):
    """Quadratic form of Eq. (1) in exact rationals (pure Python loops)."""
    H, D, eps = int(meta["H"]), int(meta["D"]), meta["eps"]
    C = H * D

    def phi(x, g):
        ms = sum(v * v for v in x) / C
        r = 1 / _exact_sqrt(ms + eps)
        return [max(Fraction(0), x[c] * r * g[c]) for c in range(C)]

    pq = [phi(x, meta["gq"]) for x in rows["q"]]
    pk = [phi(x, meta["gk"]) for x in rows["k"]]
    out = []
    for i in range(len(pq)):
        orow = []
        for h in range(H):
            sl = slice(h * D, (h + 1) * D)
            a = [sum(x * y for x, y in zip(pq[i][sl], pk[j][sl])) for j in range(len(pk))]
            den = sum(a) + eps
            for e in range(D):
                num = sum(a[j] * rows["v"][j][h * D + e] for j in range(len(pk)))
                orow.append(num / den if den != 0 else Fraction(0))
        out.append(orow)
    return out


def _rand_inputs(seed, B, N, H, D, dtype=np.float64):
    rng = np.random.default_rng(seed)
    C = H * D
    q = rng.standard_normal((B, N, C))
    k = rng.standard_normal((B, N, C))
    v = rng.standard_normal((B, N, C))
    gq = 1 + 0.1 * rng.standard_normal(C)
    gk = 1 + 0.1 * rng.standard_normal(C)
    return q, k, v, gq, gk


def _quadratic_numpy(q, k, v, gq, gk, H, D, eps):
    """Dense O(N^2) form per head: A = phi(Q) phi(K)^T, O = A V / (A 1 + eps)."""
    pq = oracle.feature_map(q, gq, eps)
    pk = oracle.feature_map(k, gk, eps)
    B, N, C = q.shape
    o = np.zeros((B, N, C))
    for b in range(B):
        for h in range(H):
            sl = slice(h * D, (h + 1) * D)
            A = pq[b, :, sl] @ pk[b, :, sl].T
            o[b, :, sl] = (A @ v[b, :, sl]) / (A.sum(axis=1, keepdims=True) + eps)
    return o


# ----------------------------------------------------------------------------- golden
@pytest.mark.parametrize("name", ["worked_example_eps0.txt", "worked_example_eps3.txt"])
def test_golden_worked_example(name):
    meta, rows = _parse_golden(name)
    # the fixture's hand derivation agrees with the exact rational quadratic form
    exact = _quadratic_exact(meta, rows)
    assert exact == rows["o"], (exact, rows["o"])
    H, D, eps = int(meta["H"]), int(meta["D"]), float(meta["eps"])
    f = lambda rs: np.array([[float(x) for x in r] for r in rs])[None]  # noqa: E731
    o = oracle.linear_attn(f(rows["q"]), f(rows["k"]), f(rows["v"]),
                           np.array([float(x) for x in meta["gq"]]),
                           np.array([float(x) for x in meta["gk"]]), H, D, eps)
    np.testing.assert_allclose(o[0], f(rows["o"])[0], rtol=1e-14, atol=1e-15)


# ----------------------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed,B,N,H,D", [(1, 1, 1, 1, 1), (2, 2, 5, 2, 3), (3, 1, 7, 3, 2), (4, 2, 4, 1, 4)])
def test_quadratic_form_40_digits(seed, B, N, H, D):
    """Oracle vs a 40-significant-digit pure-Python quadratic form, eps = 1e-6 (irrational roots)."""
    eps = 1e-6
    q, k, v, gq, gk = _rand_inputs(seed, B, N, H, D)
    o = oracle.linear_attn(q, k, v, gq, gk, H, D, eps)
    ctx = decimal.Context(prec=40)
    Dm = lambda x: decimal.Decimal(float(x))  # noqa: E731  (exact conversion of the double)
    C = H * D
    E = Dm(eps)

    def phi(row, g):
        ms = ctx.divide(sum((ctx.multiply(Dm(x), Dm(x)) for x in row), decimal.Decimal(0)), C)
        r = ctx.divide(1, ctx.sqrt(ctx.add(ms, E)))
        return [max(decimal.Decimal(0), ctx.multiply(ctx.multiply(Dm(row[c]), r), Dm(g[c]))) for c in range(C)]

    for b in range(B):
        pq = [phi(q[b, i], gq) for i in range(N)]
        pk = [phi(k[b, j], gk) for j in range(N)]
        for i in range(N):
            for h in range(H):
                sl = range(h * D, (h + 1) * D)
                a = [sum((ctx.multiply(pq[i][c], pk[j][c]) for c in sl), decimal.Decimal(0)) for j in range(N)]
                den = ctx.add(sum(a, decimal.Decimal(0)), E)
                for e in range(D):
                    num = sum((ctx.multiply(a[j], Dm(v[b, j, h * D + e])) for j in range(N)), decimal.Decimal(0))
                    want = float(ctx.divide(num, den))
                    assert abs(o[b, i, h * D + e] - want) <= 1e-13 * max(1.0, abs(want))


@pytest.mark.parametrize("N", [1, 2, 3, 17, 40])
@pytest.mark.parametrize("H,D", [(1, 1), (2, 4), (3, 8)])
def test_quadratic_form_dense(N, H, D):
    eps = 1e-6
    q, k, v, gq, gk = _rand_inputs(100 + N * 7 + H, 2, N, H, D)
    o = oracle.linear_attn(q, k, v, gq, gk, H, D, eps)
    np.testing.assert_allclose(o, _quadratic_numpy(q, k, v, gq, gk, H, D, eps), rtol=1e-12, atol=1e-13)


def test_quadratic_form_sana_shape():
    """Full SANA head layout (70 x 32) at small N, where the quadratic form is cheap."""
    H, D, eps = 70, 32, 1e-6
    q, k, v, gq, gk = _rand_inputs(7, 1, 48, H, D)
    o = oracle.linear_attn(q, k, v, gq, gk, H, D, eps)
    np.testing.assert_allclose(o, _quadratic_numpy(q, k, v, gq, gk, H, D, eps), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- closed forms
def test_single_token_closed_form():
    """N = 1: O = v * a / (a + eps) with a = phi(q).phi(k) per head."""
    H, D = 3, 4
    for eps in (1e-6, 0.5):
        q, k, v, gq, gk = _rand_inputs(11, 2, 1, H, D)
        o = oracle.linear_attn(q, k, v, gq, gk, H, D, eps)
        pq = oracle.feature_map(q, gq, eps).reshape(2, 1, H, D)
        pk = oracle.feature_map(k, gk, eps).reshape(2, 1, H, D)
        a = (pq * pk).sum(-1, keepdims=True)
        want = (v.reshape(2, 1, H, D) * a / (a + eps)).reshape(2, 1, H * D)
        np.testing.assert_allclose(o, want, rtol=1e-13, atol=1e-15)


def test_one_channel_weighted_mean():
    """D = H = 1: phi(q_i) factors out, so O_i = phi_q,i * sum_j phi_k,j v_j / (phi_q,i * sum_j phi_k,j + eps)."""
    rng = np.random.default_rng(5)
    N, eps = 9, 0.25
    q = np.abs(rng.standard_normal((1, N, 1))) + 0.5
    k = rng.standard_normal((1, N, 1))
    v = rng.standard_normal((1, N, 1))
    g = np.array([1.3])
    o = oracle.linear_attn(q, k, v, g, g, 1, 1, eps)
    # one channel: RMSNorm maps x to x / sqrt(x^2 + eps), so phi = g * x / sqrt(x^2 + eps) for x > 0
    pq = np.maximum(g * q[0, :, 0] / np.sqrt(q[0, :, 0] ** 2 + eps), 0)
    pk = np.maximum(g * k[0, :, 0] / np.sqrt(k[0, :, 0] ** 2 + eps), 0)
    want = pq * (pk @ v[0, :, 0]) / (pq * pk.sum() + eps)
    np.testing.assert_allclose(o[0, :, 0], want, rtol=1e-13)


# ----------------------------------------------------------------------------- invariants
def test_linear_in_v():
    H, D, eps = 2, 8, 1e-6
    q, k, v1, gq, gk = _rand_inputs(21, 2, 30, H, D)
    v2 = np.random.default_rng(22).standard_normal(v1.shape)
    a, b = 1.7, -0.3
    o = oracle.linear_attn(q, k, a * v1 + b * v2, gq, gk, H, D, eps)
    want = a * oracle.linear_attn(q, k, v1, gq, gk, H, D, eps) + b * oracle.linear_attn(q, k, v2, gq, gk, H, D, eps)
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-13)


def test_constant_shift_of_v():
    """Adding a vector c to every V row adds c * (phi_q.z) / (phi_q.z + eps)."""
    H, D, eps = 2, 4, 0.1
    q, k, v, gq, gk = _rand_inputs(23, 1, 12, H, D)
    c = np.random.default_rng(24).standard_normal(H * D)
    o0, parts = oracle.linear_attn(q, k, v, gq, gk, H, D, eps, return_parts=True)
    o1 = oracle.linear_attn(q, k, v + c, gq, gk, H, D, eps)
    pq = parts["phiq"].reshape(1, 12, H, D)
    den = np.einsum("bnhd,bhd->bnh", pq, parts["z"])
    frac = np.repeat(den / (den + eps), D, axis=-1)
    np.testing.assert_allclose(o1 - o0, c * frac, rtol=1e-11, atol=1e-12)


def test_hull_of_v():
    """Per head and channel, O lies in [min(0, min_j v), max(0, max_j v)] (a shrunken weighted mean)."""
    H, D, eps = 3, 8, 1e-6
    q, k, v, gq, gk = _rand_inputs(25, 2, 64, H, D)
    o = oracle.linear_attn(q, k, v, gq, gk, H, D, eps)
    lo = np.minimum(0, v.min(axis=1, keepdims=True))
    hi = np.maximum(0, v.max(axis=1, keepdims=True))
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


def test_token_permutations_and_batch_independence():
    H, D, eps = 2, 4, 1e-6
    q, k, v, gq, gk = _rand_inputs(26, 3, 20, H, D)
    o = oracle.linear_attn(q, k, v, gq, gk, H, D, eps)
    perm = np.random.default_rng(27).permutation(20)
    # joint K/V permutation leaves O unchanged
    np.testing.assert_allclose(oracle.linear_attn(q, k[:, perm], v[:, perm], gq, gk, H, D, eps), o, rtol=1e-13, atol=1e-14)
    # a Q permutation permutes O
    np.testing.assert_allclose(oracle.linear_attn(q[:, perm], k, v, gq, gk, H, D, eps), o[:, perm], rtol=1e-13, atol=1e-14)
    # changing sample 1 does not move samples 0 and 2
    k2 = k.copy()
    k2[1] = -k2[1]
    o2 = oracle.linear_attn(q, k2, v, gq, gk, H, D, eps)
    np.testing.assert_array_equal(o2[[0, 2]], o[[0, 2]])
    assert not np.allclose(o2[1], o[1])


def test_positive_scaling_of_phi():
    """phi_q -> s phi_q or phi_k -> s phi_k changes O only through eps (relative O(eps/den))."""
    H, D, eps = 2, 8, 1e-6
    q, k, v, gq, gk = _rand_inputs(28, 1, 50, H, D)
    o, parts = oracle.linear_attn(q, k, v, gq, gk, H, D, eps, return_parts=True)
    den = np.einsum("bnhd,bhd->bnh", parts["phiq"].reshape(1, 50, H, D), parts["z"])
    for s in (0.125, 3.0, 40.0):
        # scaling the gain scales phi (the gain is applied after the norm); the ratio moves by
        # at most eps * |1 - 1/s| / den relative
        live = np.repeat(den > 0, D, axis=-1)            # den = 0 rows are 0 both ways
        bound = np.repeat(eps * abs(1 - 1 / s) / np.where(den > 0, den, 1.0), D, axis=-1) * 1.01 + 1e-13
        for o_s in (oracle.linear_attn(q, k, v, s * gq, gk, H, D, eps),
                    oracle.linear_attn(q, k, v, gq, s * gk, H, D, eps)):
            assert np.all(o_s[~live] == 0.0) and np.all(o[~live] == 0.0)
            assert np.all(np.abs(o_s - o)[live] <= (bound * np.abs(o))[live] + 1e-15)
    # with eps = 0 the invariance is exact up to rounding
    o0 = oracle.linear_attn(q, k, v, gq, gk, H, D, 0.0)
    np.testing.assert_allclose(oracle.linear_attn(q, k, v, 5 * gq, 0.2 * gk, H, D, 0.0), o0, rtol=1e-12, atol=1e-14)


def test_zero_feature_rows_give_zero():
    H, D, eps = 2, 4, 1e-6
    q, k, v, gq, gk = _rand_inputs(29, 1, 10, H, D)
    q[0, 3] = -np.abs(q[0, 3])          # every phi(q) entry of token 3 is 0 (gains are positive)
    o = oracle.linear_attn(q, k, v, gq, gk, H, D, eps)
    assert np.all(o[0, 3] == 0.0)
    # all-negative K: S = 0 and z = 0, so O = 0 everywhere through eps
    o2 = oracle.linear_attn(q, -np.abs(k), v, gq, gk, H, D, eps)
    assert np.all(o2 == 0.0)


# ----------------------------------------------------------------------------- RMSNorm readings
def test_rmsnorm_properties():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((4, 6, 24)) * 3
    eps = 1e-3
    r = oracle.rms_inverse(x, eps)
    ms = np.mean(x * x, axis=-1)
    # with unit gains the normalised row has mean square ms / (ms + eps): pins mean (not sum),
    # the square root and eps inside it
    np.testing.assert_allclose(np.mean((x * r[..., None]) ** 2, axis=-1), ms / (ms + eps), rtol=1e-13)
    # textbook value: [3, 4] has mean square 12.5
    assert oracle.rms_inverse(np.array([3.0, 4.0]), 0.0) == pytest.approx(1 / math.sqrt(12.5), rel=1e-15)
    # scale invariance at eps = 0
    np.testing.assert_allclose(oracle.rms_inverse(7 * x, 0.0), oracle.rms_inverse(x, 0.0) / 7, rtol=1e-14)


def test_rmsnorm_spans_all_heads():
    """Whole-row norm keeps a 10:1 ratio between heads; a per-head norm would erase it."""
    H, D = 2, 4
    rng = np.random.default_rng(32)
    base = np.abs(rng.standard_normal(D)) + 0.1
    x = np.concatenate([10 * base, base])[None, None, :]
    g = np.ones(H * D)
    phi = oracle.feature_map(x, g, 0.0)[0, 0]
    np.testing.assert_allclose(phi[:D], 10 * phi[D:], rtol=1e-14)


def test_gain_applied_after_norm_and_before_relu():
    rng = np.random.default_rng(33)
    x = rng.standard_normal((1, 5, 12))
    g = np.abs(rng.standard_normal(12)) + 0.5
    # uniform gain c scales phi by c (RMSNorm(c x) = RMSNorm(x) would not)
    np.testing.assert_allclose(oracle.feature_map(x, 3 * np.ones(12), 0.0),
                               3 * oracle.feature_map(x, np.ones(12), 0.0), rtol=1e-14)
    # a negative gain flips which entries survive the ReLU
    phi_neg = oracle.feature_map(x, -g, 0.0)
    assert np.all((phi_neg > 0) == (x < 0))
    # the norm uses the signed entries, not only the positive ones
    r = 1 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
    np.testing.assert_allclose(oracle.feature_map(x, g, 0.0), np.maximum(x, 0) * r * g, rtol=1e-14)


def test_norm_off_is_plain_relu():
    rng = np.random.default_rng(34)
    x = rng.standard_normal((2, 3, 8))
    np.testing.assert_array_equal(oracle.feature_map(x, None, 1e-6), np.where(x > 0, x, 0.0))


def test_head_channel_blocks():
    """Head h owns channels [h*D, (h+1)*D): zeroing one head's K removes only that head's output."""
    H, D, eps = 3, 4, 1e-6
    q, k, v, gq, gk = _rand_inputs(35, 1, 8, H, D)
    k2 = k.copy()
    k2[..., D:2 * D] = -np.abs(k2[..., D:2 * D]) - 1.0  # head 1 keys all negative -> phi = 0
    o = oracle.linear_attn(q, k2, v, gq, gk, H, D, eps)
    assert np.all(o[..., D:2 * D] == 0.0)
    assert np.count_nonzero(o[..., :D]) > o[..., :D].size // 2
    assert np.count_nonzero(o[..., 2 * D:]) > o[..., 2 * D:].size // 2


# ----------------------------------------------------------------------------- QKV projection
def test_qkv_projection_triple_loop():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((2, 3, 4))
    w = rng.standard_normal((4, 12))
    got = oracle.qkv_project(x, w)
    want = np.zeros((2, 3, 12))
    for b in range(2):
        for n in range(3):
            for j in range(12):
                want[b, n, j] = sum(x[b, n, c] * w[c, j] for c in range(4))
    np.testing.assert_allclose(got, want, rtol=1e-14)


def test_qkv_column_blocks():
    """W = [I | 2I | 3I] gives q = x, k = 2x, v = 3x."""
    H, D, eps = 2, 3, 1e-6
    C = H * D
    rng = np.random.default_rng(42)
    x = rng.standard_normal((1, 7, C))
    w = np.concatenate([np.eye(C), 2 * np.eye(C), 3 * np.eye(C)], axis=1)
    gq = 1 + 0.1 * rng.standard_normal(C)
    gk = 1 + 0.1 * rng.standard_normal(C)
    o = oracle.qkv_linear_attn(x, w, gq, gk, H, D, eps)
    np.testing.assert_allclose(o, oracle.linear_attn(x, 2 * x, 3 * x, gq, gk, H, D, eps), rtol=1e-14)


# ----------------------------------------------------------------------------- fp16 range
def test_denominator_leaves_fp16_range_at_4k():
    """The SANA-1.5 notes warn that linear-attention values leave the FP16 range.  With QK-Norm on,
    N(0,1) data and N = 16384 tokens, phi(q).z is already above 65504 (binary16's largest finite
    value), so the state and the denominator must be accumulated in fp32."""
    H, D, N, eps = 1, 32, 16384, 1e-6
    rng = np.random.default_rng(43)
    q = rng.standard_normal((1, N, H * D))
    k = rng.standard_normal((1, N, H * D))
    g = np.ones(H * D)
    pq = oracle.feature_map(q, g, eps)
    S, z = oracle.kv_state(oracle.feature_map(k, g, eps), rng.standard_normal((1, N, H * D)), H, D)
    den = pq[0] @ z[0, 0]
    assert np.median(den) > 65504.0


def test_fp16_accumulated_state_overflows_without_norm():
    """The SANA notes report FP16 overflow (NaN) in linear attention without QK-Norm.  With the 4K
    workload's keys (sd 30, 1% of rows x100) and the norm off, z = sum_j ReLU(k_j) reaches ~4.6e5: a
    running sum kept in binary16 overflows to inf and the output of Eq. (1) becomes NaN, while the
    fp64 state of the oracle (and the fp32 state of the GPU path) stays finite."""
    from synth import gen_attn
    inp = gen_attn(4, 1, 16384, H=1, dtype="bf16", k_scale=30.0, outlier_frac=0.01, norm=False)
    k0 = inp.k[0].astype(np.float64)
    v0 = inp.v[0].astype(np.float64)
    q0 = inp.q[0].astype(np.float64)
    phik = np.maximum(k0, 0.0)
    z64 = phik.sum(axis=0)
    assert z64.max() > 65504.0 and np.isfinite(z64).all()
    phiq = np.maximum(q0, 0.0).astype(np.float16)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):  # the overflow is the point
        z16 = np.cumsum(phik.astype(np.float16), axis=0, dtype=np.float16)[-1]
        S16 = (phik.astype(np.float16).T @ v0.astype(np.float16)).astype(np.float16)
        o16 = (phiq @ S16) / (phiq @ z16 + np.float16(inp.eps))[:, None]
    assert np.isinf(z16).any()
    assert np.isnan(o16).any() or not np.isfinite(o16).all()
    o64 = oracle.linear_attn(inp.q, inp.k, inp.v, None, None, 1, 32, inp.eps)
    assert np.isfinite(o64).all()

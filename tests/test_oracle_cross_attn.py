"""CPU pins of the cross-attention oracle (oracle/cross_attn.py) against what the mathematics fixes:
closed forms (one text token, identical keys, two keys whose logit gap is set by hand), a pure-Python
brute force with math.exp on tiny cases, and invariants (key permutation, masking = truncation, the
norm's indifference to per-token positive scaling, the norm spanning all heads).  Each of these
mistakes fails at least one pin: no 1/sqrt(D), softmax over the queries, a per-head norm, the norm on
v, the gain inside the mean, the mask ignored, keys of another head."""
import math

import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _case(seed, B=2, N=5, L=7, H=3, D=4):
    r = _rng(seed)
    C = H * D
    q, k, v = r.normal(size=(B, N, C)), r.normal(size=(B, L, C)), r.normal(size=(B, L, C))
    gq, gk = 1.0 + 0.3 * r.normal(size=C), 1.0 + 0.3 * r.normal(size=C)
    return q, k, v, gq, gk


@pytest.mark.parametrize("norm", [True, False])
def test_single_text_token_returns_its_value(norm):
    q, k, v, gq, gk = _case(1, L=1)
    o = oracle.cross_attn(q, k, v, gq if norm else None, gk if norm else None, H=3, D=4)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), rtol=0, atol=1e-15)


@pytest.mark.parametrize("norm", [True, False])
def test_identical_keys_give_the_mean_value(norm):
    q, k, v, gq, gk = _case(2, L=6)
    k[:] = k[:, :1]
    lens = [6, 3]
    o = oracle.cross_attn(q, k, v, gq if norm else None, gk if norm else None, H=3, D=4, kv_len=lens)
    for b, n in enumerate(lens):
        np.testing.assert_allclose(o[b], np.broadcast_to(v[b, :n].mean(axis=0), o[b].shape), rtol=0, atol=1e-14)


def test_two_keys_closed_form_with_the_sqrt_d_scale():
    """Norm off, one head of D = 4: logits q.k0 = 6 and q.k1 = 2, so after the 1/sqrt(D) = 1/2 scale
    the weight of key 0 is 1 / (1 + e^-2)."""
    q = np.array([[[1.0, 1.0, 1.0, 1.0]]])
    k = np.array([[[3.0, 1.0, 1.0, 1.0], [0.5, 0.5, 0.5, 0.5]]])
    v = np.array([[[1.0, 0.0, 2.0, -1.0], [0.0, 4.0, 2.0, 3.0]]])
    o = oracle.cross_attn(q, k, v, None, None, H=1, D=4)
    w0 = 1.0 / (1.0 + math.exp(-2.0))
    np.testing.assert_allclose(o[0, 0], w0 * v[0, 0] + (1 - w0) * v[0, 1], rtol=1e-13)


def test_gains_act_after_the_norm():
    """Rows of +-1 have RMS 1, so with eps = 0 the norm leaves them as they are and only the gains act:
    a query gain of 3 on every channel triples the logit gap of the case above."""
    q = np.array([[[1.0, 1.0, -1.0, 1.0]]])
    k = np.array([[[1.0, 1.0, -1.0, 1.0], [1.0, -1.0, 1.0, 1.0]]])  # q.k0 = 4, q.k1 = 0
    v = np.array([[[2.0, 0.0, 0.0, 0.0], [0.0, 2.0, 0.0, 0.0]]])
    ones = np.ones(4)
    o1 = oracle.cross_attn(q, k, v, ones, ones, H=1, D=4, eps=0.0)
    o3 = oracle.cross_attn(q, k, v, 3 * ones, ones, H=1, D=4, eps=0.0)
    for o, gap in ((o1, 2.0), (o3, 6.0)):
        w0 = 1.0 / (1.0 + math.exp(-gap))
        np.testing.assert_allclose(o[0, 0], [2 * w0, 2 * (1 - w0), 0.0, 0.0], rtol=1e-13, atol=1e-300)


def _brute(q, k, v, gq, gk, H, D, eps, kv_len):
    """Pure-Python loops with math.exp and math.sqrt."""
    B, N, C = q.shape
    out = np.zeros((B, N, C))

    def norm(row, g):
        if g is None:
            return [float(x) for x in row]
        ms = sum(float(x) * float(x) for x in row) / len(row)
        return [float(x) / math.sqrt(ms + eps) * float(gi) for x, gi in zip(row, g)]

    for b in range(B):
        keys = [norm(k[b, j], gk) for j in range(kv_len[b])]
        for i in range(N):
            qi = norm(q[b, i], gq)
            for h in range(H):
                lo = h * D
                logits = [sum(qi[lo + d] * keys[j][lo + d] for d in range(D)) / math.sqrt(D) for j in range(kv_len[b])]
                m = max(logits)
                e = [math.exp(x - m) for x in logits]
                s = sum(e)
                for d in range(D):
                    out[b, i, lo + d] = sum(e[j] / s * float(v[b, j, lo + d]) for j in range(kv_len[b]))
    return out


@pytest.mark.parametrize("norm", [True, False])
def test_brute_force_tiny(norm):
    q, k, v, gq, gk = _case(3, B=2, N=3, L=5, H=2, D=3)
    lens = [5, 2]
    args = (gq, gk) if norm else (None, None)
    o = oracle.cross_attn(q, k, v, *args, H=2, D=3, eps=1e-3, kv_len=lens)
    np.testing.assert_allclose(o, _brute(q, k, v, *args, H=2, D=3, eps=1e-3, kv_len=lens), rtol=1e-12, atol=1e-14)


def test_key_permutation_invariance():
    q, k, v, gq, gk = _case(4, L=9)
    perm = _rng(5).permutation(9)
    o = oracle.cross_attn(q, k, v, gq, gk, H=3, D=4)
    np.testing.assert_allclose(oracle.cross_attn(q, k[:, perm], v[:, perm], gq, gk, H=3, D=4), o, rtol=1e-12, atol=1e-14)


def test_masking_equals_truncation():
    q, k, v, gq, gk = _case(6, B=1, L=8)
    o_mask = oracle.cross_attn(q, k, v, gq, gk, H=3, D=4, kv_len=[5])
    o_cut = oracle.cross_attn(q, k[:, :5], v[:, :5], gq, gk, H=3, D=4)
    np.testing.assert_allclose(o_mask, o_cut, rtol=0, atol=0)
    assert not np.allclose(o_mask, oracle.cross_attn(q, k, v, gq, gk, H=3, D=4))


def test_norm_ignores_positive_token_scaling():
    """With eps = 0 the RMSNorm output of c*x is that of x for c > 0, for queries and keys alike."""
    q, k, v, gq, gk = _case(7)
    r = _rng(8)
    cq, ck = r.uniform(0.1, 10, size=q.shape[:2] + (1,)), r.uniform(0.1, 10, size=k.shape[:2] + (1,))
    o = oracle.cross_attn(q, k, v, gq, gk, H=3, D=4, eps=0.0)
    np.testing.assert_allclose(oracle.cross_attn(q * cq, k * ck, v, gq, gk, H=3, D=4, eps=0.0), o, rtol=1e-12, atol=1e-14)
    # without the norm the scaling changes the result
    o_off = oracle.cross_attn(q, k, v, None, None, H=3, D=4)
    assert not np.allclose(oracle.cross_attn(q * cq, k * ck, v, None, None, H=3, D=4), o_off, atol=1e-6)


def test_norm_spans_all_heads():
    """Scaling head 0's query channels changes the token's RMS and so the other heads' outputs; values
    are not normalised, so scaling v scales the output."""
    q, k, v, gq, gk = _case(9)
    o = oracle.cross_attn(q, k, v, gq, gk, H=3, D=4)
    q2 = q.copy()
    q2[..., :4] *= 5.0
    o2 = oracle.cross_attn(q2, k, v, gq, gk, H=3, D=4)
    assert np.abs(o2[..., 4:] - o[..., 4:]).max() > 1e-3
    np.testing.assert_allclose(oracle.cross_attn(q, k, 2.5 * v, gq, gk, H=3, D=4), 2.5 * o, rtol=1e-13)


def test_heads_see_only_their_own_channels():
    q, k, v, gq, gk = _case(10)
    o = oracle.cross_attn(q, k, v, None, None, H=3, D=4)
    v2 = v.copy()
    v2[..., 8:] += 1.0  # head 2's values only
    o2 = oracle.cross_attn(q, k, v2, None, None, H=3, D=4)
    np.testing.assert_allclose(o2[..., :8], o[..., :8], rtol=0, atol=0)
    np.testing.assert_allclose(o2[..., 8:], o[..., 8:] + 1.0, rtol=1e-13)


def test_dominant_key_takes_the_weight():
    """A logit gap of 200 (after the scale) leaves the others e^-200 of the weight: o = v of that key."""
    q = np.zeros((1, 1, 4))
    q[0, 0, 0] = 20.0
    k = np.zeros((1, 3, 4))
    k[0, 1, 0] = 20.0  # q.k1 = 400 -> 200 after the scale
    v = _rng(11).normal(size=(1, 3, 4))
    o = oracle.cross_attn(q, k, v, None, None, H=1, D=4)
    np.testing.assert_allclose(o[0, 0], v[0, 1], rtol=1e-15, atol=1e-80)


def test_argument_errors():
    q, k, v, gq, gk = _case(12)
    with pytest.raises(ValueError):
        oracle.cross_attn(q, k, v, gq, None, H=3, D=4)
    with pytest.raises(ValueError):
        oracle.cross_attn(q, k, v, gq, gk, H=3, D=4, kv_len=[0, 3])
    with pytest.raises(ValueError):
        oracle.cross_attn(q, k, v, gq, gk, H=3, D=4, kv_len=[8, 3])

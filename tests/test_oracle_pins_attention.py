"""Pins of the oracle's scaled dot-product attention: torch CPU float64
scaled_dot_product_attention (with and without the causal mask, square and
rectangular), its log-sum-exp against an independent log-sum-exp of the
scores, and closed forms (identical keys average the values; a dominant key
copies its value; the causal first query sees only the first key)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(99)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Sk", [(7, 7), (33, 64), (64, 33), (1, 5)])
def test_torch_float64(causal, Sq, Sk):
    B, H, D = 2, 3, 16
    q = RNG.normal(size=(B, H, Sq, D))
    k = RNG.normal(size=(B, H, Sk, D))
    v = RNG.normal(size=(B, H, Sk, D))
    scale = 0.3
    o, lse = oracle.attention(q, k, v, causal=causal, scale=scale)
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    if causal:
        # queries aligned to the end of the keys: key j visible to query i iff j <= i + Sk - Sq
        mask = torch.ones(Sq, Sk, dtype=torch.bool).tril(diagonal=Sk - Sq)
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
        vis = mask.numpy()
    else:
        ref = F.scaled_dot_product_attention(tq, tk, tv, scale=scale)
        vis = np.ones((Sq, Sk), bool)
    ok = vis.any(1)
    assert np.max(np.abs(o[:, :, ok] - ref.numpy()[:, :, ok])) <= 1e-13
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    s = np.where(vis, s, -np.inf)
    m = s.max(-1, keepdims=True)
    with np.errstate(invalid="ignore"):
        want = (m + np.log(np.exp(s - m).sum(-1, keepdims=True)))[..., 0]
    assert np.max(np.abs(lse[:, :, ok] - want[:, :, ok])) <= 1e-13
    assert np.all(o[:, :, ~ok] == 0) and np.all(np.isneginf(lse[:, :, ~ok]))


def test_closed_forms():
    D = 8
    v = RNG.normal(size=(1, 1, 5, D))
    q = RNG.normal(size=(1, 1, 4, D))
    k = np.repeat(RNG.normal(size=(1, 1, 1, D)), 5, axis=2)      # identical keys
    o, lse = oracle.attention(q, k, v, scale=1.0)
    assert np.allclose(o[0, 0], v[0, 0].mean(0)[None, :], rtol=0, atol=1e-14)
    k2 = np.zeros((1, 1, 5, D))
    k2[0, 0, 3, 0] = 1.0
    q2 = np.zeros((1, 1, 1, D))
    q2[0, 0, 0, 0] = 1000.0                                       # key 3 dominates
    o2, lse2 = oracle.attention(q2, k2, v, scale=1.0)
    assert np.allclose(o2[0, 0, 0], v[0, 0, 3], rtol=0, atol=1e-12)
    assert lse2[0, 0, 0] == pytest.approx(1000.0, rel=1e-15)
    o3, lse3 = oracle.attention(q, RNG.normal(size=(1, 1, 4, D)), v[:, :, :4], causal=True)
    assert np.array_equal(o3[0, 0, 0], v[0, 0, 0])               # the first query sees key 0 only


def test_stored_inputs_decode_exactly():
    q = RNG.normal(size=(1, 2, 9, 16)).astype(np.float32)
    k = RNG.normal(size=(1, 2, 11, 16)).astype(np.float32)
    v = RNG.normal(size=(1, 2, 11, 16)).astype(np.float32)
    a = oracle.attention(q, k, v, causal=True)
    b = oracle.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                         causal=True, scale=float(np.float32(0.25)))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])

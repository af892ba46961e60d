"""Pins of the backward oracle (CPU only): torch float64 autograd through
SDPA, central finite differences, grouped heads against summed expanded
heads, and closed forms (constant values give zero dQ and dK; the rows of P
sum to one, so the dV rows sum to the dO rows). The pages ask for exactly
these references ("Intermediate and advanced workshop validation",
backward checks: float64 autograd and finite differences).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import backward, dense


def _case(seed, n, d, scale_q=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, d)) * scale_q
    k, v, do = (rng.standard_normal((n, d)) for _ in range(3))
    return q, k, v, do


@pytest.mark.parametrize("n,d", [(1, 4), (3, 2), (17, 8), (64, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_vs_torch_autograd(n, d, causal):
    q, k, v, do = _case(n * 10 + d, n, d, 1.5)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = backward.attention_backward(q, k, v, do, scale, causal)
    qt, kt, vt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    o = F.scaled_dot_product_attention(qt[None], kt[None], vt[None], is_causal=causal, scale=scale)[0]
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_central_finite_differences(causal):
    """d/dx of L = sum(dO * O(q, k, v)) by central differences on every
    entry, with O from the forward oracle."""
    q, k, v, do = _case(5, 4, 3, 1.0)
    dq, dk, dv = backward.attention_backward(q, k, v, do, 0.8, causal)
    h = 1e-6

    def loss(q_, k_, v_):
        return float((dense.attention(q_, k_, v_, 0.8, causal)[0] * do).sum())
    for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_constant_values_give_zero_query_and_key_gradients():
    """Every v_j = c: O = c whatever the weights, so dQ = dK = 0; and since
    each row of P sums to one, sum_j dV_j = sum_i dO_i."""
    q, k, _, do = _case(6, 20, 5, 2.0)
    v = np.tile(np.arange(5.0), (20, 1))
    for causal in (False, True):
        dq, dk, dv = backward.attention_backward(q, k, v, do, 0.5, causal)
        assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
        np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)


def test_grouped_heads_sum_expanded_gradients():
    rng = np.random.default_rng(7)
    q, do = (rng.standard_normal((2, 6, 9, 4)) for _ in range(2))
    k, v = (rng.standard_normal((2, 2, 9, 4)) for _ in range(2))
    dq, dk, dv = backward.attention_backward_bhnd(q, k, v, do, 0.5, True)
    qt = torch.from_numpy(q).requires_grad_(True)
    kt = torch.from_numpy(k).requires_grad_(True)
    vt = torch.from_numpy(v).requires_grad_(True)
    o = F.scaled_dot_product_attention(qt, kt.repeat_interleave(3, 1), vt.repeat_interleave(3, 1),
                                       is_causal=True, scale=0.5)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_linear_in_output_gradient():
    q, k, v, do = _case(8, 12, 4)
    a = backward.attention_backward(q, k, v, do, 0.5, True)
    b = backward.attention_backward(q, k, v, 3.0 * do, 0.5, True)
    for x, y in zip(a, b):
        np.testing.assert_allclose(y, 3.0 * x, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_vs_autograd_through_packed_mask(causal):
    """Packed sequences (one of them empty) with grouped heads: torch float64
    autograd through SDPA over all T tokens with an explicit mask (same
    sequence, and causal by position within it), on KV heads repeated over
    their query heads, so autograd itself sums each KV head's gradients."""
    rng = np.random.default_rng(31)
    lengths = [5, 0, 9, 1, 7]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    t, hq, hkv, d = int(cu[-1]), 4, 2, 6
    q, do = rng.standard_normal((t, hq, d)), rng.standard_normal((t, hq, d))
    k, v = rng.standard_normal((t, hkv, d)), rng.standard_normal((t, hkv, d))
    scale = 0.45
    dq, dk, dv = backward.attention_backward_varlen(q, k, v, do, cu, scale, causal)
    seq = np.repeat(np.arange(len(lengths)), lengths)
    pos = np.arange(t) - cu[seq]
    allowed = seq[:, None] == seq[None, :]
    if causal:
        allowed &= pos[None, :] <= pos[:, None]
    qt, kt, vt = (torch.from_numpy(x.transpose(1, 0, 2).copy()).requires_grad_(True) for x in (q, k, v))
    o = F.scaled_dot_product_attention(qt[None], kt.repeat_interleave(hq // hkv, 0)[None],
                                       vt.repeat_interleave(hq // hkv, 0)[None],
                                       attn_mask=torch.from_numpy(allowed), scale=scale)[0]
    o.backward(torch.from_numpy(do.transpose(1, 0, 2).copy()))
    np.testing.assert_allclose(dq, qt.grad.numpy().transpose(1, 0, 2), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy().transpose(1, 0, 2), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy().transpose(1, 0, 2), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_sparse_vs_autograd_through_the_mask(causal):
    """Window, global tokens and a per-head block mask with grouped heads:
    torch float64 autograd through SDPA with the same boolean mask, on KV
    heads repeated over their query heads. The block mask keeps every
    diagonal block, so every row has an eligible key."""
    rng = np.random.default_rng(41)
    n, hq, hkv, d = 40, 4, 2, 5
    q, do = rng.standard_normal((1, hq, n, d)), rng.standard_normal((1, hq, n, d))
    k, v = rng.standard_normal((1, hkv, n, d)), rng.standard_normal((1, hkv, n, d))
    bm = rng.integers(0, 2, size=(hq, 5, 5)).astype(np.uint8)
    for h in range(hq):
        np.fill_diagonal(bm[h], 1)
    dq, dk, dv = backward.attention_backward_sparse_bhnd(q, k, v, do, 0.4, causal, 6, 3, 2, bm, 8, 8)
    mask = torch.from_numpy(np.stack([dense.sparse_eligibility(n, n, causal, 6, 3, 2, bm[h], 8, 8)
                                      for h in range(hq)]))
    assert mask.any(dim=2).all()
    qt, kt, vt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    o = F.scaled_dot_product_attention(qt, kt.repeat_interleave(2, 1), vt.repeat_interleave(2, 1),
                                       attn_mask=mask[None], scale=0.4)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_sparse_rows_without_keys_contribute_nothing():
    """A query block whose mask row is all zero has no eligible key: its dQ
    is exactly 0 and dK, dV equal those of the same problem with its dO set
    to zero (no other row is affected)."""
    rng = np.random.default_rng(42)
    n, d = 32, 4
    q, k, v, do = (rng.standard_normal((1, 1, n, d)) for _ in range(4))
    bm = np.ones((4, 4), dtype=np.uint8)
    bm[1, :] = 0                                          # rows 8..15: no key
    dq, dk, dv = backward.attention_backward_sparse_bhnd(q, k, v, do, 0.5, True, -1, -1, 0, bm, 8, 8)
    assert np.all(dq[0, 0, 8:16] == 0.0)
    do2 = do.copy()
    do2[0, 0, 8:16] = 0.0
    _, dk2, dv2 = backward.attention_backward_sparse_bhnd(q, k, v, do2, 0.5, True, -1, -1, 0, bm, 8, 8)
    np.testing.assert_array_equal(dk, dk2)
    np.testing.assert_array_equal(dv, dv2)


def test_unrestricted_sparse_is_dense_backward():
    rng = np.random.default_rng(43)
    q, do = rng.standard_normal((2, 4, 20, 3)), rng.standard_normal((2, 4, 20, 3))
    k, v = rng.standard_normal((2, 2, 20, 3)), rng.standard_normal((2, 2, 20, 3))
    for causal in (False, True):
        a = backward.attention_backward_sparse_bhnd(q, k, v, do, 0.5, causal)
        b = backward.attention_backward_bhnd(q, k, v, do, 0.5, causal)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("nq,nk", [(1, 9), (5, 17), (12, 12), (9, 4)])
def test_cache_vs_autograd_bottom_right(nq, nk):
    """Unequal lengths, causal with query i at position i + (Nk - Nq):
    torch float64 autograd through SDPA with the explicit mask, grouped heads
    repeated. Queries before the first key (Nq > Nk) have no key: autograd
    runs on the other rows only, and those rows' dQ is exactly 0."""
    rng = np.random.default_rng(nq * 31 + nk)
    hq, hkv, d = 4, 2, 5
    q, do = rng.standard_normal((1, hq, nq, d)), rng.standard_normal((1, hq, nq, d))
    k, v = rng.standard_normal((1, hkv, nk, d)), rng.standard_normal((1, hkv, nk, d))
    dq, dk, dv = backward.attention_backward_cache_bhnd(q, k, v, do, 0.45, True)
    pos = np.arange(nq) + (nk - nq)
    live = pos >= 0
    mask = torch.from_numpy(np.arange(nk)[None, :] <= pos[live][:, None])
    qt, kt, vt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q[:, :, live], k, v))
    o = F.scaled_dot_product_attention(qt, kt.repeat_interleave(2, 1), vt.repeat_interleave(2, 1),
                                       attn_mask=mask, scale=0.45)
    o.backward(torch.from_numpy(do[:, :, live].copy()))
    np.testing.assert_allclose(dq[:, :, live], qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    assert np.all(dq[:, :, ~live] == 0.0)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_cache_noncausal_and_equal_lengths_reduce_to_dense():
    rng = np.random.default_rng(44)
    q, do = rng.standard_normal((1, 2, 7, 3)), rng.standard_normal((1, 2, 7, 3))
    k, v = rng.standard_normal((1, 2, 7, 3)), rng.standard_normal((1, 2, 7, 3))
    for causal in (False, True):
        a = backward.attention_backward_cache_bhnd(q, k, v, do, 0.5, causal)
        b = backward.attention_backward_bhnd(q, k, v, do, 0.5, causal)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
    k2, v2 = rng.standard_normal((1, 2, 11, 3)), rng.standard_normal((1, 2, 11, 3))
    dq, dk, dv = backward.attention_backward_cache_bhnd(q, k2, v2, do, 0.5, False)
    qt, kt, vt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k2, v2))
    F.scaled_dot_product_attention(qt, kt, vt, scale=0.5).backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-11, atol=1e-12)

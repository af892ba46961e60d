"""Pins of the dense float64 oracle (CPU only).

Each test ties ``oracle.dense`` to something other than itself: hand-derived
cases, closed forms, invariants of softmax attention, or an independent
library routine (torch CPU float64 ``scaled_dot_product_attention`` and
``torch.logsumexp``). The cases are chosen so that a plausible slip in the
oracle (a dropped max shift, a wrong sign, a transposed operand, an excluded
diagonal, log2 instead of ln, a head map h % Hkv instead of h // group)
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_derived_cases.json")


def _f(x):
    return float(x)   # JSON strings such as "-inf" parse with float()


def _load():
    with open(GOLDEN) as fh:
        return json.load(fh)


# --------------------------------------------------------------- golden cases
@pytest.mark.parametrize("case", _load()["attention"], ids=lambda c: c["name"])
def test_hand_derived_attention(case):
    q, k, v = (np.array(case[x], dtype=np.float64) for x in ("q", "k", "v"))
    for mode in ("noncausal", "causal"):
        if mode not in case:
            continue
        o, lse = dense.attention(q, k, v, case["scale"], causal=(mode == "causal"))
        np.testing.assert_allclose(o, np.array(case[mode]["o"]), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, np.array(case[mode]["lse"]), rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("case", _load()["merge"], ids=lambda c: c["name"])
def test_hand_derived_merge(case):
    m = np.array([_f(x) for x in case["m"]])
    l = np.array(case["l"], dtype=np.float64)
    acc = np.array(case["acc"], dtype=np.float64)
    o, lse = dense.merge_partials(m[None], l[None], acc[None])
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    np.testing.assert_allclose(o[0], np.array(case["o"]), rtol=1e-13, atol=1e-13)
    exp_lse = _f(case["lse"])
    if math.isinf(exp_lse):
        assert lse[0] == exp_lse
    else:
        assert abs(lse[0] - exp_lse) < 1e-13


# ------------------------------------------------------- independent library
def _torch_ref(q, k, v, scale, causal):
    """torch CPU float64 SDPA and logsumexp of the masked scaled scores."""
    qt, kt, vt = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)[0, 0]
    s = scale * (qt[0, 0] @ kt[0, 0].transpose(0, 1))
    if causal:
        mask = torch.ones(s.shape, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


@pytest.mark.parametrize("n,d", [(1, 4), (2, 3), (3, 8), (5, 2), (17, 16), (129, 32)])
@pytest.mark.parametrize("causal", [False, True])
def test_vs_torch_sdpa(n, d, causal):
    rng = np.random.default_rng(100 + n * 7 + d)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    scale = 1.0 / math.sqrt(d)
    o, lse = dense.attention(q, k, v, scale, causal)
    o_ref, lse_ref = _torch_ref(q, k, v, scale, causal)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_rectangular_noncausal_vs_torch():
    """Nq != Nk (and Dv != D) exposes a transposed operand."""
    rng = np.random.default_rng(7)
    q = rng.standard_normal((5, 6))
    k = rng.standard_normal((9, 6))
    v = rng.standard_normal((9, 3))
    o, lse = dense.attention(q, k, v, 0.3, causal=False)
    qt, kt, vt = (torch.from_numpy(x)[None] for x in (q, k, v))
    o_ref = F.scaled_dot_product_attention(qt, kt, vt, scale=0.3)[0].numpy()
    lse_ref = torch.logsumexp(0.3 * qt[0] @ kt[0].T, dim=-1).numpy()
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------- closed forms
def test_single_key_is_identity():
    """N = 1: the only key gets weight 1: O = v0, lse = s00 (causal or not)."""
    q = np.array([[0.5, -1.5, 2.0]])
    k = np.array([[1.0, 2.0, -0.25]])
    v = np.array([[3.0, -4.0, 5.0]])
    for causal in (False, True):
        o, lse = dense.attention(q, k, v, 0.7, causal)
        np.testing.assert_array_equal(o, v)
        assert abs(lse[0] - 0.7 * float(q[0] @ k[0])) < 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_logits_mean_of_values(causal):
    """Q = 0: every eligible key has score 0, so O_i is the mean of the
    eligible values and lse_i = ln(#eligible)."""
    rng = np.random.default_rng(3)
    n, d = 37, 5
    q = np.zeros((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    o, lse = dense.attention(q, k, v, 0.25, causal)
    for i in range(n):
        cnt = i + 1 if causal else n
        np.testing.assert_allclose(o[i], v[:cnt].mean(axis=0), rtol=1e-13, atol=1e-14)
        assert abs(lse[i] - math.log(cnt)) < 1e-13


def test_one_hot_large_gap():
    """A key whose score exceeds every other by >= 60 takes all the weight
    (within e^-60); lse equals that score within the same bound."""
    rng = np.random.default_rng(4)
    n, d = 16, 8
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d)) * 0.01
    v = rng.standard_normal((n, d))
    jstar = 11
    k[jstar] = q[5] * 200.0        # row 5's score on key 11 is huge
    o, lse = dense.attention(q, k, v, 1.0, causal=False)
    s = q[5] @ k.T
    assert s[jstar] - np.delete(s, jstar).max() >= 60
    np.testing.assert_allclose(o[5], v[jstar], rtol=0, atol=1e-20 + 1e-24 * np.abs(v).max() + 1e-25)
    assert abs(lse[5] - s[jstar]) < 1e-12 * abs(s[jstar])


def test_extreme_logits_finite():
    """Scores near 1e4 would overflow exp() without the max shift."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((8, 4)) * 100.0
    k = rng.standard_normal((8, 4)) * 100.0
    v = rng.standard_normal((8, 4))
    for causal in (False, True):
        o, lse = dense.attention(q, k, v, 1.0, causal)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        o_ref, lse_ref = _torch_ref(q, k, v, 1.0, causal)
        np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(lse, lse_ref, rtol=1e-14, atol=0)


# --------------------------------------------------------------- invariants
def test_causal_future_perturbation_bitwise():
    """Changing K[j], V[j] must leave causal rows i < j bit-identical."""
    rng = np.random.default_rng(6)
    n, d = 40, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o0, lse0 = dense.attention(q, k, v, 0.35, causal=True)
    for j in (1, 17, 39):
        k2, v2 = k.copy(), v.copy()
        k2[j] = rng.standard_normal(d) * 50
        v2[j] = rng.standard_normal(d) * 50
        o1, lse1 = dense.attention(q, k2, v2, 0.35, causal=True)
        np.testing.assert_array_equal(o1[:j], o0[:j])
        np.testing.assert_array_equal(lse1[:j], lse0[:j])
        assert not np.array_equal(o1[j:], o0[j:])


def test_noncausal_key_permutation_equivariance():
    rng = np.random.default_rng(8)
    n, d = 23, 6
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    perm = rng.permutation(n)
    o0, lse0 = dense.attention(q, k, v, 0.4, causal=False)
    o1, lse1 = dense.attention(q, k[perm], v[perm], 0.4, causal=False)
    np.testing.assert_allclose(o1, o0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse1, lse0, rtol=1e-13, atol=1e-13)


def test_linear_in_values():
    rng = np.random.default_rng(9)
    n, d = 19, 4
    q, k, v1, v2 = (rng.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        a, _ = dense.attention(q, k, v1, 0.5, causal)
        b, _ = dense.attention(q, k, v2, 0.5, causal)
        c, _ = dense.attention(q, k, 2.0 * v1 - 3.0 * v2, 0.5, causal)
        np.testing.assert_allclose(c, 2.0 * a - 3.0 * b, rtol=1e-12, atol=1e-12)


def test_row_blocking_is_invisible():
    rng = np.random.default_rng(10)
    n, d = 70, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    for causal in (False, True):
        a = dense.attention(q, k, v, 0.3, causal, row_block=512)
        b = dense.attention(q, k, v, 0.3, causal, row_block=7)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


def test_sampled_rows_match_full():
    rng = np.random.default_rng(11)
    b_, h_, n, d = 2, 3, 33, 8
    q, k, v = (rng.standard_normal((b_, h_, n, d)) for _ in range(3))
    rows = np.stack([np.stack([rng.choice(n, 6, replace=False) for _ in range(h_)]) for _ in range(b_)])
    for causal in (False, True):
        of, lf = dense.attention_bhnd(q, k, v, 0.3, causal)
        os_, ls = dense.attention_bhnd(q, k, v, 0.3, causal, rows=rows)
        for b in range(b_):
            for h in range(h_):
                np.testing.assert_allclose(os_[b, h], of[b, h][rows[b, h]], rtol=1e-13, atol=1e-14)
                np.testing.assert_allclose(ls[b, h], lf[b, h][rows[b, h]], rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------ varlen + GQA
def _packed_case(seed, lengths, hq, hkv, d):
    rng = np.random.default_rng(seed)
    t = int(sum(lengths))
    q = rng.standard_normal((t, hq, d))
    k = rng.standard_normal((t, hkv, d))
    v = rng.standard_normal((t, hkv, d))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return q, k, v, cu


def test_varlen_gqa_vs_torch_enable_gqa():
    """Each packed sequence equals torch SDPA with enable_gqa (which repeats
    each KV head over its Hq/Hkv consecutive query heads)."""
    lengths = [5, 1, 12, 7]
    hq, hkv, d = 8, 2, 4
    q, k, v, cu = _packed_case(12, lengths, hq, hkv, d)
    o, lse = dense.varlen_gqa(q, k, v, cu, 0.5, causal=True)
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        qt = torch.from_numpy(q[a:b]).permute(1, 0, 2)[None]
        kt = torch.from_numpy(k[a:b]).permute(1, 0, 2)[None]
        vt = torch.from_numpy(v[a:b]).permute(1, 0, 2)[None]
        o_ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.5,
                                               enable_gqa=True)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(o[a:b], o_ref, rtol=1e-12, atol=1e-12)
        kt_e = kt.repeat_interleave(hq // hkv, dim=1)
        sc = 0.5 * qt[0] @ kt_e[0].transpose(1, 2)
        sc = sc.masked_fill(~torch.ones(sc.shape[1:], dtype=torch.bool).tril(), -math.inf)
        np.testing.assert_allclose(lse[:, a:b], torch.logsumexp(sc, dim=-1).numpy(),
                                   rtol=1e-12, atol=1e-12)


def test_varlen_cross_sequence_isolation():
    """Perturbing one sequence's tokens leaves every other sequence bitwise
    unchanged."""
    lengths = [6, 9, 4]
    q, k, v, cu = _packed_case(13, lengths, 4, 2, 8)
    o0, lse0 = dense.varlen_gqa(q, k, v, cu, 0.3, causal=True)
    a, b = cu[1], cu[2]
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[a:b] += 3.0
    k2[a:b] *= -2.0
    v2[a:b] += 7.0
    o1, lse1 = dense.varlen_gqa(q2, k2, v2, cu, 0.3, causal=True)
    for s in (0, 2):
        x, y = cu[s], cu[s + 1]
        np.testing.assert_array_equal(o1[x:y], o0[x:y])
        np.testing.assert_array_equal(lse1[:, x:y], lse0[:, x:y])


def test_varlen_rows_subset():
    lengths = [10, 3]
    q, k, v, cu = _packed_case(14, lengths, 4, 1, 4)
    o, lse = dense.varlen_gqa(q, k, v, cu, 0.3, causal=True)
    sub = dense.varlen_gqa(q, k, v, cu, 0.3, causal=True, rows={(0, 3): [0, 4, 9], (1, 0): [2]})
    np.testing.assert_allclose(sub[(0, 3)][0], o[[0, 4, 9], 3], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(sub[(0, 3)][1], lse[3, [0, 4, 9]], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(sub[(1, 0)][0], o[[12], 0], rtol=1e-14, atol=1e-15)


# ------------------------------------------------------ split partial state
@pytest.mark.parametrize("nk,chunk", [(64, 16), (70, 16), (5, 8), (33, 1), (100, 100)])
def test_split_merge_equals_dense(nk, chunk):
    """Partition invariance: merging the per-chunk partials of any chunking
    reproduces dense attention."""
    rng = np.random.default_rng(nk * 31 + chunk)
    q = rng.standard_normal((3, 8)) * 2
    k = rng.standard_normal((nk, 8))
    v = rng.standard_normal((nk, 8))
    m, l, acc = dense.split_partials(q, k, v, 0.3, chunk)
    assert m.shape == (3, -(-nk // chunk))
    o, lse = dense.merge_partials(m, l, acc)
    o_ref, lse_ref = dense.attention(q, k, v, 0.3, causal=False)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=1e-13)


def test_single_partial_vs_library():
    """One chunk's state: m + ln l is that chunk's logsumexp (torch), and
    acc / l is SDPA restricted to the chunk's keys."""
    rng = np.random.default_rng(15)
    q = rng.standard_normal((4, 6))
    k = rng.standard_normal((20, 6))
    v = rng.standard_normal((20, 6))
    m, l, acc = dense.split_partials(q, k, v, 0.5, 8)
    for c, (j0, j1) in enumerate([(0, 8), (8, 16), (16, 20)]):
        qt, kt, vt = (torch.from_numpy(x) for x in (q, k[j0:j1], v[j0:j1]))
        lse_ref = torch.logsumexp(0.5 * qt @ kt.T, dim=-1).numpy()
        np.testing.assert_allclose(m[:, c] + np.log(l[:, c]), lse_ref, rtol=1e-13, atol=1e-13)
        o_ref = F.scaled_dot_product_attention(qt[None], kt[None], vt[None], scale=0.5)[0].numpy()
        np.testing.assert_allclose(acc[:, c] / l[:, c, None], o_ref, rtol=1e-12, atol=1e-13)
        s = 0.5 * q @ k[j0:j1].T
        np.testing.assert_array_equal(m[:, c], s.max(axis=1))


def test_merge_order_and_empty_partials():
    rng = np.random.default_rng(16)
    q = rng.standard_normal((2, 4))
    k = rng.standard_normal((40, 4))
    v = rng.standard_normal((40, 4))
    m, l, acc = dense.split_partials(q, k, v, 1.0, 10)
    perm = np.array([2, 0, 3, 1])
    o0, lse0 = dense.merge_partials(m, l, acc)
    o1, lse1 = dense.merge_partials(m[:, perm], l[:, perm], acc[:, perm])
    np.testing.assert_allclose(o1, o0, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse1, lse0, rtol=1e-14, atol=1e-14)
    me = np.concatenate([m, np.full((2, 2), -np.inf)], axis=1)
    le = np.concatenate([l, np.zeros((2, 2))], axis=1)
    ae = np.concatenate([acc, np.zeros((2, 2, 4))], axis=1)
    o2, lse2 = dense.merge_partials(me, le, ae)
    np.testing.assert_array_equal(o2, o0)
    np.testing.assert_array_equal(lse2, lse0)

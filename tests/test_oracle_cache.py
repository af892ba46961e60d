"""Pins of the K/V-cache oracle: unequal query/key lengths with bottom-right
causal alignment, grouped KV heads, and causal split partial states (CPU).

The queries are the last Nq tokens of a sequence whose cache holds Nk
positions, so query i sits at logical position i + (Nk - Nq) ("Attention
algorithms and data movement", lessons 04 and 05: unequal-length alignment
and cache payload from logical positions; the rule itself is the reading
taken here). Each test ties ``oracle.dense.attention_cache`` or the causal
``split_partials`` to something other than itself: brute-force loops, the
suffix of full self-attention computed by torch's float64 SDPA, torch's SDPA
with an explicit mask, and closed forms (a single decode query sees every
key; queries before the cache are empty rows).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import dense


def _case(seed, b, hq, hkv, nq, nk, d, dv=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, hq, nq, d))
    k = rng.standard_normal((b, hkv, nk, d))
    v = rng.standard_normal((b, hkv, nk, dv or d))
    return q, k, v


def _brute(q, k, v, scale, causal):
    """Stdlib loops over one (b, h) slice with bottom-right alignment."""
    nq, nk = len(q), len(k)
    o, lse = [], []
    for i in range(nq):
        pos = i + nk - nq
        keys = [j for j in range(nk) if (not causal) or j <= pos]
        if not keys:
            o.append([0.0] * len(v[0]))
            lse.append(-math.inf)
            continue
        s = [scale * sum(a * b for a, b in zip(q[i], k[j])) for j in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = sum(w)
        o.append([sum(w[t] * v[j][c] for t, j in enumerate(keys)) / tot for c in range(len(v[0]))])
        lse.append(mx + math.log(tot))
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("nq,nk", [(1, 1), (2, 5), (3, 3), (5, 2), (4, 1), (1, 6)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(nq, nk, causal):
    q, k, v = _case(10 * nq + nk, 1, 4, 2, nq, nk, 3, dv=2)
    o, lse = dense.attention_cache(q, k, v, 0.7, causal)
    for h in range(4):
        g = h // 2
        o_ref, lse_ref = _brute(q[0, h].tolist(), k[0, g].tolist(), v[0, g].tolist(), 0.7, causal)
        np.testing.assert_allclose(o[0, h], o_ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[0, h], lse_ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("nq,nk", [(1, 40), (7, 40), (40, 40), (33, 97)])
def test_suffix_of_full_causal_self_attention(nq, nk):
    """The last Nq queries of causal self-attention over Nk tokens (torch SDPA,
    float64, equal lengths) are exactly the cached-query problem."""
    rng = np.random.default_rng(nq + 3 * nk)
    d = 8
    q_full = rng.standard_normal((nk, d))
    k = rng.standard_normal((nk, d))
    v = rng.standard_normal((nk, d))
    qt, kt, vt = (torch.from_numpy(x)[None, None] for x in (q_full, k, v))
    o_full = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.4)[0, 0].numpy()
    s = 0.4 * qt[0, 0] @ kt[0, 0].T
    s = s.masked_fill(~torch.ones(s.shape, dtype=torch.bool).tril(), -math.inf)
    lse_full = torch.logsumexp(s, dim=-1).numpy()
    o, lse = dense.attention_cache(q_full[nk - nq:][None, None], k[None, None], v[None, None], 0.4, True)
    np.testing.assert_allclose(o[0, 0], o_full[nk - nq:], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], lse_full[nk - nq:], rtol=1e-12, atol=1e-13)


def test_gqa_vs_sdpa_explicit_bottom_right_mask():
    """Nq < Nk, Hq = 3 * Hkv: torch SDPA with an explicit boolean mask
    j <= i + (Nk - Nq) on KV heads repeated over consecutive query heads."""
    q, k, v = _case(5, 2, 6, 2, 9, 23, 4)
    o, lse = dense.attention_cache(q, k, v, 0.5, True)
    kt = torch.from_numpy(k).repeat_interleave(3, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(3, dim=1)
    qt = torch.from_numpy(q)
    mask = torch.arange(23)[None, :] <= (torch.arange(9) + 14)[:, None]
    o_ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.5).numpy()
    s = (0.5 * qt @ kt.transpose(-1, -2)).masked_fill(~mask, -math.inf)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-13)


def test_noncausal_sees_whole_cache():
    q, k, v = _case(6, 1, 2, 1, 5, 11, 4)
    o, lse = dense.attention_cache(q, k, v, 0.5, False)
    qt, kt, vt = torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)
    o_ref = F.scaled_dot_product_attention(qt, kt, vt, scale=0.5, enable_gqa=True).numpy()
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)


def test_single_decode_query_sees_every_key():
    """Nq = 1: the query is the newest token, so causal equals non-causal."""
    q, k, v = _case(7, 1, 2, 2, 1, 50, 8)
    a = dense.attention_cache(q, k, v, 0.3, True)
    b = dense.attention_cache(q, k, v, 0.3, False)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_queries_before_the_cache_are_empty_rows():
    """Nq > Nk: the first Nq - Nk queries have no eligible key (O = 0,
    lse = -inf exactly); the rest equal the Nq = Nk problem on those rows."""
    q, k, v = _case(8, 1, 2, 1, 10, 4, 5)
    o, lse = dense.attention_cache(q, k, v, 0.6, True)
    assert np.all(o[:, :, :6] == 0.0) and np.all(lse[:, :, :6] == -np.inf)
    o2, lse2 = dense.attention_cache(q[:, :, 6:], k, v, 0.6, True)
    np.testing.assert_array_equal(o[:, :, 6:], o2)
    np.testing.assert_array_equal(lse[:, :, 6:], lse2)
    assert np.isfinite(o).all()


def test_empty_cache():
    q, k, v = _case(9, 1, 2, 1, 3, 0, 4)
    for causal in (False, True):
        o, lse = dense.attention_cache(q, k, v, 0.5, causal)
        assert np.all(o == 0.0) and np.all(lse == -np.inf)


def test_rows_subset_matches_full():
    q, k, v = _case(11, 2, 4, 2, 30, 45, 4)
    o, lse = dense.attention_cache(q, k, v, 0.5, True)
    rows = np.array([[[0, 7, 29]] * 4] * 2)
    o_s, lse_s = dense.attention_cache(q, k, v, 0.5, True, rows=rows)
    np.testing.assert_array_equal(o_s, o[:, :, [0, 7, 29]])
    np.testing.assert_array_equal(lse_s, lse[:, :, [0, 7, 29]])


# ----------------------------------------------------- causal split partials
@pytest.mark.parametrize("nq,nk,chunk", [(1, 64, 16), (5, 70, 16), (20, 20, 8), (12, 7, 3), (3, 33, 1)])
def test_causal_split_merge_equals_cache_attention(nq, nk, chunk):
    """Partition invariance with causal chunks: merged partials reproduce the
    bottom-right causal result, including rows with no eligible key."""
    rng = np.random.default_rng(nq * 101 + nk + chunk)
    q = rng.standard_normal((nq, 6)) * 2
    k = rng.standard_normal((nk, 6))
    v = rng.standard_normal((nk, 6))
    m, l, acc = dense.split_partials(q, k, v, 0.4, chunk, causal=True)
    o, lse = dense.merge_partials(m, l, acc)
    o_ref, lse_ref = dense.attention_cache(q[None, None], k[None, None], v[None, None], 0.4, True)
    np.testing.assert_allclose(o, o_ref[0, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref[0, 0], rtol=1e-12, atol=1e-13)


def test_causal_chunks_after_the_query_are_empty_states():
    """A chunk that starts after a query's position gives exactly the empty
    state; a chunk cut by the position keeps only keys up to it (torch
    logsumexp over those keys)."""
    rng = np.random.default_rng(21)
    nq, nk, chunk = 4, 40, 10
    q = rng.standard_normal((nq, 5))
    k = rng.standard_normal((nk, 5))
    v = rng.standard_normal((nk, 5))
    m, l, acc = dense.split_partials(q, k, v, 0.5, chunk, causal=True)
    pos = np.arange(nq) + nk - nq          # 36..39
    for i in range(nq):
        for c in range(4):
            j0, j1 = c * chunk, min(nk, (c + 1) * chunk)
            keys = np.arange(j0, min(j1, pos[i] + 1))
            if keys.size == 0:
                assert m[i, c] == -np.inf and l[i, c] == 0.0 and np.all(acc[i, c] == 0.0)
                continue
            s = 0.5 * torch.from_numpy(k[keys]) @ torch.from_numpy(q[i])
            np.testing.assert_allclose(m[i, c] + np.log(l[i, c]), torch.logsumexp(s, 0).item(), rtol=1e-13)
    # explicit positions: earlier rows, so the last chunk is empty for all
    m2, l2, _ = dense.split_partials(q, k, v, 0.5, chunk, causal=True, q_pos=np.array([0, 5, 12, 29]))
    assert np.all(m2[:, 3] == -np.inf) and np.all(l2[:, 3] == 0.0)
    assert m2[0, 1] == -np.inf and np.isfinite(m2[2, 1])

"""Pins of the sparse-operator oracle: sliding windows with global tokens and
block-sparse masks ("Attention algorithms and data movement", lessons 06
and 07). CPU only.

The eligibility rule is pinned by stdlib set arithmetic and by closed-form
pair counts (window and global sets united, never double-counted); the
attention over it by torch float64 SDPA with the same boolean mask, by
independent per-block attention for a block-diagonal mask, and by closed
forms (a one-key window returns v_i).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import dense


def _brute_eligible(nq, nk, causal, left, right, g, bm, bq, bk):
    out = []
    for i in range(nq):
        p = i + nk - nq
        row = set()
        for j in range(nk):
            in_win = (left < 0 or j >= p - left) and (right < 0 or j <= p + right)
            ok = in_win or j < g or p < g
            if bm is not None and not bm[i // bq][j // bk]:
                ok = False
            if causal and j > p:
                ok = False
            if ok:
                row.add(j)
        out.append(row)
    return out


@pytest.mark.parametrize("seed", range(12))
def test_eligibility_matches_set_arithmetic(seed):
    rng = np.random.default_rng(seed)
    nk = int(rng.integers(1, 40))
    nq = int(rng.integers(1, nk + 5))
    causal = bool(rng.integers(0, 2))
    left = int(rng.integers(-1, 9))
    right = int(rng.integers(-1, 9))
    g = int(rng.integers(0, 4))
    bq, bk = int(rng.integers(1, 6)), int(rng.integers(1, 6))
    bm = rng.integers(0, 2, size=(-(-nq // bq), -(-nk // bk))) if seed % 3 else None
    got = dense.sparse_eligibility(nq, nk, causal, left, right, g, bm, bq, bk)
    want = _brute_eligible(nq, nk, causal, left, right, g, None if bm is None else bm.tolist(), bq, bk)
    for i in range(nq):
        assert set(np.nonzero(got[i])[0].tolist()) == want[i], (i, seed)


@pytest.mark.parametrize("n,w,g", [(100, 16, 0), (100, 16, 5), (64, 64, 3), (50, 1, 0), (30, 40, 2), (80, 8, 12)])
def test_causal_window_with_globals_pair_count_closed_form(n, w, g):
    """Causal window of w keys (left = w - 1) united with g global tokens:
    row i < g sees i + 1 keys; row i >= g sees min(i+1, w) window keys plus
    the g global keys, minus the global keys already inside the window."""
    m = dense.sparse_eligibility(n, n, causal=True, left=w - 1, n_global=g)
    want = 0
    for i in range(n):
        if i < g:
            want += i + 1
        else:
            lo = max(0, i - w + 1)
            want += min(i + 1, w) + g - max(0, g - lo)
    assert int(m.sum()) == want


def test_noncausal_band_pair_count_closed_form():
    n, left, right = 90, 7, 3
    m = dense.sparse_eligibility(n, n, left=left, right=right)
    want = sum(min(n - 1, i + right) - max(0, i - left) + 1 for i in range(n))
    assert int(m.sum()) == want


@pytest.mark.parametrize("causal", [False, True])
def test_unrestricted_is_dense(causal):
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 2, 40, 8)) for _ in range(3))
    o, lse = dense.attention_sparse(q, k, v, 0.4, causal)
    qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
    o_ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=0.4).numpy()
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)


def test_one_key_window_returns_own_value():
    """Causal window of one key: O_i = v_i and lse_i = scale * q_i . k_i."""
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, 1, 30, 6)) for _ in range(3))
    o, lse = dense.attention_sparse(q, k, v, 0.7, causal=True, left=0)
    np.testing.assert_allclose(o[0, 0], v[0, 0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], 0.7 * np.einsum("nd,nd->n", q[0, 0], k[0, 0]), rtol=1e-13, atol=1e-14)


def test_block_diagonal_mask_is_independent_block_attention():
    """Only diagonal 16x16 blocks active (non-causal): each block of rows is
    ordinary attention over its own 16 keys (torch SDPA per block)."""
    rng = np.random.default_rng(5)
    n, bs = 64, 16
    q, k, v = (rng.standard_normal((1, 2, n, 8)) for _ in range(3))
    bm = np.eye(n // bs, dtype=np.uint8)
    o, lse = dense.attention_sparse(q, k, v, 0.5, block_mask=bm, block_q=bs, block_k=bs)
    for a in range(0, n, bs):
        qt, kt, vt = (torch.from_numpy(x[:, :, a:a + bs]) for x in (q, k, v))
        o_ref = F.scaled_dot_product_attention(qt, kt, vt, scale=0.5).numpy()
        lse_ref = torch.logsumexp(0.5 * qt @ kt.transpose(-1, -2), dim=-1).numpy()
        np.testing.assert_allclose(o[:, :, a:a + bs], o_ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, a:a + bs], lse_ref, rtol=1e-12, atol=1e-13)


def test_window_globals_blocks_vs_sdpa_mask_gqa():
    """All restrictions at once, grouped heads, per-head block masks: torch
    SDPA with the same boolean mask on repeated KV heads (rows that keep at
    least one key), exact empty rows otherwise."""
    rng = np.random.default_rng(6)
    n, hq, hkv = 96, 4, 2
    q = rng.standard_normal((2, hq, n, 8))
    k, v = (rng.standard_normal((2, hkv, n, 8)) for _ in range(2))
    bm = rng.integers(0, 2, size=(hq, n // 32, n // 16)).astype(np.uint8)
    bm[1, 1, :] = 0                                   # head 1, rows 32..63: no active block
    o, lse = dense.attention_sparse(q, k, v, 0.5, causal=True, left=20, n_global=3, block_mask=bm,
                                    block_q=32, block_k=16)
    kt = torch.from_numpy(k).repeat_interleave(2, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(2, dim=1)
    for h in range(hq):
        allowed = torch.from_numpy(dense.sparse_eligibility(n, n, True, 20, -1, 3, bm[h], 32, 16))
        ne = allowed.any(dim=1)
        qt = torch.from_numpy(q[:, h:h + 1])
        o_ref = F.scaled_dot_product_attention(qt[:, :, ne], kt[:, h:h + 1], vt[:, h:h + 1],
                                               attn_mask=allowed[ne], scale=0.5).numpy()
        s = (0.5 * qt[:, :, ne] @ kt[:, h:h + 1].transpose(-1, -2)).masked_fill(~allowed[ne], -math.inf)
        np.testing.assert_allclose(o[:, h:h + 1, ne.numpy()], o_ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[:, h:h + 1, ne.numpy()], torch.logsumexp(s, -1).numpy(), rtol=1e-12)
        assert np.all(o[:, h, ~ne.numpy()] == 0.0) and np.all(lse[:, h, ~ne.numpy()] == -np.inf)
    assert (~dense.sparse_eligibility(n, n, True, 20, -1, 3, bm[1], 32, 16)[32:64]).all()


def test_shared_block_mask_equals_per_head_copies():
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((1, 3, 64, 4)) for _ in range(3))
    bm = rng.integers(0, 2, size=(2, 4)).astype(np.uint8)
    a = dense.attention_sparse(q, k, v, 0.5, block_mask=bm, block_q=32, block_k=16)
    b = dense.attention_sparse(q, k, v, 0.5, block_mask=np.stack([bm] * 3), block_q=32, block_k=16)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_rows_subset_matches_full():
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((1, 2, 50, 4)) for _ in range(3))
    o, lse = dense.attention_sparse(q, k, v, 0.5, causal=True, left=6, n_global=2)
    rows = np.array([[[0, 9, 49]] * 2])
    o2, l2 = dense.attention_sparse(q, k, v, 0.5, causal=True, left=6, n_global=2, rows=rows)
    np.testing.assert_array_equal(o2, o[:, :, [0, 9, 49]])
    np.testing.assert_array_equal(l2, lse[:, :, [0, 9, 49]])

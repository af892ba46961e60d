"""Float64 gradients of exact softmax attention (numpy). TEST INFRASTRUCTURE ONLY.

For the scalar loss L = sum(dO * O), the vector-Jacobian product of
O = softmax(S) V with S = scale * Q K^T over the eligible keys, written from
the softmax row derivative without forming a Jacobian ("Intermediate and
advanced extension", workshop table, softmax-backward row; "Attention
algorithms and data movement", lesson 03: differentiate the normalized row,
probabilities recomputed from the saved normalization state):

    P     = softmax over eligible keys of S (masked entries are 0)
    dV    = P^T dO
    dP    = dO V^T
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)          (the softmax row VJP)
    dQ    = scale * dS K
    dK    = scale * dS^T Q

An empty row (no eligible key) has P = 0 and contributes nothing. With
grouped heads (lesson 05, shared gradients) the gradient of a KV head is the
sum over the query heads that read it, KV head h // (Hq / Hkv).
"""
import numpy as np

from oracle.dense import NEG_INF


def attention_backward(q, k, v, do, scale, causal=False, allowed=None):
    """One head. q, do: [Nq, D]; k, v: [Nk, D] float64. Query i sits at
    position i + (Nk - Nq) (equal lengths: i), and causal keeps key j iff
    j <= that position ("Attention algorithms and data movement", lessons 04
    and 05, bottom-right alignment). ``allowed`` [Nq, Nk] (optional) restricts
    the eligible pairs further. Returns dq, dk, dv."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    n = q.shape[0]
    s = scale * (q @ k.T)
    if causal:
        # query i sits at position i + (Nk - Nq): the last Nq tokens of the keys
        pos = np.arange(n) + (k.shape[0] - n)
        s = np.where(np.arange(k.shape[0])[None, :] <= pos[:, None], s, NEG_INF)
    if allowed is not None:
        s = np.where(np.asarray(allowed, dtype=bool), s, NEG_INF)
    m = s.max(axis=1, keepdims=True) if s.size else np.zeros((n, 1))
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    denom = e.sum(axis=1, keepdims=True)
    p = np.where(denom > 0, e / np.where(denom > 0, denom, 1.0), 0.0)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_backward_bhnd(q, k, v, do, scale, causal=False):
    """q, do: [B, Hq, N, D]; k, v: [B, Hkv, N, D]. Returns dq [B, Hq, N, D]
    and dk, dv [B, Hkv, N, D], the latter summed over each KV head's query
    heads in ascending head order."""
    b_, hq = q.shape[0], q.shape[1]
    hkv = k.shape[1]
    group = hq // hkv
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(b_):
        for h in range(hq):
            g = h // group
            a, bk, bv = attention_backward(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal)
            dq[b, h] = a
            dk[b, g] += bk
            dv[b, g] += bv
    return dq, dk, dv


def attention_backward_varlen(q, k, v, do, cu_seqlens, scale, causal=True):
    """Packed variable-length grouped-query gradients. q, do: [T, Hq, D];
    k, v: [T, Hkv, D]; sequence s owns tokens [cu[s], cu[s+1]) and sees only
    its own keys, causal by position within the sequence ("Attention
    algorithms and data movement", lesson 04); query head h reads KV head
    h // (Hq / Hkv), whose gradients sum over its query heads in ascending
    order (lesson 05). Returns dq [T, Hq, D], dk and dv [T, Hkv, D]; tokens of
    empty sequences contribute nothing."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    hq, hkv = q.shape[1], k.shape[1]
    group = hq // hkv
    cu = [int(x) for x in cu_seqlens]
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b == a:
            continue
        for h in range(hq):
            g = h // group
            x, y, z = attention_backward(q[a:b, h], k[a:b, g], v[a:b, g], do[a:b, h], scale, causal)
            dq[a:b, h] = x
            dk[a:b, g] += y
            dv[a:b, g] += z
    return dq, dk, dv


def attention_backward_sparse_bhnd(q, k, v, do, scale, causal=False, left=-1, right=-1, n_global=0,
                                   block_mask=None, block_q=64, block_k=64):
    """Gradients of the sparse operator (window, global tokens, block mask;
    "Attention algorithms and data movement", lessons 06 and 07) on equal
    lengths: q, do [B, Hq, N, D]; k, v [B, Hkv, N, D]; block_mask None,
    [nqb, nkb] shared by every query head, or [Hq, nqb, nkb]. Eligibility is
    ``dense.sparse_eligibility`` with Nq = Nk; rows with no eligible key
    contribute nothing. KV-head gradients sum their query heads in order."""
    from oracle.dense import sparse_eligibility
    b_, hq, n = q.shape[0], q.shape[1], q.shape[2]
    hkv = k.shape[1]
    group = hq // hkv
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for h in range(hq):
        bm = None
        if block_mask is not None:
            bm = np.asarray(block_mask)
            bm = bm[h] if bm.ndim == 3 else bm
        allowed = sparse_eligibility(n, n, causal, left, right, n_global, bm, block_q, block_k)
        g = h // group
        for b in range(b_):
            x, y, z = attention_backward(q[b, h], k[b, g], v[b, g], do[b, h], scale, False, allowed)
            dq[b, h] = x
            dk[b, g] += y
            dv[b, g] += z
    return dq, dk, dv


def attention_backward_cache_bhnd(q, k, v, do, scale, causal=False):
    """q, do: [B, Hq, Nq, D]; k, v: [B, Hkv, Nk, D], queries at positions
    i + (Nk - Nq). Returns dq and dk, dv (summed over each KV head's query
    heads in ascending order); queries with no eligible key contribute
    nothing."""
    b_, hq = q.shape[0], q.shape[1]
    group = hq // k.shape[1]
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(b_):
        for h in range(hq):
            g = h // group
            x, y, z = attention_backward(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal)
            dq[b, h] = x
            dk[b, g] += y
            dv[b, g] += z
    return dq, dk, dv

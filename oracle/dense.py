"""Dense float64 attention oracle (numpy). TEST INFRASTRUCTURE ONLY.

What it computes follows the plain definition of exact softmax attention that
the pages centre on ("Attention algorithms and data movement", module header:
exact tiled attention; "Intermediate and advanced extension", workshop table,
streaming-attention row). The pages print no formula, so the reading is the
standard one:

    S_ij   = scale * <q_i, k_j>                  for eligible keys j
    m_i    = max_j S_ij
    l_i    = sum_j exp(S_ij - m_i)
    O_i    = sum_j exp(S_ij - m_i) v_j / l_i
    lse_i  = m_i + ln(l_i)                        (natural log)

Causal eligibility (equal query/key lengths): key j is eligible for the query
at logical position p iff j <= p, so the diagonal is included (the key at the
query's own position counts; "Logic review before implementation"). A row with
no eligible key is the empty row: O = 0, lse = -inf, never NaN (lesson 01 of
"Attention algorithms and data movement" asks for an explicit empty-row
contract; the values 0 / -inf are the reading taken here).

All inputs are float64 arrays that already hold the exact values of the stored
fp16/bf16 tensors; ``scale`` is the float32-rounded scale the GPU receives.
Rows are processed in blocks only to bound memory; no other reordering.
"""
import numpy as np

NEG_INF = -np.inf


def attention(q, k, v, scale, causal=False, q_pos=None, row_block=512):
    """Single-head dense attention.

    q: [Nq, D], k: [Nk, D], v: [Nk, Dv] float64.
    causal: key j is eligible for query i iff j <= q_pos[i]; q_pos defaults
    to arange(Nq) (equal-length self-attention, diagonal included).
    Returns (o [Nq, Dv], lse [Nq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    o = np.zeros((nq, v.shape[1]), dtype=np.float64)
    lse = np.full((nq,), NEG_INF, dtype=np.float64)
    if nq == 0 or nk == 0:
        return o, lse
    if q_pos is None:
        q_pos = np.arange(nq)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    key_idx = np.arange(nk)
    for r0 in range(0, nq, row_block):
        r1 = min(nq, r0 + row_block)
        s = scale * (q[r0:r1] @ k.T)                       # [rows, Nk]
        if causal:
            eligible = key_idx[None, :] <= q_pos[r0:r1, None]
            s = np.where(eligible, s, NEG_INF)
        m = s.max(axis=1)                                    # row maximum
        nonempty = np.isfinite(m)
        m_safe = np.where(nonempty, m, 0.0)
        p = np.exp(s - m_safe[:, None])                      # exp(-inf) = 0
        l = p.sum(axis=1)
        num = p @ v
        with np.errstate(invalid="ignore", divide="ignore"):
            o_blk = num / np.where(nonempty, l, 1.0)[:, None]
            lse_blk = m_safe + np.log(np.where(nonempty, l, 1.0))
        o[r0:r1] = np.where(nonempty[:, None], o_blk, 0.0)
        lse[r0:r1] = np.where(nonempty, lse_blk, NEG_INF)
    return o, lse


def attention_bhnd(q, k, v, scale, causal=False, rows=None):
    """Batched multi-head attention on [B, H, N, D] arrays (equal lengths for
    causal). ``rows`` optionally restricts the computed query rows: an int
    array [B, H, R] of row indices (logical positions); returns o [B,H,R,D]
    and lse [B,H,R] for those rows only. Without it all rows are returned."""
    b_, h_ = q.shape[0], q.shape[1]
    if rows is None:
        o = np.zeros(q.shape[:3] + (v.shape[3],), dtype=np.float64)
        lse = np.zeros(q.shape[:3], dtype=np.float64)
        for b in range(b_):
            for h in range(h_):
                o[b, h], lse[b, h] = attention(q[b, h], k[b, h], v[b, h], scale, causal)
        return o, lse
    rows = np.asarray(rows)
    o = np.zeros((b_, h_, rows.shape[2], v.shape[3]), dtype=np.float64)
    lse = np.zeros((b_, h_, rows.shape[2]), dtype=np.float64)
    for b in range(b_):
        for h in range(h_):
            r = rows[b, h]
            o[b, h], lse[b, h] = attention(q[b, h][r], k[b, h], v[b, h], scale, causal, q_pos=r)
    return o, lse


def varlen_gqa(q, k, v, cu_seqlens, scale, causal=True, rows=None):
    """Packed variable-length grouped-query attention.

    q: [T, Hq, D]; k, v: [T, Hkv, D]; cu_seqlens: [S+1] prefix offsets of the
    packed sequences (cu[0] = 0, cu[S] = T). Sequence s owns tokens
    [cu[s], cu[s+1]); its tokens attend only to keys of the same sequence, and
    causal eligibility uses logical positions within the sequence
    ("Attention algorithms and data movement", lesson 04). Query head h reads
    KV head h // (Hq / Hkv) (lesson 05, GQA head mapping).

    Returns o [T, Hq, D] and lse [Hq, T]. ``rows`` (optional) is a dict
    {(s, h): array of within-sequence positions}; then only those rows are
    computed and the result is a dict {(s, h): (o [R, D], lse [R])}.
    """
    t_, hq = q.shape[0], q.shape[1]
    hkv = k.shape[1]
    assert hq % hkv == 0
    group = hq // hkv
    cu = [int(x) for x in cu_seqlens]
    if rows is not None:
        out = {}
        for (s, h), r in rows.items():
            a, b = cu[s], cu[s + 1]
            g = h // group
            r = np.asarray(r, dtype=np.int64)
            out[(s, h)] = attention(q[a + r, h], k[a:b, g], v[a:b, g], scale, causal, q_pos=r)
        return out
    o = np.zeros((t_, hq, v.shape[2]), dtype=np.float64)
    lse = np.full((hq, t_), NEG_INF, dtype=np.float64)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        for h in range(hq):
            g = h // group
            o[a:b, h], lse[h, a:b] = attention(q[a:b, h], k[a:b, g], v[a:b, g], scale, causal)
    return o, lse


def cache_positions(nq, nk):
    """Logical positions of Nq queries that are the last Nq tokens of a
    sequence whose keys/values (the cache) hold Nk positions: query i sits at
    i + (Nk - Nq) (bottom-right alignment). Lesson 04 of "Attention
    algorithms and data movement" asks for unequal-length alignment derived
    from logical positions but prints no rule; this is the reading used here.
    With Nq > Nk the first Nq - Nk queries sit before position 0."""
    return np.arange(nq, dtype=np.int64) + (nk - nq)


def attention_cache(q, k, v, scale, causal=False, rows=None):
    """Queries against a key/value cache of another length, grouped heads.

    q: [B, Hq, Nq, D]; k, v: [B, Hkv, Nk, D]. Query head h reads KV head
    h // (Hq / Hkv) (lesson 05, GQA head mapping; the cache holds Hkv heads).
    Causal eligibility: key j is eligible for query i iff
    j <= i + (Nk - Nq) (``cache_positions``); a query with no eligible key is
    the empty row (O = 0, lse = -inf). Non-causal queries see all Nk keys.
    ``rows``: optional int array [B, Hq, R] of query indices; then only those
    rows are computed. Returns o [B, Hq, Nq or R, Dv] and lse [B, Hq, Nq or R].
    """
    b_, hq, nq = q.shape[0], q.shape[1], q.shape[2]
    hkv, nk = k.shape[1], k.shape[2]
    assert hq % hkv == 0
    group = hq // hkv
    pos = cache_positions(nq, nk)
    r_count = nq if rows is None else np.asarray(rows).shape[2]
    o = np.zeros((b_, hq, r_count, v.shape[3]), dtype=np.float64)
    lse = np.full((b_, hq, r_count), NEG_INF, dtype=np.float64)
    for b in range(b_):
        for h in range(hq):
            g = h // group
            r = np.arange(nq) if rows is None else np.asarray(rows)[b, h]
            o[b, h], lse[b, h] = attention(q[b, h][r], k[b, g], v[b, g], scale, causal, q_pos=pos[r])
    return o, lse


def split_partials(q, k, v, scale, chunk, causal=False, q_pos=None):
    """Unnormalized per-chunk partial states of attention.

    Keys are split into consecutive chunks [c*chunk, min(Nk, (c+1)*chunk)).
    For each query row i and chunk c (the partial-statistics stage of the
    split structure in "Intermediate and advanced extension", workshop table,
    split-softmax row, applied to attention), over the eligible keys j of c:

        m_ic   = max_{j in c} S_ij
        l_ic   = sum_{j in c} exp(S_ij - m_ic)
        acc_ic = sum_{j in c} exp(S_ij - m_ic) v_j       (not divided by l)

    Causal: key j is eligible for row i iff j <= q_pos[i] (q_pos defaults to
    ``cache_positions(Nq, Nk)``). A chunk with no eligible key for a row gives
    that row the empty state m = -inf, l = 0, acc = 0, the element that
    leaves any other state unchanged when merged with it (lesson 01).

    q: [Nq, D], k, v: [Nk, D]. Returns m [Nq, C], l [Nq, C], acc [Nq, C, Dv].
    """
    nq, nk = q.shape[0], k.shape[0]
    nchunk = -(-nk // chunk)
    if q_pos is None:
        q_pos = cache_positions(nq, nk)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    m = np.full((nq, nchunk), NEG_INF)
    l = np.zeros((nq, nchunk))
    acc = np.zeros((nq, nchunk, v.shape[1]))
    for c in range(nchunk):
        j0, j1 = c * chunk, min(nk, (c + 1) * chunk)
        s = scale * (q @ k[j0:j1].T)
        if causal:
            s = np.where(np.arange(j0, j1)[None, :] <= q_pos[:, None], s, NEG_INF)
        mc = s.max(axis=1)
        nonempty = np.isfinite(mc)
        p = np.exp(s - np.where(nonempty, mc, 0.0)[:, None])   # exp(-inf) = 0
        m[:, c] = mc
        l[:, c] = p.sum(axis=1)
        acc[:, c, :] = p @ v[j0:j1]
    return m, l, acc


def merge_partials(m, l, acc):
    """Combine partial states into the normalized output and logsumexp.

    m, l: [..., C]; acc: [..., C, Dv]. With M = max_c m_c and weights
    w_c = exp(m_c - M) (w_c = 0 for an empty partial, m_c = -inf):

        L = sum_c w_c l_c,   O = sum_c w_c acc_c / L,   lse = M + ln L.

    The partials are weighted by their rescaled denominators, never averaged
    ("Attention algorithms and data movement", lesson 01). A row whose
    partials are all empty gives O = 0 and lse = -inf.
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    acc = np.asarray(acc, dtype=np.float64)
    big_m = m.max(axis=-1)
    nonempty = np.isfinite(big_m)
    m0 = np.where(nonempty, big_m, 0.0)
    w = np.where(np.isfinite(m), np.exp(m - m0[..., None]), 0.0)
    big_l = (w * l).sum(axis=-1)
    num = (w[..., None] * acc).sum(axis=-2)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = num / np.where(nonempty, big_l, 1.0)[..., None]
        lse = m0 + np.log(np.where(nonempty, big_l, 1.0))
    o = np.where(nonempty[..., None], o, 0.0)
    lse = np.where(nonempty, lse, NEG_INF)
    return o, lse


def sparse_eligibility(nq, nk, causal=False, left=-1, right=-1, n_global=0, block_mask=None, block_q=64,
                       block_k=64):
    """Element eligibility [Nq, Nk] of the changed (sparse) operators, for
    queries at positions i + (Nk - Nq) (``cache_positions``).

    Window and global tokens ("Attention algorithms and data movement",
    lesson 07; the rule is the reading taken here): key j is eligible for the
    query at position p iff it lies in the window p - left <= j <= p + right
    (a negative bound is unlimited), or j < n_global (a global key, visible
    to every query), or p < n_global (a global query sees every key). The
    three sets are united, so a pair is counted once however many of them
    hold it.
    Block sparsity (lesson 06): block_mask [nqb, nkb] (nonzero = active)
    keeps pair (i, j) only if block (i // block_q, j // block_k) is active;
    the mask rows are indexed by query index i, not by position.
    Causal: additionally j <= p. All conditions are intersected.
    """
    p = cache_positions(nq, nk)[:, None]
    j = np.arange(nk)[None, :]
    win = np.ones((nq, nk), dtype=bool)
    if left >= 0:
        win &= j >= p - left
    if right >= 0:
        win &= j <= p + right
    ok = win | (j < n_global) | (p < n_global)
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        ok &= bm[np.arange(nq)[:, None] // block_q, j // block_k]
    if causal:
        ok &= j <= p
    return ok


def attention_allowed(q, k, v, scale, allowed):
    """Softmax attention of one head over an explicit eligibility mask
    ``allowed`` [Nq, Nk]; a row with no eligible key is the empty row
    (O = 0, lse = -inf). The plain definition with the mask applied."""
    nq = q.shape[0]
    o = np.zeros((nq, v.shape[1]), dtype=np.float64)
    lse = np.full((nq,), NEG_INF, dtype=np.float64)
    if nq == 0 or k.shape[0] == 0:
        return o, lse
    s = np.where(allowed, scale * (q @ k.T), NEG_INF)
    m = s.max(axis=1)
    nonempty = np.isfinite(m)
    m_safe = np.where(nonempty, m, 0.0)
    p = np.exp(s - m_safe[:, None])
    l = p.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        o_all = (p @ v) / np.where(nonempty, l, 1.0)[:, None]
        lse_all = m_safe + np.log(np.where(nonempty, l, 1.0))
    o[nonempty] = o_all[nonempty]
    lse[nonempty] = lse_all[nonempty]
    return o, lse


def attention_sparse(q, k, v, scale, causal=False, left=-1, right=-1, n_global=0, block_mask=None, block_q=64,
                     block_k=64, rows=None):
    """The matching sparse reference: exact softmax attention restricted to
    ``sparse_eligibility`` (lessons 06 and 07: a changed operator, not an
    approximation of dense attention).

    q: [B, Hq, Nq, D]; k, v: [B, Hkv, Nk, D], KV head h // (Hq / Hkv).
    block_mask: None, [nqb, nkb] (every head) or [Hq, nqb, nkb] (per query
    head). ``rows``: optional [B, Hq, R] query indices. Returns o, lse as
    ``attention_cache``.
    """
    b_, hq, nq = q.shape[0], q.shape[1], q.shape[2]
    hkv, nk = k.shape[1], k.shape[2]
    group = hq // hkv
    bm = None if block_mask is None else np.asarray(block_mask)
    r_count = nq if rows is None else np.asarray(rows).shape[2]
    o = np.zeros((b_, hq, r_count, v.shape[3]), dtype=np.float64)
    lse = np.full((b_, hq, r_count), NEG_INF, dtype=np.float64)
    masks = {}
    for h in range(hq):
        key = 0 if (bm is None or bm.ndim == 2) else h
        if key not in masks:
            masks[key] = sparse_eligibility(nq, nk, causal, left, right, n_global,
                                            None if bm is None else (bm if bm.ndim == 2 else bm[h]),
                                            block_q, block_k)
    for b in range(b_):
        for h in range(hq):
            g = h // group
            allowed = masks[0 if (bm is None or bm.ndim == 2) else h]
            r = np.arange(nq) if rows is None else np.asarray(rows)[b, h]
            o[b, h], lse[b, h] = attention_allowed(q[b, h][r], k[b, g], v[b, g], scale, allowed[r])
    return o, lse

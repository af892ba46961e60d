"""GPU parity: the HIP path (through the C ABI) against the FP64 oracle.

Inputs come from the seeded generators in ``workloads``; expected values come
only from ``oracle``. Small cases are compared in full (several tiles and a
ragged tail); the full-size workloads are compared on seeded samples of rows
the oracle computes one by one.
"""
import hashlib

import numpy as np
import pytest
import torch

import workloads as W
from exact_tiled_attention_sattn_amd import (sattn_fwd, sattn_fwd_split, sattn_merge, sattn_fwd_varlen,
                                             sattn_fwd_cache, sattn_fwd_split_cache, sattn_fwd_strided,
                                             sattn_fwd_sparse, sattn_bwd, sattn_bwd_cache, sattn_bwd_varlen, sattn_bwd_sparse,
                                             SattnError)
from oracle import dense
from tests.parity import check_attention, check_o, check_lse, TOL, grad_bounds, check_grad

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _banner(*a):
    print("[case]", *a, flush=True)


def _dense_inputs(b, h, n, d, dtype, seed, qmul=1.0):
    q, k, v = W.qkv((b, h, n, d), (b, h, n, d), dtype, seed)
    if qmul != 1.0:
        q = (q.float() * qmul).to(q.dtype)   # power of two: exact
    return q, k, v


def _run_fwd(q, k, v, causal, scale):
    o, lse = sattn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


# ------------------------------------------------------------ dense, small
SMALL = [
    # (B, H, N, D, dtype)
    (1, 1, 1, 32, "fp16"), (1, 1, 2, 64, "bf16"), (1, 2, 31, 128, "bf16"), (2, 3, 65, 32, "fp16"),
    (1, 2, 127, 64, "bf16"), (1, 1, 129, 128, "fp16"), (2, 2, 200, 64, "fp16"), (1, 3, 333, 128, "bf16"),
    (1, 1, 257, 32, "bf16"), (1, 2, 513, 128, "fp16"),
    # many heads: D <= 64 problems that take the streaming kernel rather than
    # the small-problem kernel (more than 256 workgroups of 32 rows)
    (4, 16, 300, 64, "fp16"), (2, 40, 200, 32, "bf16"),
    # ... and with long key walks (18 key tiles, ragged)
    (2, 8, 1100, 64, "bf16"), (2, 8, 1100, 32, "fp16"),
]


@pytest.mark.parametrize("b,h,n,d,dt", SMALL)
@pytest.mark.parametrize("causal", [False, True])
def test_dense_small_full(b, h, n, d, dt, causal):
    _banner("dense", b, h, n, d, dt, causal)
    q, k, v = _dense_inputs(b, h, n, d, dt, seed=1000 + n + d + h)
    scale = W.scale_f32(d)
    o, lse = _run_fwd(q, k, v, causal, scale)
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal)
    check_attention(o, lse, o_ref, lse_ref, W.DTYPES[dt], "dense")


def test_c1_single_head_129x32_fp16_causal():
    cfg = W.WORKLOADS["single_head_129x32_fp16_causal"]
    _banner("129x32 fp16 causal")
    q, k, v = _dense_inputs(1, 1, 129, 32, "fp16", cfg["seed"])
    scale = W.scale_f32(32)
    o, lse = _run_fwd(q, k, v, True, scale)
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, True)
    check_attention(o, lse, o_ref, lse_ref, torch.float16, "129x32")


@pytest.mark.parametrize("qmul", [1.0, 16.0])
@pytest.mark.parametrize("causal", [True, False])
def test_c2_single_head_512x64_fp16(causal, qmul):
    cfg = W.WORKLOADS["single_head_512x64_fp16"]
    _banner("512x64 fp16", causal, qmul)
    q, k, v = _dense_inputs(1, 1, 512, 64, "fp16", cfg["seed"], qmul)
    scale = W.scale_f32(64)
    o, lse = _run_fwd(q, k, v, causal, scale)
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal)
    check_attention(o, lse, o_ref, lse_ref, torch.float16, "512x64")


@pytest.mark.parametrize("causal", [True, False])
def test_c3_batched_4x16x4096x128_bf16_sampled(causal):
    cfg = W.WORKLOADS["batched_4x16x4096x128_bf16"]
    _banner("4x16x4096x128 bf16", causal)
    b, h, n, d = 4, 16, 4096, 128
    q, k, v = _dense_inputs(b, h, n, d, "bf16", cfg["seed"])
    scale = W.scale_f32(d)
    o, lse = _run_fwd(q, k, v, causal, scale)
    rows = W.sample_rows(cfg["seed"], n, cfg["sampled_rows_per_head"], groups=b * h).reshape(b, h, -1)
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal, rows=rows)
    idx = torch.from_numpy(rows)
    o_s = torch.stack([torch.stack([o[i, j].cpu()[idx[i, j]] for j in range(h)]) for i in range(b)])
    lse_s = torch.stack([torch.stack([lse[i, j].cpu()[idx[i, j]] for j in range(h)]) for i in range(b)])
    check_attention(o_s, lse_s, o_ref, lse_ref, torch.bfloat16, "4096x128")
    # every row written and finite (outputs were fresh torch.empty)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


# Causal grids large enough that workgroups take query-tile pairs (j,
# nqt-1-j), with an odd tile count (the middle tile runs once) and a ragged
# last tile: 256-row tiles at D = 128, 64-row tiles at D = 64.
PAIRED = [(1, 205, 1270, 128, "bf16"), (1, 34, 1940, 64, "fp16")]


@pytest.mark.parametrize("b,h,n,d,dt", PAIRED)
def test_causal_paired_tiles_sampled(b, h, n, d, dt):
    _banner("paired causal", b, h, n, d, dt)
    seed = 4000 + n
    q, k, v = _dense_inputs(b, h, n, d, dt, seed)
    scale = W.scale_f32(d)
    o, lse = _run_fwd(q, k, v, True, scale)
    rows = W.sample_rows(seed, n, 24, groups=b * h).reshape(b, h, -1)
    # rows around tile edges too: the middle tile and the last (ragged) one
    edge = np.array([0, 255, 256, 511, 512, 767, 768, 1023, 1024, n - 2, n - 1])
    edge = edge[edge < n]
    rows = np.sort(np.concatenate([rows, np.broadcast_to(edge, (b, h, edge.size))], axis=2), axis=2)
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, True, rows=rows)
    idx = torch.from_numpy(rows)
    oc, lc = o.cpu(), lse.cpu()
    o_s = torch.stack([torch.stack([oc[i, j][idx[i, j]] for j in range(h)]) for i in range(b)])
    lse_s = torch.stack([torch.stack([lc[i, j][idx[i, j]] for j in range(h)]) for i in range(b)])
    check_attention(o_s, lse_s, o_ref, lse_ref, W.DTYPES[dt], "paired causal")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


# ------------------------------------------------------- closed form on GPU
@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_zero_q_gives_mean_of_values(dt):
    """Q = 0: every eligible score is 0, P = 1 exactly; O_i = mean(V[0..i])
    causal, lse_i = ln(i+1)."""
    _banner("zero-q", dt)
    n, d = 300, 64
    _, k, v = _dense_inputs(1, 1, n, d, dt, seed=77)
    q = torch.zeros_like(k)
    o, lse = _run_fwd(q, k, v, True, 0.125)
    vv = W.to_f64(v)[0, 0]
    ref = np.cumsum(vv, axis=0) / np.arange(1, n + 1)[:, None]
    check_o(o[0, 0], ref, W.DTYPES[dt], "zero-q o")
    check_lse(lse[0, 0], np.log(np.arange(1, n + 1)), "zero-q lse")


# ------------------------------------------------------------ invariants
def test_causal_future_perturbation_bitwise():
    _banner("future perturbation")
    n, d = 512, 64
    q, k, v = _dense_inputs(1, 2, n, d, "fp16", seed=2)
    o0, l0 = _run_fwd(q, k, v, True, 0.125)
    for j in (1, 64, 65, 300, 511):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, j] = 30.0
        v2[:, :, j] = -500.0
        o1, l1 = _run_fwd(q, k2, v2, True, 0.125)
        assert torch.equal(o1[:, :, :j], o0[:, :, :j]), j
        assert torch.equal(l1[:, :, :j], l0[:, :, :j]), j
        assert not torch.equal(o1[:, :, j:], o0[:, :, j:])


def test_deterministic_bitwise_and_inputs_preserved():
    _banner("determinism")
    q, k, v = (x.to(DEV) for x in _dense_inputs(2, 4, 700, 128, "bf16", seed=9))
    digest = [hashlib.sha256(x.cpu().view(torch.int16).numpy().tobytes()).hexdigest() for x in (q, k, v)]
    a = sattn_fwd(q, k, v, causal=True)
    b = sattn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    after = [hashlib.sha256(x.cpu().view(torch.int16).numpy().tobytes()).hexdigest() for x in (q, k, v)]
    assert after == digest


def test_fresh_outputs_overwritten_and_nondefault_stream():
    _banner("fresh outputs / stream")
    q, k, v = (x.to(DEV) for x in _dense_inputs(1, 3, 257, 64, "fp16", seed=10))
    ref = sattn_fwd(q, k, v, causal=False)
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sattn_fwd(q, k, v, causal=False, out=out, lse=lse)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])


def test_alias_rejected_on_device():
    q, k, v = (x.to(DEV) for x in _dense_inputs(1, 1, 64, 64, "fp16", seed=11))
    with pytest.raises(SattnError, match="ALIAS"):
        sattn_fwd(q, k, v, out=q)


# ---------------------------------------------------------------- split
SPLIT_SMALL = [
    # (B, Hq, Hkv, Nq, Nk, D, chunk, dtype); Hq > Hkv with Nq <= 64 packs a
    # KV head's query heads into one slice
    (1, 2, 2, 1, 100, 128, 32, "bf16"),
    (2, 4, 1, 1, 4096, 128, 1024, "bf16"),
    (1, 4, 2, 3, 777, 64, 256, "fp16"),
    (1, 1, 1, 40, 130, 32, 64, "fp16"),
    (1, 2, 1, 1, 50, 128, 4096, "bf16"),       # one chunk larger than Nk
    (1, 1, 1, 2, 65, 64, 1, "bf16"),           # one key per chunk
    # one query row per slice (the vector-unit row kernel): ragged last
    # chunks, chunks too short to give every wave keys, one key per chunk
    (2, 3, 3, 1, 1000, 32, 96, "fp16"),
    (1, 2, 2, 1, 777, 64, 200, "bf16"),
    (1, 1, 1, 1, 5, 128, 4096, "fp16"),
    (1, 2, 2, 1, 300, 128, 1, "bf16"),
    (1, 2, 2, 1, 4099, 128, 1030, "fp16"),
    # one query row per head, 2, 4 or 8 query heads per KV head: the group's
    # rows packed into one slice
    (1, 8, 2, 1, 999, 64, 200, "fp16"),
    (2, 4, 2, 1, 333, 32, 64, "bf16"),
    (1, 8, 1, 1, 500, 128, 128, "bf16"),
]


@pytest.mark.parametrize("b,hq,hkv,nq,nk,d,chunk,dt", SPLIT_SMALL)
def test_split_partials_and_merge_small(b, hq, hkv, nq, nk, d, chunk, dt):
    _banner("split", b, hq, hkv, nq, nk, d, chunk, dt)
    q, k, v = W.qkv((b, hq, nq, d), (b, hkv, nk, d), dt, seed=2000 + nk)
    scale = W.scale_f32(d)
    pm, pl, pa = sattn_fwd_split(q.to(DEV), k.to(DEV), v.to(DEV), chunk, scale)
    o, lse = sattn_merge(pm, pl, pa, W.DTYPES[dt])
    torch.cuda.synchronize()
    qf, kf, vf = W.to_f64(q), W.to_f64(k), W.to_f64(v)
    g = hq // hkv
    pm_, pl_, pa_ = (x.cpu().double().numpy() for x in (pm, pl, pa))
    for bb in range(b):
        for h in range(hq):
            m_ref, l_ref, a_ref = dense.split_partials(qf[bb, h], kf[bb, h // g], vf[bb, h // g], scale, chunk)
            # each partial: its max, its logsumexp and its normalized output
            np.testing.assert_allclose(pm_[bb, h], m_ref, rtol=0, atol=1e-3)
            check_lse(pm_[bb, h] + np.log(pl_[bb, h]), m_ref + np.log(l_ref), "partial lse")
            check_o(pa_[bb, h] / pl_[bb, h][..., None], a_ref / l_ref[..., None], W.DTYPES[dt], "partial o")
            o_ref, lse_ref = dense.attention(qf[bb, h], kf[bb, h // g], vf[bb, h // g], scale)
            check_attention(o[bb, h], lse[bb, h], o_ref, lse_ref, W.DTYPES[dt], "merged")


@pytest.mark.parametrize("d,dt,hq,hkv", [(128, "bf16", 2, 2), (64, "fp16", 2, 2), (128, "bf16", 8, 2)])
def test_split_row_large_logits(d, dt, hq, hkv):
    """One query row per head with Q x 16 (score spread of about 16 nats):
    the running maximum changes many times within a chunk, for a query head
    alone (the row kernel) and for four sharing a KV head (packed)."""
    _banner("split row large logits", d, dt, hq, hkv)
    q, k, v = W.qkv((2, hq, 1, d), (2, hkv, 3000, d), dt, seed=2600 + d + hq)
    q = q * 16
    scale = W.scale_f32(d)
    chunk = 512
    pm, pl, pa = sattn_fwd_split(q.to(DEV), k.to(DEV), v.to(DEV), chunk, scale)
    o, lse = sattn_merge(pm, pl, pa, W.DTYPES[dt])
    torch.cuda.synchronize()
    qf, kf, vf = W.to_f64(q), W.to_f64(k), W.to_f64(v)
    pm_, pl_, pa_ = (x.cpu().double().numpy() for x in (pm, pl, pa))
    g = hq // hkv
    for bb in range(2):
        for h in range(hq):
            m_ref, l_ref, a_ref = dense.split_partials(qf[bb, h], kf[bb, h // g], vf[bb, h // g], scale, chunk)
            np.testing.assert_allclose(pm_[bb, h], m_ref, rtol=0, atol=1e-3 * max(1.0, np.abs(m_ref).max()))
            check_lse(pm_[bb, h] + np.log(pl_[bb, h]), m_ref + np.log(l_ref), "partial lse")
            check_o(pa_[bb, h] / pl_[bb, h][..., None], a_ref / l_ref[..., None], W.DTYPES[dt], "partial o")
            o_ref, lse_ref = dense.attention(qf[bb, h], kf[bb, h // g], vf[bb, h // g], scale)
            check_attention(o[bb, h], lse[bb, h], o_ref, lse_ref, W.DTYPES[dt], "merged")


def test_split_matches_fwd():
    _banner("split vs fwd")
    q, k, v = (x.to(DEV) for x in _dense_inputs(1, 4, 1000, 128, "bf16", seed=12))
    o1, l1 = sattn_fwd(q, k, v, causal=False)
    pm, pl, pa = sattn_fwd_split(q, k, v, 256)
    o2, l2 = sattn_merge(pm, pl, pa, torch.bfloat16)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    assert (o1.float() - o2.float()).abs().max().item() <= tol[0] + tol[1]
    assert (l1 - l2).abs().max().item() <= 1e-3


@pytest.mark.parametrize("d", [32, 64, 128])
def test_merge_many_chunks(d):
    """150 partials per row (the weights are taken 64 chunks at a time and
    the partial rows loaded 16 at a time): a row with every partial empty but
    the last, one with a whole group of 64 empty, and rows whose maximum sits
    in the last, ragged group."""
    _banner("merge many chunks", d)
    rows, c = 9, 150
    g = torch.Generator().manual_seed(150 + d)
    pm = torch.randn(rows, c, generator=g) * 4
    pl = torch.rand(rows, c, generator=g) * 50 + 1
    pa = torch.randn(rows, c, d, generator=g) * 3
    pm[0, :-1] = -float("inf"); pl[0, :-1] = 0; pa[0, :-1] = 0
    pm[1, 64:128] = -float("inf"); pl[1, 64:128] = 0; pa[1, 64:128] = 0
    pm[2:5, 140] += 20.0
    o, lse = sattn_merge(pm.to(DEV), pl.to(DEV), pa.to(DEV), torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, lse_ref = dense.merge_partials(pm.double().numpy(), pl.double().numpy(), pa.double().numpy())
    check_attention(o, lse, o_ref, lse_ref, torch.bfloat16, "merge many chunks")


def test_merge_empty_partials_identity():
    """Empty partials (m=-inf, l=0, acc=0) change nothing; all-empty rows give
    O = 0, lse = -inf."""
    _banner("merge empty")
    rows, c, d = 5, 6, 128
    g = torch.Generator().manual_seed(13)
    pm = torch.randn(rows, c, generator=g) * 3
    pl = torch.rand(rows, c, generator=g) * 10 + 1
    pa = torch.randn(rows, c, d, generator=g) * 5
    pm[1, 2] = -float("inf"); pl[1, 2] = 0; pa[1, 2] = 0
    pm[3, :] = -float("inf"); pl[3, :] = 0; pa[3, :] = 0
    o, lse = sattn_merge(pm.to(DEV), pl.to(DEV), pa.to(DEV), torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, lse_ref = dense.merge_partials(pm.double().numpy(), pl.double().numpy(), pa.double().numpy())
    check_attention(o, lse, o_ref, lse_ref, torch.bfloat16, "merge")
    assert torch.equal(o[3].float().cpu(), torch.zeros(d)) and lse[3].item() == -float("inf")


def test_c4_splitkv_decode_all_rows():
    """16x32 query rows, 131072 keys each, 4096-key chunks: every one of the
    512 merged rows against the oracle, each row's q, K and V slices (64 MiB)
    streamed to the host in turn."""
    cfg = W.WORKLOADS["splitkv_decode_16x32x131072x128_bf16"]
    _banner("decode 16x32x131072x128 bf16, all rows")
    b, hq, hkv, nk, d, chunk = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["Nk"], cfg["D"], cfg["chunk"]
    g = torch.Generator(device=DEV)
    g.manual_seed(cfg["seed"])
    q = W.randn_device_sliced((b, hq, 1, d), "bf16", g, DEV)
    k = W.randn_device_sliced((b, hkv, nk, d), "bf16", g, DEV)
    v = W.randn_device_sliced((b, hkv, nk, d), "bf16", g, DEV)
    scale = W.scale_f32(d)
    pm, pl, pa = sattn_fwd_split(q, k, v, chunk, scale)
    o, lse = sattn_merge(pm, pl, pa, torch.bfloat16)
    torch.cuda.synchronize()
    assert pm.shape == (b, hq, 1, 32)
    o_c, l_c = o.cpu(), lse.cpu()
    worst = 0.0
    for flat in range(b * hq):
        bb, h = divmod(flat, hq)
        o_ref, lse_ref = dense.attention(W.to_f64(q[bb, h]), W.to_f64(k[bb, h]), W.to_f64(v[bb, h]), scale)
        res = check_attention(o_c[bb, h], l_c[bb, h], o_ref, lse_ref, torch.bfloat16, "decode row %d" % flat)
        worst = max(worst, res["o_err_over_bound"])
    print("[decode] 512 rows, worst o err/bound %.3f" % worst, flush=True)
    del k, v
    torch.cuda.empty_cache()


# --------------------------------------------------------------- varlen
def _varlen_inputs(lengths, hq, hkv, d, dt, seed):
    t = int(sum(lengths))
    q, k, v = W.qkv((t, hq, d), (t, hkv, d), dt, seed)
    cu = W.cu_seqlens_of(lengths)
    return q, k, v, cu


VARLEN_SMALL = [
    # (lengths, Hq, Hkv, D, dtype, causal)
    ([5, 1, 130, 64], 4, 1, 128, "bf16", True),
    ([200, 0, 33], 8, 2, 64, "fp16", True),
    ([1], 2, 2, 32, "fp16", True),
    ([300, 129, 7], 4, 4, 128, "bf16", False),
    ([64, 64, 65], 32, 8, 128, "bf16", True),
]


@pytest.mark.parametrize("lengths,hq,hkv,d,dt,causal", VARLEN_SMALL)
def test_varlen_small_full(lengths, hq, hkv, d, dt, causal):
    _banner("varlen", lengths, hq, hkv, d, dt, causal)
    q, k, v, cu = _varlen_inputs(lengths, hq, hkv, d, dt, seed=3000 + sum(lengths))
    scale = W.scale_f32(d)
    o, lse = sattn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(cu), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = dense.varlen_gqa(W.to_f64(q), W.to_f64(k), W.to_f64(v), cu, scale, causal)
    check_attention(o, lse, o_ref, lse_ref, W.DTYPES[dt], "varlen")


def test_varlen_gqa_equals_expanded_heads_bitwise():
    _banner("gqa vs expanded")
    q, k, v, cu = _varlen_inputs([100, 37], 8, 2, 128, "bf16", seed=14)
    cu_t = torch.from_numpy(cu)
    o1, l1 = sattn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_t)
    ke = k.repeat_interleave(4, dim=1).contiguous()
    ve = v.repeat_interleave(4, dim=1).contiguous()
    o2, l2 = sattn_fwd_varlen(q.to(DEV), ke.to(DEV), ve.to(DEV), cu_t)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_varlen_cross_sequence_isolation_bitwise():
    _banner("cross-sequence")
    lengths = [150, 90, 200]
    q, k, v, cu = _varlen_inputs(lengths, 4, 2, 64, "fp16", seed=15)
    cu_t = torch.from_numpy(cu)
    o0, l0 = sattn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_t)
    a, b = int(cu[1]), int(cu[2])
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[a:b] = 3.0
    k2[a:b] = -2.0
    v2[a:b] = 100.0
    o1, l1 = sattn_fwd_varlen(q2.to(DEV), k2.to(DEV), v2.to(DEV), cu_t)
    torch.cuda.synchronize()
    for x, y in ((0, a), (b, int(cu[3]))):
        assert torch.equal(o1[x:y], o0[x:y]) and torch.equal(l1[:, x:y], l0[:, x:y])


def test_varlen_matches_dense_per_sequence_bitwise():
    """A packed sequence gives the same bits as the batched kernel on it."""
    _banner("varlen vs dense")
    q, k, v, cu = _varlen_inputs([257], 4, 4, 128, "bf16", seed=16)
    o1, l1 = sattn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(cu))
    qd, kd, vd = (x.permute(1, 0, 2)[None].contiguous().to(DEV) for x in (q, k, v))
    o2, l2 = sattn_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[0].permute(1, 0, 2)) and torch.equal(l1, l2[0])


def test_c5_varlen_gqa_full_size_sampled():
    cfg = W.WORKLOADS["varlen_gqa_8seq_32q8kv_128_bf16_causal"]
    lengths = W.varlen_lengths(cfg["seed"], cfg["S"], cfg["max_len"])
    _banner("varlen gqa full", lengths.tolist())
    hq, hkv, d = cfg["Hq"], cfg["Hkv"], cfg["D"]
    q, k, v, cu = _varlen_inputs(lengths, hq, hkv, d, "bf16", cfg["seed"])
    scale = W.scale_f32(d)
    o, lse = sattn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(cu), causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    rows = {}
    for s, L in enumerate(lengths):
        for h in range(hq):
            rows[(s, h)] = W.sample_rows(cfg["seed"] * 1000 + s * 64 + h, int(L), 16)[0]
    ref = dense.varlen_gqa(W.to_f64(q), W.to_f64(k), W.to_f64(v), cu, scale, True, rows=rows)
    o_c, l_c = o.cpu(), lse.cpu()
    for (s, h), r in rows.items():
        t = int(cu[s]) + torch.from_numpy(r)
        check_attention(o_c[t, h], l_c[h, t], ref[(s, h)][0], ref[(s, h)][1], torch.bfloat16,
                        "seq %d head %d" % (s, h))


def test_varlen_bad_table_rejected_by_binding():
    q, k, v, cu = _varlen_inputs([10, 10], 2, 1, 64, "bf16", seed=17)
    bad = torch.tensor([0, 12, 20], dtype=torch.int32)
    with pytest.raises(ValueError):
        sattn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), bad, max_seqlen=10)


# ------------------------------------------------- fixed-reference fast path
def _growth_inputs(n, d, dt, jump, seed):
    """q = 1; k_j constant along d: 0 for the first 64 keys, `jump` after, so
    every row's score grows by sqrt(D)*jump after the first key tile."""
    g = torch.Generator().manual_seed(seed)
    q = torch.ones((1, 2, n, d), dtype=W.DTYPES[dt])
    k = torch.zeros((1, 2, n, d), dtype=torch.float32)
    k[:, :, 64:, :] = jump
    k = k.to(W.DTYPES[dt])
    v = torch.randn((1, 2, n, d), generator=g).to(W.DTYPES[dt])
    return q, k, v


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("jump", [0.25, 3.0, 50.0])
def test_score_growth_after_first_tile(dt, causal, jump):
    """Scores grow after the first key tile by sqrt(D)*jump*scale: jump 0.25
    is 2^4 in exp2 units (absorbed by the fixed reference in both dtypes);
    jump 3 is 2^49, absorbed for bf16 but past the fp16 range of the rounded
    P, so fp16 takes the exact online update; jump 50: the tile sums overflow
    and both take it. All must match the oracle."""
    _banner("growth", dt, causal, jump)
    n, d = 300, 128
    q, k, v = _growth_inputs(n, d, dt, jump, seed=21)
    scale = W.scale_f32(d)
    o, lse = _run_fwd(q, k, v, causal, scale)
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal)
    check_attention(o, lse, o_ref, lse_ref, W.DTYPES[dt], "growth")


@pytest.mark.parametrize("causal", [False, True])
def test_huge_values_under_score_growth(causal):
    """bf16 values of magnitude ~1e25 with every score growing by 2^50 after
    the first key tile: the tile sums stay under the fixed-reference limit,
    but p*v would overflow the fp32 numerator; the workgroup must take the
    exact update and return the finite result."""
    _banner("huge values", causal)
    n, d = 300, 128
    q, k, v = _growth_inputs(n, d, "bf16", 3.0625, seed=25)
    # positive values: a causal row that sees two keys of opposite sign would
    # otherwise test the cancellation of 1e25-sized terms, not the fallback
    v = ((v.float().abs() + 0.5) * 1e25).to(torch.bfloat16)
    scale = W.scale_f32(d)
    o, lse = _run_fwd(q, k, v, causal, scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal)
    check_attention(o, lse, o_ref, lse_ref, torch.bfloat16, "huge values")


@pytest.mark.parametrize("causal", [False, True])
def test_large_logits_fp16_streaming_kernel(causal):
    """The large-logit variant (Q x 16, score spread ~16) on an fp16 shape
    that takes the streaming kernel (more than 256 workgroups of 32 rows):
    later tiles exceed the first tile's max by far more than the fp16 range
    of the rounded P allows under the fixed reference."""
    _banner("large logits fp16", causal)
    q, k, v = _dense_inputs(1, 16, 1024, 64, "fp16", seed=23, qmul=16.0)
    scale = W.scale_f32(64)
    o, lse = _run_fwd(q, k, v, causal, scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal)
    check_attention(o, lse, o_ref, lse_ref, torch.float16, "large logits fp16")


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("step", [1.0, 5.0])
def test_score_growth_in_steps(dt, causal, step):
    """Scores rise by sqrt(D)*step*scale every 256 keys (q = 1, k constant
    along d), so on the streaming kernel rows outgrow their reference
    several times during the walk: step 1 (16 in exp2 units) exceeds the
    fp16 limit at each rise, step 5 (82) the bf16 limit too. Every redone
    tile must still match the oracle."""
    _banner("growth steps", dt, causal, step)
    n, d = 1500, 128
    g = torch.Generator().manual_seed(29)
    q = torch.ones((1, 2, n, d), dtype=W.DTYPES[dt])
    k = (step * (torch.arange(n) // 256).float())[None, None, :, None].expand(1, 2, n, d).to(W.DTYPES[dt])
    k = k.contiguous()
    v = torch.randn((1, 2, n, d), generator=g).to(W.DTYPES[dt])
    scale = W.scale_f32(d)
    o, lse = _run_fwd(q, k, v, causal, scale)
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal)
    check_attention(o, lse, o_ref, lse_ref, W.DTYPES[dt], "growth steps")


def test_redone_tiles_keep_rows_independent_bitwise():
    """Large logits (Q x 16, fp16, D = 128) make waves redo many tiles; a
    future key j perturbed so that it forces a redo for the rows that see it
    must leave every earlier causal row bit-identical (the rows sharing a
    wave with them recompute the same bits)."""
    _banner("redo rows independent")
    n, d = 1100, 128
    q, k, v = _dense_inputs(1, 2, n, d, "fp16", seed=31, qmul=16.0)
    scale = W.scale_f32(d)
    o0, l0 = _run_fwd(q, k, v, True, scale)
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, True)
    check_attention(o0, l0, o_ref, lse_ref, torch.float16, "large logits")
    for j in (70, 300, 517, 1000):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, j] = (q[:, :, j].float() * 0.25).to(torch.float16)   # score at key j jumps for row j
        v2[:, :, j] = -500.0
        o1, l1 = _run_fwd(q, k2, v2, True, scale)
        assert torch.equal(o1[:, :, :j], o0[:, :, :j]), j
        assert torch.equal(l1[:, :, :j], l0[:, :, :j]), j
        assert not torch.equal(o1[:, :, j:], o0[:, :, j:])
        if j == 517:
            o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k2), W.to_f64(v2), scale, True)
            check_attention(o1, l1, o_ref, lse_ref, torch.float16, "perturbed key %d" % j)


# Many heads at D = 128 (more query tiles than CUs, so a CU runs several
# workgroups in turn): key-tile counts per query tile even, odd and one;
# causal pairs with and without a repeated middle tile. Some heads force the
# exact-update rerun while the other workgroups take the fixed reference.
# Outputs start as NaN, so every row must be written.
MANY_HEADS = [(300, 200, False), (300, 150, False), (300, 60, False), (512, 300, True), (1100, 150, True)]


@pytest.mark.parametrize("h,n,causal", MANY_HEADS)
def test_many_heads_with_rerun_heads(h, n, causal):
    _banner("many heads", h, n, causal)
    d = 128
    q, k, v = _dense_inputs(1, h, n, d, "bf16", seed=5000 + h + n)
    grow = [hh for hh in (3, h // 2, h - 1)] if n > 64 else []
    for hh in grow:                         # tile sums overflow the fixed reference
        q[:, hh] = 1.0
        k[:, hh, :64] = 0.0
        k[:, hh, 64:] = 50.0
    scale = W.scale_f32(d)
    o = torch.full((1, h, n, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((1, h, n), float("nan"), dtype=torch.float32, device=DEV)
    sattn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    heads = sorted({x for x in (0, 1, 2, 7, 255, 256, 257, h - 2) + tuple(grow) if 0 <= x < h})
    hs = torch.tensor(heads)
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q[:, hs]), W.to_f64(k[:, hs]), W.to_f64(v[:, hs]), scale, causal)
    check_attention(o[:, hs.to(DEV)].cpu(), lse[:, hs.to(DEV)].cpu(), o_ref, lse_ref, torch.bfloat16, "many heads")


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("jump", [3.0, 50.0])
def test_score_growth_varlen_fallback(dt, jump):
    """The first sequence's scores grow after its first key tile: by 2^49 in
    exp2 units (jump 3: the fixed reference for bf16, the exact update for
    fp16) or far past the tile-sum limit (jump 50: the exact update)."""
    _banner("growth varlen", dt, jump)
    lengths = [200, 130]
    t = sum(lengths)
    g = torch.Generator().manual_seed(22)
    q = torch.ones((t, 4, 128), dtype=W.DTYPES[dt])
    k = torch.zeros((t, 2, 128), dtype=torch.float32)
    k[64:200] = jump
    k = k.to(W.DTYPES[dt])
    v = torch.randn((t, 2, 128), generator=g).to(W.DTYPES[dt])
    cu = W.cu_seqlens_of(lengths)
    o, lse = sattn_fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(cu), causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = dense.varlen_gqa(W.to_f64(q), W.to_f64(k), W.to_f64(v), cu, W.scale_f32(128), True)
    check_attention(o, lse, o_ref, lse_ref, W.DTYPES[dt], "growth varlen")


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq", [100, 600])
def test_score_growth_cache(dt, causal, nq):
    """Queries against a cache whose keys after the first tile raise every
    score by 2^49 in exp2 units: fp16 must leave the fixed reference (its
    rounded P would overflow), bf16 keeps it. 600 queries take the 256-row
    workgroups."""
    _banner("growth cache", dt, causal, nq)
    nk, d = 700, 128
    g = torch.Generator().manual_seed(24)
    q = torch.ones((1, 4, nq, d), dtype=W.DTYPES[dt])
    k = torch.zeros((1, 2, nk, d), dtype=torch.float32)
    k[:, :, 64:] = 3.0
    k = k.to(W.DTYPES[dt])
    v = torch.randn((1, 2, nk, d), generator=g).to(W.DTYPES[dt])
    scale = W.scale_f32(d)
    o, lse = sattn_fwd_cache(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = dense.attention_cache(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal)
    check_attention(o, lse, o_ref, lse_ref, W.DTYPES[dt], "growth cache")


# ------------------------------------------------- queries against a K/V cache
CACHE_SMALL = [
    # (B, Hq, Hkv, Nq, Nk, D, dtype)
    (1, 2, 1, 1, 300, 128, "bf16"),      # one decode query
    (1, 4, 2, 37, 300, 64, "fp16"),      # a prefill chunk, ragged tiles
    (2, 4, 4, 129, 129, 32, "bf16"),     # equal lengths
    (1, 2, 1, 200, 70, 128, "bf16"),     # more queries than cache: empty rows
    (1, 8, 2, 300, 1000, 128, "fp16"),   # several tiles both ways, 4 heads per KV head
    (1, 2, 2, 5, 0, 64, "bf16"),         # empty cache
    # long chunks at D = 128 take 256-row workgroups
    (1, 4, 2, 700, 1500, 128, "bf16"),   # ragged tiles, 2 heads per KV head
    (1, 2, 1, 600, 300, 128, "fp16"),    # more queries than cache: empty rows
]


def _cache_run(b, hq, hkv, nq, nk, d, dt, causal, seed):
    q, k, v = W.qkv((b, hq, nq, d), (b, hkv, nk, d), dt, seed)
    scale = W.scale_f32(d)
    o, lse = sattn_fwd_cache(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return q, k, v, scale, o, lse


@pytest.mark.parametrize("b,hq,hkv,nq,nk,d,dt", CACHE_SMALL)
@pytest.mark.parametrize("causal", [False, True])
def test_cache_small_full(b, hq, hkv, nq, nk, d, dt, causal):
    _banner("cache", b, hq, hkv, nq, nk, d, dt, causal)
    q, k, v, scale, o, lse = _cache_run(b, hq, hkv, nq, nk, d, dt, causal, seed=5000 + nq + nk)
    o_ref, lse_ref = dense.attention_cache(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal)
    check_attention(o, lse, o_ref, lse_ref, W.DTYPES[dt], "cache")


def test_cache_empty_rows_exact():
    """Queries before the cache: O is exactly 0 and lse exactly -inf."""
    _banner("cache empty rows")
    _, _, _, _, o, lse = _cache_run(1, 2, 1, 300, 44, 128, "bf16", True, seed=5101)
    assert torch.count_nonzero(o[:, :, :256].float()).item() == 0
    assert bool((lse[:, :, :256] == -float("inf")).all())
    assert torch.isfinite(lse[:, :, 256:]).all()


def test_cache_equal_lengths_matches_fwd_bitwise():
    """Nq = Nk with one KV head per query head gives each row the same
    arithmetic as sattn_fwd (same 64-key tiles in the same order; the
    workgroups differ in size only): bitwise equal."""
    _banner("cache == fwd")
    q, k, v = (x.to(DEV) for x in _dense_inputs(1, 3, 700, 128, "bf16", seed=5102))
    for causal in (False, True):
        o1, l1 = sattn_fwd(q, k, v, causal=causal)
        o2, l2 = sattn_fwd_cache(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), causal


def test_cache_future_perturbation_bitwise():
    """Changing cache position j leaves every query at a position before j
    bitwise unchanged (bottom-right alignment)."""
    _banner("cache future perturbation")
    nq, nk = 200, 500
    q, k, v = W.qkv((1, 4, nq, 128), (1, 2, nk, 128), "bf16", 5103)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    o0, l0 = sattn_fwd_cache(q, k, v, causal=True)
    for j in (300, 301, 364, 499):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, j] = 30.0
        v2[:, :, j] = -500.0
        o1, l1 = sattn_fwd_cache(q, k2, v2, causal=True)
        i = j - (nk - nq)          # first query whose position is >= j
        assert torch.equal(o1[:, :, :i], o0[:, :, :i]) and torch.equal(l1[:, :, :i], l0[:, :, :i]), j
        assert not torch.equal(o1[:, :, i:], o0[:, :, i:])


def test_cache_chunked_prefill_sampled():
    """A 2048-token chunk against a 16384-token cache, 32 query heads on 8
    KV heads, bf16 causal: sampled rows per head, edges included."""
    _banner("chunked prefill 2048 vs 16384")
    b, hq, hkv, nq, nk, d = 1, 32, 8, 2048, 16384, 128
    q, k, v, scale, o, lse = _cache_run(b, hq, hkv, nq, nk, d, "bf16", True, seed=5104)
    rows = W.sample_rows(5104, nq, 16, groups=b * hq).reshape(b, hq, -1)
    o_ref, lse_ref = dense.attention_cache(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, True, rows=rows)
    idx = torch.from_numpy(rows)
    oc, lc = o.cpu(), lse.cpu()
    o_s = torch.stack([torch.stack([oc[0, h][idx[0, h]] for h in range(hq)])])
    l_s = torch.stack([torch.stack([lc[0, h][idx[0, h]] for h in range(hq)])])
    check_attention(o_s, l_s, o_ref, lse_ref, torch.bfloat16, "chunked prefill")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


SPLIT_CACHE_SMALL = [
    # (B, Hq, Hkv, Nq, Nk, D, chunk, dtype)
    (1, 4, 1, 1, 1000, 128, 256, "bf16"),    # causal decode: equals non-causal
    (1, 2, 2, 16, 700, 128, 128, "bf16"),    # a few queries: last chunk partly eligible
    (1, 2, 1, 300, 260, 64, 64, "fp16"),     # more queries than keys: empty rows
    (2, 2, 1, 70, 70, 32, 16, "fp16"),       # equal lengths, many empty chunks
    # grouped heads packed into one slice per KV head (Nq <= 64): rows of
    # several query heads share a tile and repeat the same positions
    (1, 8, 2, 5, 333, 128, 64, "bf16"),
    (2, 6, 2, 40, 500, 64, 128, "fp16"),     # 120 rows per slice over two 64-row tiles
    (1, 4, 1, 64, 64, 32, 32, "bf16"),       # every row's own chunk cut at its position
    (1, 2, 2, 1, 300, 64, 64, "bf16"),       # one row per slice (the row kernel), causal
]


@pytest.mark.parametrize("b,hq,hkv,nq,nk,d,chunk,dt", SPLIT_CACHE_SMALL)
def test_split_cache_causal_partials_and_merge(b, hq, hkv, nq, nk, d, chunk, dt):
    _banner("split cache causal", b, hq, hkv, nq, nk, d, chunk, dt)
    q, k, v = W.qkv((b, hq, nq, d), (b, hkv, nk, d), dt, seed=6000 + nq + nk)
    scale = W.scale_f32(d)
    pm, pl, pa = sattn_fwd_split_cache(q.to(DEV), k.to(DEV), v.to(DEV), chunk, causal=True, scale=scale)
    o, lse = sattn_merge(pm, pl, pa, W.DTYPES[dt])
    torch.cuda.synchronize()
    qf, kf, vf = W.to_f64(q), W.to_f64(k), W.to_f64(v)
    g = hq // hkv
    pm_, pl_, pa_ = (x.cpu().double().numpy() for x in (pm, pl, pa))
    o_ref, lse_ref = dense.attention_cache(qf, kf, vf, scale, True)
    check_attention(o, lse, o_ref, lse_ref, W.DTYPES[dt], "merged")
    for bb in range(b):
        for h in range(hq):
            m_ref, l_ref, a_ref = dense.split_partials(qf[bb, h], kf[bb, h // g], vf[bb, h // g], scale, chunk,
                                                       causal=True)
            empty = np.isinf(m_ref)
            # empty states exactly; the others by their max, logsumexp and output
            assert np.all(pm_[bb, h][empty] == -np.inf) and np.all(pl_[bb, h][empty] == 0.0)
            assert np.all(pa_[bb, h][empty] == 0.0)
            np.testing.assert_allclose(pm_[bb, h][~empty], m_ref[~empty], rtol=0, atol=1e-3)
            ok = ~empty
            check_lse(pm_[bb, h][ok] + np.log(pl_[bb, h][ok]), m_ref[ok] + np.log(l_ref[ok]), "partial lse")
            check_o(pa_[bb, h][ok] / pl_[bb, h][ok][..., None], a_ref[ok] / l_ref[ok][..., None],
                    W.DTYPES[dt], "partial o")


def test_split_cache_noncausal_is_split_bitwise():
    _banner("split cache noncausal == split")
    q, k, v = W.qkv((1, 4, 3, 128), (1, 2, 900, 128), "bf16", 6100)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    a = sattn_fwd_split(q, k, v, 256)
    b_ = sattn_fwd_split_cache(q, k, v, 256, causal=False)
    torch.cuda.synchronize()
    for x, y in zip(a, b_):
        assert torch.equal(x, y)


# ---------------------------------------------- strided, sliced, broadcast
def _strided_views(kind, b, hq, hkv, nq, nk, d, dt, seed):
    """Views q [B,Hq,Nq,D], k, v [B,Hkv,Nk,D] of the given layout kind (last
    dim contiguous), built on the GPU from seeded values."""
    g = torch.Generator().manual_seed(seed)
    rnd = lambda *s: W.randn(s, dt, g).to(DEV)  # noqa: E731
    if kind == "transposed":            # [B, N, H, D] storage
        q = rnd(b, nq, hq, d).permute(0, 2, 1, 3)
        k = rnd(b, nk, hkv, d).permute(0, 2, 1, 3)
        v = rnd(b, nk, hkv, d).permute(0, 2, 1, 3)
    elif kind == "sliced":              # the first D of a wider last dim; every other row
        q = rnd(b, hq, 2 * nq, d + 64)[:, :, ::2, :d]
        k = rnd(b, hkv, nk, d + 32)[..., 16:16 + d]
        v = rnd(b, hkv, nk, d + 32)[..., 16:16 + d]
    elif kind == "broadcast":           # one K/V for every batch entry, one q row set for every head
        q = rnd(b, 1, nq, d).expand(b, hq, nq, d)
        k = rnd(1, hkv, nk, d).expand(b, hkv, nk, d)
        v = rnd(1, hkv, nk, d).expand(b, hkv, nk, d)
    else:                               # packed qkv [B, N, 3, H, D] (Hq = Hkv)
        x = rnd(b, nq, 3, hq, d)
        q, k, v = (x[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    return q, k, v


STRIDED = [
    ("transposed", 2, 8, 2, 300, 300, 128, "bf16"),
    ("transposed", 1, 4, 4, 100, 257, 64, "fp16"),
    ("sliced", 1, 4, 2, 129, 400, 128, "fp16"),
    ("broadcast", 3, 4, 2, 70, 190, 64, "bf16"),
    ("packed", 2, 4, 4, 333, 333, 128, "bf16"),
    ("packed", 1, 2, 2, 65, 65, 32, "fp16"),
    ("transposed", 1, 4, 2, 600, 900, 128, "bf16"),   # a long chunk: 256-row workgroups
]


@pytest.mark.parametrize("kind,b,hq,hkv,nq,nk,d,dt", STRIDED)
@pytest.mark.parametrize("causal", [False, True])
def test_strided_inputs(kind, b, hq, hkv, nq, nk, d, dt, causal):
    _banner("strided", kind, b, hq, hkv, nq, nk, d, dt, causal)
    q, k, v = _strided_views(kind, b, hq, hkv, nq, nk, d, dt, seed=7000 + nq + d)
    assert not (q.is_contiguous() and k.is_contiguous())
    scale = W.scale_f32(d)
    q0, k0, v0 = (x.clone() for x in (q, k, v))
    o, lse = sattn_fwd_strided(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = dense.attention_cache(W.to_f64(q.cpu()), W.to_f64(k.cpu()), W.to_f64(v.cpu()), scale, causal)
    check_attention(o, lse, o_ref, lse_ref, W.DTYPES[dt], "strided " + kind)
    # inputs untouched; same bits as the dense-layout call on contiguous copies
    assert torch.equal(q, q0) and torch.equal(k, k0) and torch.equal(v, v0)
    o2, l2 = sattn_fwd_cache(q.contiguous(), k.contiguous(), v.contiguous(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)


# ----------------------------------------- sparse: windows, globals, blocks
SPARSE = [
    # (B, Hq, Hkv, Nq, Nk, D, dtype, causal, left, right, n_global, mask (heads, bq, bk) or None)
    (1, 4, 2, 600, 600, 128, "bf16", True, 100, -1, 0, None),       # causal sliding window
    (1, 2, 2, 700, 700, 64, "fp16", True, 64, -1, 5, None),         # window + global tokens
    (1, 2, 1, 300, 300, 128, "bf16", False, 40, 40, 3, None),       # band, global queries and keys
    (2, 4, 4, 512, 512, 128, "bf16", False, -1, -1, 0, (4, 64, 64)),  # per-head block mask
    (1, 4, 2, 1000, 1000, 64, "fp16", True, 300, -1, 0, (1, 128, 128)),  # shared mask + causal window
    (1, 2, 1, 200, 900, 128, "bf16", True, 256, -1, 0, None),       # cache alignment, Nq < Nk
    (1, 2, 2, 333, 333, 32, "fp16", True, 17, 2, 1, (2, 32, 64)),   # small blocks, ragged
    (1, 2, 1, 700, 700, 128, "fp16", True, 300, -1, 4, (2, 64, 128)),  # 64-row blocks: 64-row workgroups
    (1, 2, 2, 500, 800, 128, "bf16", True, -1, -1, 0, (1, 96, 64)),    # 96-row blocks, cache alignment
]


def _sparse_case(b, hq, hkv, nq, nk, d, dt, mask, seed):
    q, k, v = W.qkv((b, hq, nq, d), (b, hkv, nk, d), dt, seed)
    bm = None
    if mask is not None:
        heads, bq, bk = mask
        g = torch.Generator().manual_seed(seed)
        bm = torch.randint(0, 2, (heads, -(-nq // bq), -(-nk // bk)), generator=g, dtype=torch.uint8)
        bm[0, 1, :] = 0                   # one query block with no key at all: empty rows
    return q, k, v, bm


@pytest.mark.parametrize("b,hq,hkv,nq,nk,d,dt,causal,left,right,ng,mask", SPARSE)
def test_sparse_full(b, hq, hkv, nq, nk, d, dt, causal, left, right, ng, mask):
    _banner("sparse", b, hq, hkv, nq, nk, d, dt, causal, left, right, ng, mask)
    q, k, v, bm = _sparse_case(b, hq, hkv, nq, nk, d, dt, mask, seed=8000 + nq + d)
    scale = W.scale_f32(d)
    bq, bk = (mask[1], mask[2]) if mask else (64, 64)
    o, lse = sattn_fwd_sparse(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=(left, right), n_global=ng,
                              block_mask=None if bm is None else bm.to(DEV), block_q=bq, block_k=bk, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = dense.attention_sparse(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal, left, right, ng,
                                            None if bm is None else bm.numpy()[0] if bm.shape[0] == 1 else bm.numpy(),
                                            bq, bk)
    check_attention(o, lse, o_ref, lse_ref, W.DTYPES[dt], "sparse")


@pytest.mark.parametrize("causal,masked", [(True, False), (False, True)])
def test_sparse_longest_tile_list(causal, masked):
    """Nk = 65536, the longest key range a sparse workgroup can list (1024
    tiles): the last 160 queries of the cache with every tile kept (causal,
    no window), or about half of them kept by a random block mask with
    128-key blocks spread over the whole range."""
    _banner("sparse longest list", causal, masked)
    b, hq, hkv, nq, nk, d = 1, 2, 1, 160, 65536, 128
    q, k, v = W.qkv((b, hq, nq, d), (b, hkv, nk, d), "bf16", 8100 + int(causal))
    bm = None
    if masked:
        g = torch.Generator().manual_seed(8101)
        bm = torch.randint(0, 2, (hq, -(-nq // 64), nk // 128), generator=g, dtype=torch.uint8)
    scale = W.scale_f32(d)
    o, lse = sattn_fwd_sparse(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, n_global=0,
                              block_mask=None if bm is None else bm.to(DEV), block_q=64, block_k=128, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = dense.attention_sparse(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal, -1, -1, 0,
                                            None if bm is None else bm.numpy(), 64, 128)
    check_attention(o, lse, o_ref, lse_ref, torch.bfloat16, "sparse longest list")


def test_sparse_keys_outside_the_window_do_not_matter_bitwise():
    """Causal window of 128 keys: changing key j changes no row whose window
    does not contain it, bit for bit."""
    _banner("sparse window perturbation")
    n, w = 1000, 128
    q, k, v = (x.to(DEV) for x in W.qkv((1, 2, n, 128), (1, 2, n, 128), "bf16", 8100))
    o0, l0 = sattn_fwd_sparse(q, k, v, causal=True, window=(w - 1, -1))
    for j in (0, 300, 640):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, j] = 30.0
        v2[:, :, j] = -500.0
        o1, l1 = sattn_fwd_sparse(q, k2, v2, causal=True, window=(w - 1, -1))
        torch.cuda.synchronize()
        keep = torch.ones(n, dtype=torch.bool)
        keep[j:j + w] = False                      # rows j .. j+w-1 see key j
        assert torch.equal(o1[:, :, keep], o0[:, :, keep]) and torch.equal(l1[:, :, keep], l0[:, :, keep]), j
        assert not torch.equal(o1[:, :, ~keep], o0[:, :, ~keep])


# ------------------------------------------------------------- backward
def _check_grads(grads, refs, q, k, v, do, o, scale, causal, dtype, what=""):
    """grads/refs: (dq, dk, dv) for [B, Hq, N, D] / [B, Hkv, N, D]."""
    qf, kf, vf, dof, of = (W.to_f64(x.cpu()) for x in (q, k, v, do, o))
    b_, hq, hkv = qf.shape[0], qf.shape[1], kf.shape[1]
    grp = hq // hkv
    rel = [np.zeros(x.shape) for x in (qf, kf, vf)]
    und = [np.zeros(x.shape) for x in (qf, kf, vf)]
    for b in range(b_):
        for h in range(hq):
            g = h // grp
            r3, a3 = grad_bounds(qf[b, h], kf[b, g], vf[b, g], dof[b, h], of[b, h], scale, causal)
            for dst, src in ((rel, r3), (und, a3)):
                dst[0][b, h] = src[0]
                dst[1][b, g] += src[1]
                dst[2][b, g] += src[2]
    for i, (name, g, r) in enumerate(zip(("dq", "dk", "dv"), grads, refs)):
        check_grad(g, r, rel[i], und[i], dtype, what + name)


BWD_SMALL = [
    # (B, Hq, Hkv, N, D, dtype)
    (1, 1, 1, 1, 32, "fp16"),
    (1, 2, 2, 64, 64, "bf16"),
    (1, 2, 1, 100, 128, "bf16"),
    (2, 4, 2, 300, 64, "fp16"),
    (1, 3, 3, 257, 128, "bf16"),
    (1, 8, 2, 513, 128, "fp16"),
    (1, 2, 2, 200, 32, "bf16"),
]


@pytest.mark.parametrize("b,hq,hkv,n,d,dt", BWD_SMALL)
@pytest.mark.parametrize("causal", [False, True])
def test_backward_small_full(b, hq, hkv, n, d, dt, causal):
    _banner("backward", b, hq, hkv, n, d, dt, causal)
    from oracle import backward
    seed = 9000 + n + d + hq
    q, k, v = W.qkv((b, hq, n, d), (b, hkv, n, d), dt, seed)
    g = torch.Generator().manual_seed(seed + 1)
    do = W.randn((b, hq, n, d), dt, g)
    scale = W.scale_f32(d)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = sattn_fwd_cache(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = sattn_bwd(qd, kd, vd, o, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    refs = backward.attention_backward_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), W.to_f64(do), scale, causal)
    _check_grads((dq, dk, dv), refs, q, k, v, do, o, scale, causal, W.DTYPES[dt])


def _check_grads_varlen(grads, refs, q, k, v, do, o, cu, scale, causal, dtype, what="varlen "):
    """grads/refs: (dq, dk, dv) for [T, Hq, D] / [T, Hkv, D] packed tokens;
    per-element bounds from each (sequence, head) slice."""
    qf, kf, vf, dof, of = (W.to_f64(x.cpu()) for x in (q, k, v, do, o))
    hq, hkv = qf.shape[1], kf.shape[1]
    grp = hq // hkv
    rel = [np.zeros(x.shape) for x in (qf, kf, vf)]
    und = [np.zeros(x.shape) for x in (qf, kf, vf)]
    for a, e in zip(cu[:-1], cu[1:]):
        if e == a:
            continue
        for h in range(hq):
            g = h // grp
            r3, a3 = grad_bounds(qf[a:e, h], kf[a:e, g], vf[a:e, g], dof[a:e, h], of[a:e, h], scale, causal)
            for dst, src in ((rel, r3), (und, a3)):
                dst[0][a:e, h] = src[0]
                dst[1][a:e, g] += src[1]
                dst[2][a:e, g] += src[2]
    for i, (name, g, r) in enumerate(zip(("dq", "dk", "dv"), grads, refs)):
        check_grad(g, r, rel[i], und[i], dtype, what + name)


BWD_VARLEN = [
    # (lengths, Hq, Hkv, D, dtype)
    ([5, 0, 130, 1, 64], 4, 2, 128, "bf16"),       # an empty sequence, single tokens, tile edges
    ([300, 257], 2, 2, 64, "fp16"),
    ([200, 0, 77, 129], 8, 2, 32, "bf16"),
    ([513], 4, 1, 128, "fp16"),
]


@pytest.mark.parametrize("lengths,hq,hkv,d,dt", BWD_VARLEN)
@pytest.mark.parametrize("causal", [False, True])
def test_backward_varlen_full(lengths, hq, hkv, d, dt, causal):
    _banner("backward varlen", lengths, hq, hkv, d, dt, causal)
    from oracle import backward
    t = sum(lengths)
    cu = W.cu_seqlens_of(lengths)
    seed = 9300 + t + d + hq
    q, k, v = W.qkv((t, hq, d), (t, hkv, d), dt, seed)
    do = W.randn((t, hq, d), dt, torch.Generator().manual_seed(seed + 1))
    scale = W.scale_f32(d)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    cud = torch.from_numpy(cu).to(DEV)
    o, lse = sattn_fwd_varlen(qd, kd, vd, cud, causal=causal, scale=scale)
    nan = float("nan")
    dq, dk, dv = (torch.full_like(x, nan) for x in (qd, kd, vd))
    sattn_bwd_varlen(qd, kd, vd, o, dod, lse, cud, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    refs = backward.attention_backward_varlen(W.to_f64(q), W.to_f64(k), W.to_f64(v), W.to_f64(do), cu, scale,
                                              causal)
    _check_grads_varlen((dq, dk, dv), refs, q, k, v, do, o, [int(x) for x in cu], scale, causal, W.DTYPES[dt])


@pytest.mark.parametrize("causal", [False, True])
def test_backward_varlen_one_sequence_is_dense_bitwise(causal):
    """One packed sequence of length N is the dense [1, H, N, D] problem:
    same tiles, same sums in the same order, so the same bits."""
    _banner("backward varlen == dense", causal)
    n, hq, hkv, d = 777, 4, 2, 128
    q, k, v = (x.to(DEV) for x in W.qkv((n, hq, d), (n, hkv, d), "bf16", 9400))
    do = W.randn((n, hq, d), "bf16", torch.Generator().manual_seed(9401)).to(DEV)
    cu = torch.tensor([0, n], dtype=torch.int32, device=DEV)
    o, lse = sattn_fwd_varlen(q, k, v, cu, causal=causal)
    got = sattn_bwd_varlen(q, k, v, o, do, lse, cu, causal=causal)
    bh = lambda x: x.permute(1, 0, 2).unsqueeze(0).contiguous()      # [T, H, D] -> [1, H, T, D]
    want = sattn_bwd(bh(q), bh(k), bh(v), bh(o), bh(do), lse.unsqueeze(0).contiguous(), causal=causal)
    torch.cuda.synchronize()
    for g, w in zip(got, want):
        assert torch.equal(bh(g), w)


def test_backward_varlen_sequences_are_isolated_bitwise():
    """Changing every token of one sequence leaves the other sequences'
    gradients bit-identical."""
    _banner("backward varlen isolation")
    lengths = [300, 450, 200]
    t = sum(lengths)
    cu = torch.from_numpy(W.cu_seqlens_of(lengths)).to(DEV)
    q, k, v = (x.to(DEV) for x in W.qkv((t, 4, 64), (t, 2, 64), "fp16", 9500))
    do = W.randn((t, 4, 64), "fp16", torch.Generator().manual_seed(9501)).to(DEV)
    o, lse = sattn_fwd_varlen(q, k, v, cu)
    a = sattn_bwd_varlen(q, k, v, o, do, lse, cu)
    q2, k2, v2, do2 = (x.clone() for x in (q, k, v, do))
    for x in (q2, k2, v2, do2):
        x[300:750] = -x[300:750] * 0.5
    o2, lse2 = sattn_fwd_varlen(q2, k2, v2, cu)
    b_ = sattn_bwd_varlen(q2, k2, v2, o2, do2, lse2, cu)
    torch.cuda.synchronize()
    for x, y in zip(a, b_):
        assert torch.equal(x[:300], y[:300]) and torch.equal(x[750:], y[750:])
        assert not torch.equal(x[300:750], y[300:750])


BWD_SPARSE = [
    # (B, Hq, Hkv, N, D, dtype, causal, left, right, n_global, mask (heads, bq, bk) or None)
    (1, 4, 2, 600, 128, "bf16", True, 100, -1, 0, None),          # causal sliding window
    (1, 2, 2, 700, 64, "fp16", True, 64, -1, 5, None),            # window + global tokens
    (1, 2, 1, 300, 128, "bf16", False, 40, 40, 3, None),          # band, global queries and keys
    (2, 4, 4, 512, 128, "bf16", False, -1, -1, 0, (4, 64, 64)),   # per-head block mask, empty query block
    (1, 4, 2, 1000, 64, "fp16", True, 300, -1, 0, (1, 128, 128)),  # shared mask + causal window
    (1, 2, 2, 333, 32, "fp16", True, 17, 2, 1, (2, 32, 64)),      # small blocks, ragged
]


@pytest.mark.parametrize("b,hq,hkv,n,d,dt,causal,left,right,ng,mask", BWD_SPARSE)
def test_backward_sparse_full(b, hq, hkv, n, d, dt, causal, left, right, ng, mask):
    _banner("backward sparse", b, hq, hkv, n, d, dt, causal, left, right, ng, mask)
    from oracle import backward
    q, k, v, bm = _sparse_case(b, hq, hkv, n, n, d, dt, mask, seed=9600 + n + d)
    do = W.randn((b, hq, n, d), dt, torch.Generator().manual_seed(9601 + n))
    scale = W.scale_f32(d)
    bq, bk = (mask[1], mask[2]) if mask else (64, 64)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    bmd = None if bm is None else bm.to(DEV)
    o, lse = sattn_fwd_sparse(qd, kd, vd, causal=causal, window=(left, right), n_global=ng, block_mask=bmd,
                              block_q=bq, block_k=bk, scale=scale)
    nan = float("nan")
    dq, dk, dv = (torch.full_like(x, nan) for x in (qd, kd, vd))
    sattn_bwd_sparse(qd, kd, vd, o, dod, lse, causal=causal, window=(left, right), n_global=ng, block_mask=bmd,
                     block_q=bq, block_k=bk, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    bmn = None if bm is None else bm.numpy()
    refs = backward.attention_backward_sparse_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), W.to_f64(do), scale,
                                                   causal, left, right, ng,
                                                   bmn[0] if bmn is not None and bmn.shape[0] == 1 else bmn, bq, bk)
    qf, kf, vf, dof, of = (W.to_f64(x.cpu()) for x in (q, k, v, do, o))
    grp = hq // hkv
    rel = [np.zeros(x.shape) for x in (qf, kf, vf)]
    und = [np.zeros(x.shape) for x in (qf, kf, vf)]
    for h in range(hq):
        mh = None if bmn is None else (bmn[h] if bmn.shape[0] > 1 else bmn[0])
        allowed = dense.sparse_eligibility(n, n, causal, left, right, ng, mh, bq, bk).astype(np.float64)
        g = h // grp
        for bi in range(b):
            r3, a3 = grad_bounds(qf[bi, h], kf[bi, g], vf[bi, g], dof[bi, h], of[bi, h], scale, False, allowed)
            for dst, src in ((rel, r3), (und, a3)):
                dst[0][bi, h] = src[0]
                dst[1][bi, g] += src[1]
                dst[2][bi, g] += src[2]
    for i, (name, gr, r) in enumerate(zip(("dq", "dk", "dv"), (dq, dk, dv), refs)):
        check_grad(gr, r, rel[i], und[i], W.DTYPES[dt], "sparse " + name)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_sparse_unrestricted_is_dense_bitwise(causal):
    """No window, no global token, no mask: the same tiles and sums as the
    dense backward, so the same bits."""
    _banner("backward sparse == dense", causal)
    q, k, v = (x.to(DEV) for x in W.qkv((2, 4, 700, 128), (2, 2, 700, 128), "bf16", 9700))
    do = W.randn((2, 4, 700, 128), "bf16", torch.Generator().manual_seed(9701)).to(DEV)
    o, lse = sattn_fwd_cache(q, k, v, causal=causal)
    a = sattn_bwd_sparse(q, k, v, o, do, lse, causal=causal)
    b_ = sattn_bwd(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    for x, y in zip(a, b_):
        assert torch.equal(x, y)


BWD_CACHE = [
    # (B, Hq, Hkv, Nq, Nk, D, dtype, causal)
    (1, 4, 2, 100, 300, 128, "bf16", True),      # chunk at the end of a longer cache
    (1, 2, 2, 300, 100, 64, "fp16", True),       # more queries than keys: empty rows
    (2, 4, 1, 129, 700, 128, "bf16", False),
    (1, 2, 2, 1, 513, 64, "fp16", True),         # one decode query
    (1, 2, 1, 257, 257, 32, "bf16", True),       # equal lengths
]


@pytest.mark.parametrize("b,hq,hkv,nq,nk,d,dt,causal", BWD_CACHE)
def test_backward_cache_full(b, hq, hkv, nq, nk, d, dt, causal):
    _banner("backward cache", b, hq, hkv, nq, nk, d, dt, causal)
    from oracle import backward
    q, k, v = W.qkv((b, hq, nq, d), (b, hkv, nk, d), dt, 9800 + nq + nk)
    do = W.randn((b, hq, nq, d), dt, torch.Generator().manual_seed(9801 + nq))
    scale = W.scale_f32(d)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = sattn_fwd_cache(qd, kd, vd, causal=causal, scale=scale)
    nan = float("nan")
    dq, dk, dv = (torch.full_like(x, nan) for x in (qd, kd, vd))
    sattn_bwd_cache(qd, kd, vd, o, dod, lse, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    refs = backward.attention_backward_cache_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), W.to_f64(do), scale,
                                                  causal)
    allowed = np.ones((nq, nk))
    if causal:
        allowed = (np.arange(nk)[None, :] <= (np.arange(nq) + nk - nq)[:, None]).astype(np.float64)
    qf, kf, vf, dof, of = (W.to_f64(x.cpu()) for x in (q, k, v, do, o))
    grp = hq // hkv
    rel = [np.zeros(x.shape) for x in (qf, kf, vf)]
    und = [np.zeros(x.shape) for x in (qf, kf, vf)]
    for h in range(hq):
        g = h // grp
        for bi in range(b):
            r3, a3 = grad_bounds(qf[bi, h], kf[bi, g], vf[bi, g], dof[bi, h], of[bi, h], scale, False, allowed)
            for dst, src in ((rel, r3), (und, a3)):
                dst[0][bi, h] = src[0]
                dst[1][bi, g] += src[1]
                dst[2][bi, g] += src[2]
    for i, (name, gr, r) in enumerate(zip(("dq", "dk", "dv"), (dq, dk, dv), refs)):
        check_grad(gr, r, rel[i], und[i], W.DTYPES[dt], "cache " + name)
    if causal and nq > nk:
        assert torch.all(dq[:, :, :nq - nk] == 0)


def test_backward_cache_equal_lengths_is_dense_and_empty_cache():
    """Nq = Nk is sattn_bwd bit for bit; an empty cache (Nk = 0) gives dq = 0
    everywhere (and no key gradients to write)."""
    _banner("backward cache == dense, empty cache")
    q, k, v = (x.to(DEV) for x in W.qkv((1, 4, 500, 128), (1, 2, 500, 128), "bf16", 9900))
    do = W.randn((1, 4, 500, 128), "bf16", torch.Generator().manual_seed(9901)).to(DEV)
    for causal in (False, True):
        o, lse = sattn_fwd_cache(q, k, v, causal=causal)
        a = sattn_bwd_cache(q, k, v, o, do, lse, causal=causal)
        b_ = sattn_bwd(q, k, v, o, do, lse, causal=causal)
        torch.cuda.synchronize()
        for x, y in zip(a, b_):
            assert torch.equal(x, y)
    k0, v0 = k[:, :, :0], v[:, :, :0]
    o, lse = sattn_fwd_cache(q, k0, v0, causal=True)
    dq = torch.full_like(q, float("nan"))
    _, dk, dv = sattn_bwd_cache(q, k0, v0, o, do, lse, causal=True, dq=dq)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and dk.numel() == 0 and dv.numel() == 0


def test_backward_deterministic_and_inputs_preserved():
    _banner("backward determinism")
    q, k, v = (x.to(DEV) for x in W.qkv((1, 4, 700, 128), (1, 2, 700, 128), "bf16", 9100))
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).to(DEV)
    o, lse = sattn_fwd_cache(q, k, v, causal=True)
    snap = [x.clone() for x in (q, k, v, o, do, lse)]
    a = sattn_bwd(q, k, v, o, do, lse, causal=True)
    b_ = sattn_bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b_):
        assert torch.equal(x, y)
    for x, y in zip(snap, (q, k, v, o, do, lse)):
        assert torch.equal(x, y)


def test_backward_batched_4x16x4096x128_bf16_two_heads():
    """The batched workload's shape, causal: two (b, h) slices checked in
    full against the float64 gradients (every key's dK/dV needs every
    query, so whole heads are compared)."""
    _banner("backward 4x16x4096x128 bf16")
    from oracle import backward
    b, h, n, d = 4, 16, 4096, 128
    q, k, v = W.qkv((b, h, n, d), (b, h, n, d), "bf16", 3)
    do = W.randn((b, h, n, d), "bf16", torch.Generator().manual_seed(33))
    scale = W.scale_f32(d)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = sattn_fwd(qd, kd, vd, causal=True, scale=scale)
    dq, dk, dv = sattn_bwd(qd, kd, vd, o, dod, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    for (bi, hi) in ((0, 0), (3, 15)):
        sl = (slice(bi, bi + 1), slice(hi, hi + 1))
        refs = backward.attention_backward(W.to_f64(q[bi, hi]), W.to_f64(k[bi, hi]), W.to_f64(v[bi, hi]),
                                           W.to_f64(do[bi, hi]), scale, True)
        _check_grads((dq[sl], dk[sl], dv[sl]), tuple(r[None, None] for r in refs), q[sl], k[sl], v[sl], do[sl],
                     o[sl], scale, True, torch.bfloat16, "[%d,%d] " % (bi, hi))
        # This grid pairs its dQ query tiles (tiles nqt-1-j and j per
        # workgroup) and its dK/dV key tiles (j and nkt-1-j); one slice alone
        # runs unpaired. The gradients of the slice do not depend on which
        # tiles share a workgroup.
        one = sattn_bwd(*(x[sl].contiguous() for x in (qd, kd, vd, o, dod)), lse[sl].contiguous(), causal=True,
                        scale=scale)
        for a, b_, name in zip((dq[sl], dk[sl], dv[sl]), one, ("dq", "dk", "dv")):
            assert torch.equal(a, b_), "[%d,%d] %s of the batched call differs from the slice alone" % (bi, hi, name)


def test_backward_paired_grids_odd_tile_counts():
    """Causal D = 128, N = 4200 (ragged): 17 dQ query tiles of 256 and 33
    dK/dV key tiles of 128 per head, 64 heads, so both grids pair their
    tiles and take the middle tile once. One head against the float64
    gradients, two heads bit for bit against the same slices run alone
    (unpaired)."""
    _banner("backward paired grids, odd tile counts")
    from oracle import backward
    b, h, n, d = 1, 64, 4200, 128
    q, k, v = W.qkv((b, h, n, d), (b, h, n, d), "bf16", 41)
    do = W.randn((b, h, n, d), "bf16", torch.Generator().manual_seed(42))
    scale = W.scale_f32(d)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = sattn_fwd(qd, kd, vd, causal=True, scale=scale)
    dq, dk, dv = sattn_bwd(qd, kd, vd, o, dod, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    sl = (slice(0, 1), slice(63, 64))
    refs = backward.attention_backward(W.to_f64(q[0, 63]), W.to_f64(k[0, 63]), W.to_f64(v[0, 63]),
                                       W.to_f64(do[0, 63]), scale, True)
    _check_grads((dq[sl], dk[sl], dv[sl]), tuple(r[None, None] for r in refs), q[sl], k[sl], v[sl], do[sl],
                 o[sl], scale, True, torch.bfloat16, "[0,63] ")
    for hi in (0, 63):
        sl = (slice(0, 1), slice(hi, hi + 1))
        one = sattn_bwd(*(x[sl].contiguous() for x in (qd, kd, vd, o, dod)), lse[sl].contiguous(), causal=True,
                        scale=scale)
        for a, b_, name in zip((dq[sl], dk[sl], dv[sl]), one, ("dq", "dk", "dv")):
            assert torch.equal(a, b_), "[0,%d] %s of the paired call differs from the slice alone" % (hi, name)


@pytest.mark.parametrize("growth", [3.0, 50.0])
def test_sparse_late_rows_and_score_growth(growth):
    """Window of 100 keys with keys growing along the sequence: rows whose
    first kept key lies after the workgroup's first tile take their reference
    from the tile that has one; growth 50 makes tile sums overflow the fixed
    reference, and the workgroup recomputes with the exact update."""
    _banner("sparse growth", growth)
    n, d = 700, 128
    g = torch.Generator().manual_seed(23)
    q = torch.ones((1, 2, n, d), dtype=torch.bfloat16)
    k = (torch.linspace(0.0, growth, n)[:, None] * torch.ones(d)).expand(1, 2, n, d).to(torch.bfloat16)
    v = torch.randn((1, 2, n, d), generator=g).to(torch.bfloat16)
    scale = W.scale_f32(d)
    o, lse = sattn_fwd_sparse(q.to(DEV), k.contiguous().to(DEV), v.to(DEV), causal=True, window=(99, -1),
                              scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = dense.attention_sparse(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, True, 99)
    check_attention(o, lse, o_ref, lse_ref, torch.bfloat16, "sparse growth")


# ------------------------------ every entry point: fresh outputs, side stream
def _nan_like(x):
    return torch.full_like(x, float("nan"))


def test_all_entry_points_fill_nan_outputs_on_a_side_stream_and_preserve_inputs():
    """Outputs pre-filled with NaN are completely overwritten when each entry
    point runs on a non-default stream, bit-identical to a default-stream
    call, and no input changes."""
    _banner("entry points: fresh outputs / side stream")
    q, k, v = W.qkv((1, 4, 300, 128), (1, 2, 300, 128), "bf16", 9200)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    qt = q.transpose(1, 2).contiguous().transpose(1, 2)          # strided view of the same values
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).to(DEV)
    snap = [x.clone() for x in (q, k, v, do)]
    cu = torch.tensor([0, 100, 300], dtype=torch.int32, device=DEV)
    qv, kv, vv = (x[0].transpose(0, 1).contiguous() for x in (q, k, v))   # [T, H, D] packed
    bm = torch.ones((1, 5, 5), dtype=torch.uint8, device=DEV)
    o0, l0 = sattn_fwd_cache(q, k, v, causal=True)

    calls = {
        "cache": lambda o, l: sattn_fwd_cache(q, k, v, causal=True, out=o, lse=l),
        "strided": lambda o, l: sattn_fwd_strided(qt, k, v, causal=True, out=o, lse=l),
        "sparse": lambda o, l: sattn_fwd_sparse(q, k, v, causal=True, window=(50, -1), n_global=2, block_mask=bm,
                                               out=o, lse=l),
        "varlen": lambda o, l: sattn_fwd_varlen(qv, kv, vv, cu, max_seqlen=200, causal=True, out=o, lse=l),
    }
    shapes = {"varlen": (qv, (4, 300))}
    for name, fn in calls.items():
        like, lshape = shapes.get(name, (q, (1, 4, 300)))
        ref_o, ref_l = fn(torch.empty_like(like), torch.empty(lshape, device=DEV))
        o, l = _nan_like(like), torch.full(lshape, float("nan"), device=DEV)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(o, l)
        s.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), name
    # split partials + merge, and the backward entry points, on the side stream
    os_, ls_ = sattn_fwd_sparse(q, k, v, causal=True, window=(50, -1), n_global=2, block_mask=bm)
    ov, lv = sattn_fwd_varlen(qv, kv, vv, cu, max_seqlen=200, causal=True)
    dov = do[0].transpose(0, 1).contiguous()
    snap += [x.clone() for x in (os_, ls_, ov, lv, dov)]
    pm = torch.full((1, 4, 300, 3), float("nan"), device=DEV)
    pl, pa = _nan_like(pm), torch.full((1, 4, 300, 3, 128), float("nan"), device=DEV)
    ref_p = sattn_fwd_split_cache(q, k, v, 128, causal=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sattn_fwd_split_cache(q, k, v, 128, causal=True, part_m=pm, part_l=pl, part_acc=pa)
        om, lm = sattn_merge(pm, pl, pa, torch.bfloat16, out=_nan_like(q), lse=torch.full((1, 4, 300), float("nan"),
                                                                                      device=DEV))
        grads = sattn_bwd(q, k, v, o0, do, l0, causal=True, dq=_nan_like(q), dk=_nan_like(k), dv=_nan_like(v))
        grads_s = sattn_bwd_sparse(q, k, v, os_, do, ls_, causal=True, window=(50, -1), n_global=2, block_mask=bm,
                                   dq=_nan_like(q), dk=_nan_like(k), dv=_nan_like(v))
        grads_v = sattn_bwd_varlen(qv, kv, vv, ov, dov, lv, cu, max_seqlen=200, causal=True, dq=_nan_like(qv),
                                   dk=_nan_like(kv), dv=_nan_like(vv))
    s.synchronize()
    torch.cuda.synchronize()
    for x, y in zip((pm, pl, pa), ref_p):
        assert torch.equal(x, y)
    ref_g = sattn_bwd(q, k, v, o0, do, l0, causal=True)
    ref_s = sattn_bwd_sparse(q, k, v, os_, do, ls_, causal=True, window=(50, -1), n_global=2, block_mask=bm)
    ref_v = sattn_bwd_varlen(qv, kv, vv, ov, dov, lv, cu, max_seqlen=200, causal=True)
    torch.cuda.synchronize()
    for got, want in ((grads, ref_g), (grads_s, ref_s), (grads_v, ref_v)):
        for x, y in zip(got, want):
            assert torch.equal(x, y)
    assert torch.isfinite(om.float()).all() and torch.isfinite(lm).all()
    for x, y in zip(snap, (q, k, v, do, os_, ls_, ov, lv, dov)):
        assert torch.equal(x, y)


# ------------------------------------------- outputs written only in bounds
def _guarded(shape, dtype, guard=4096):
    """A contiguous tensor of `shape` inside a NaN-filled buffer with `guard`
    elements before and after it (offsets keep 16-byte alignment)."""
    n = int(np.prod(shape))
    buf = torch.full((guard + n + guard,), float("nan"), dtype=dtype, device=DEV)
    return buf, buf[guard:guard + n].view(shape), guard


def _guards_intact(buf, guard, n):
    head, tail = buf[:guard], buf[guard + n:]
    return bool(torch.isnan(head.float()).all()) and bool(torch.isnan(tail.float()).all())


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_outputs_stay_in_bounds(dt, causal):
    """Every forward layout and the backward stage their output rows through
    LDS and store whole rows: with ragged row counts (partial waves and
    workgroups), nothing may be written before or after the output tensors,
    and the results still match the oracle."""
    _banner("guards", dt, causal)
    dtype = W.DTYPES[dt]
    # batched: 300 rows, D = 128 (256-row workgroups, a 44-row tail)
    b, h, n, d = 1, 3, 300, 128
    q, k, v = _dense_inputs(b, h, n, d, dt, seed=31)
    scale = W.scale_f32(d)
    ob, o, g = _guarded((b, h, n, d), dtype)
    lb, lse, gl = _guarded((b, h, n), torch.float32)
    sattn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert _guards_intact(ob, g, o.numel()) and _guards_intact(lb, gl, lse.numel())
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal)
    check_attention(o.cpu(), lse.cpu(), o_ref, lse_ref, dtype, "guards dense")
    # backward of the same call: dq, dk, dv with 300 rows / keys
    do = W.randn((b, h, n, d), dt, torch.Generator().manual_seed(32))
    gbufs = [_guarded((b, h, n, d), dtype) for _ in range(3)]
    sattn_bwd(q.to(DEV), k.to(DEV), v.to(DEV), o, do.to(DEV), lse, causal=causal, scale=scale,
              dq=gbufs[0][1], dk=gbufs[1][1], dv=gbufs[2][1])
    torch.cuda.synchronize()
    for (bb, t, gg) in gbufs:
        assert _guards_intact(bb, gg, t.numel())
        assert torch.isfinite(t.float()).all()
    # packed varlen: ragged sequences, 4 query heads on 2 KV heads, D = 64
    lengths = [37, 130, 5]
    q2, k2, v2, cu = _varlen_inputs(lengths, 4, 2, 64, dt, seed=33)
    t_ = sum(lengths)
    ob2, o2, g2 = _guarded((t_, 4, 64), dtype)
    lb2, lse2, gl2 = _guarded((4, t_), torch.float32)
    sattn_fwd_varlen(q2.to(DEV), k2.to(DEV), v2.to(DEV), torch.from_numpy(cu), causal=causal, out=o2, lse=lse2)
    torch.cuda.synchronize()
    assert _guards_intact(ob2, g2, o2.numel()) and _guards_intact(lb2, gl2, lse2.numel())
    o2_ref, lse2_ref = dense.varlen_gqa(W.to_f64(q2), W.to_f64(k2), W.to_f64(v2), cu, W.scale_f32(64), causal)
    check_attention(o2.cpu(), lse2.cpu(), o2_ref, lse2_ref, dtype, "guards varlen")
    # queries against a cache: 600 queries (256-row workgroups when non-causal), D = 32 tails elsewhere
    for (nq, nk, dd) in ((600, 900, 128), (45, 200, 32)):
        q3, k3, v3 = W.qkv((1, 4, nq, dd), (1, 2, nk, dd), dt, 34)
        ob3, o3, g3 = _guarded((1, 4, nq, dd), dtype)
        lb3, lse3, gl3 = _guarded((1, 4, nq), torch.float32)
        sc3 = W.scale_f32(dd)
        sattn_fwd_cache(q3.to(DEV), k3.to(DEV), v3.to(DEV), causal=causal, scale=sc3, out=o3, lse=lse3)
        torch.cuda.synchronize()
        assert _guards_intact(ob3, g3, o3.numel()) and _guards_intact(lb3, gl3, lse3.numel())
        o3_ref, lse3_ref = dense.attention_cache(W.to_f64(q3), W.to_f64(k3), W.to_f64(v3), sc3, causal)
        check_attention(o3.cpu(), lse3.cpu(), o3_ref, lse3_ref, dtype, "guards cache")


@pytest.mark.parametrize("nbytes,grid", [(1 << 20, 64), ((1 << 20) + 48, 7), (4096, 1024)])
def test_read_probe_reads_every_word_once(nbytes, grid):
    """The streaming-read probe behind bench.py --read-ceiling: the XOR of
    what its threads report equals the XOR of every 32-bit word of the
    buffer (a word missed or read twice changes it), for ragged sizes and
    more workgroups than 16-byte pieces."""
    import ctypes
    from exact_tiled_attention_sattn_amd.build import PROBE_LIB
    _banner("read probe", nbytes, grid)
    probe = ctypes.CDLL(PROBE_LIB)
    probe.sattn_probe_read.restype = ctypes.c_int
    probe.sattn_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_void_p]
    g = torch.Generator().manual_seed(nbytes + grid)
    words = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int64).to(torch.int32)
    buf = words.to(DEV)
    out = torch.full((grid * 256,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    rc = probe.sattn_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()), out.numel(),
                                grid, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(words.numpy().view(np.uint32))
    assert got == want

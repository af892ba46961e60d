#!/usr/bin/env python3
"""Throughput benchmark of the exact streaming attention forward on one MI355X.

One step = the batched multi-head forward B=4, H=16, N=4096, D=128 in bf16,
run once noncausal and once causal on the same resident inputs. FLOPs are
counted per head as 4*N^2*D noncausal and 2*N^2*D causal; ``value`` is the
step's FLOPs over its wall time (TFLOP/s).

Method, after the pages' timing rules ("Intermediate and advanced extension",
code review and execution gates 5; "Intermediate and advanced workshop
validation", measured examples): a correctness gate before timing (sampled
rows against a plain float64 torch computation on the host; the FP64 oracle
itself runs only in the CPU-baseline leg), untimed warmup steps, then timed steps between device
synchronizations, with a HIP event pair around every launch on the stream the
kernel runs on. Small shapes are timed separately as graph replays (20 calls
captured in one HIP graph) and as eager event timing.

Output: one JSON line on stdout (progress goes to stderr).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "attention fwd TFLOP/s and % of bf16 MFMA peak; µs latency at N,D=512×64"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
KERNEL_SOURCES = ["exact_tiled_attention_sattn_amd/csrc/fwd_kernel.hpp",
                  "exact_tiled_attention_sattn_amd/csrc/common.hpp",
                  "exact_tiled_attention_sattn_amd/csrc/fwd_small.hpp",
                  "exact_tiled_attention_sattn_amd/csrc/sattn.hip"]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "fwd_kernel_batched_4x16x4096x128_bf16_pmc.json")
DEV = "cuda:0"
PREHEAT_S = 0.5   # untimed load on the benchmark step before its warmup steps
# The pages' own figures for the two small causal fp16 shapes ("Intermediate
# and advanced workshop validation", measured examples): a Triton streaming
# kernel with 64-key blocks on an RTX 4080 SUPER, graph-timed median of 7
# samples x 20 calls. Another machine: context beside the latency, not a target.
PAGES_CONTEXT = {
    "129x32": {"graph_us": 3.366, "sdpa_graph_us": 6.758, "hardware": "RTX 4080 SUPER, Triton stream_bn64",
               "use": "context only"},
    "512x64": {"graph_us": 8.235, "sdpa_graph_us": 8.499, "hardware": "RTX 4080 SUPER, Triton stream_bn64",
               "use": "context only"},
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def dense_flops(b, h, n, d, causal):
    return (2 if causal else 4) * b * h * n * n * d


def gate_rows(o, lse, q, k, v, scale, causal, rows, pos, dtype, what, allowed=None):
    """Correctness gate for one (batch, head) slice: the GPU's rows ``rows``
    (query indices) against float64 torch on the host, computed directly from
    the definition for those rows only (``pos``: their logical positions,
    keys j <= pos eligible when causal; every gated row has an eligible key).
    """
    from tests.parity import check_attention
    qh = q[rows].detach().cpu().double()
    kh, vh = k.detach().cpu().double(), v.detach().cpu().double()
    s = scale * (qh @ kh.T)
    if causal:
        s = s.masked_fill(torch.arange(kh.shape[0])[None, :] > torch.as_tensor(pos)[:, None], -math.inf)
    if allowed is not None:                 # [R, Nk] eligibility of the gated rows
        s = s.masked_fill(~allowed, -math.inf)
    lse_ref = torch.logsumexp(s, dim=-1)
    o_ref = torch.exp(s - lse_ref[:, None]) @ vh
    return check_attention(o[rows], lse[rows], o_ref.numpy(), lse_ref.numpy(), dtype, what)


def gate_dense(fwd, q, k, v, scale, causal, rows_per_head, seed, dtype):
    """Correctness gate: seeded sampled rows of every head."""
    b, h, n, d = q.shape
    o, lse = fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = W.sample_rows(seed, n, rows_per_head, groups=b * h).reshape(b, h, -1)
    oc, lc = o.cpu(), lse.cpu()
    worst = {}
    for i in range(b):
        for j in range(h):
            r = torch.from_numpy(rows[i, j])
            res = gate_rows(oc[i, j], lc[i, j], q[i, j], k[i, j], v[i, j], scale, causal, r, r, dtype, "gate")
            for key, val in res.items():
                worst[key] = max(worst.get(key, 0.0), val)
    return worst


def time_launches(fn, steps, warmup, min_warm_s=0.2):
    """Per-launch HIP events on the current stream; returns list of ms.
    Untimed calls first: `warmup` of them, and more until `min_warm_s` of
    load has passed, so that the clock has settled after host-side setup."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_warm_s:
        fn()
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def graph_latency_us(fn, calls=20, samples=7, warmup=5):
    """Median per-call latency of ``calls`` launches captured in one graph."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn()  # warm on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for _ in range(calls):
                fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(samples):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) * 1000.0 / calls)
    return out


def event_latency_us(fn, calls=20, samples=7, warmup=5):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    out = []
    for _ in range(samples):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(calls):
            fn()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) * 1000.0 / calls)
    return out


def small_latency(fwd, n, d, dtype_name, seed, causal, qmul=1.0):
    q, k, v = W.qkv((1, 1, n, d), (1, 1, n, d), dtype_name, seed)
    if qmul != 1.0:
        q = (q.float() * qmul).to(q.dtype)
    q, k, v = (x.to(DEV) for x in (q, k, v))
    scale = W.scale_f32(d)
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, n), dtype=torch.float32, device=DEV)
    fn = lambda: fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse)  # noqa: E731
    # gate: every row
    fn()
    torch.cuda.synchronize()
    r = torch.arange(n)
    gate_rows(o[0, 0].cpu(), lse[0, 0].cpu(), q[0, 0], k[0, 0], v[0, 0], scale, causal, r, r,
              W.DTYPES[dtype_name], "gate %dx%d" % (n, d))
    gr = graph_latency_us(fn)
    ev = event_latency_us(fn)
    return {"graph_us_median": float(np.median(gr)), "graph_us_min": float(min(gr)), "graph_us_max": float(max(gr)),
            "event_us_median": float(np.median(ev)), "graph_samples_us": gr, "event_samples_us": ev}


def decode_extra(steps, host_rows=None):
    """Split-KV decode B=16, Hq=Hkv=32, Nk=131072, D=128, chunks of 4096.
    ``host_rows`` (a dict, when the CPU leg runs) receives host copies of two
    rows' q, K and V slices and the time of those device-to-host copies."""
    from exact_tiled_attention_sattn_amd import sattn_fwd_split, sattn_merge
    cfg = W.WORKLOADS["splitkv_decode_16x32x131072x128_bf16"]
    b, hq, hkv, nk, d, chunk = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["Nk"], cfg["D"], cfg["chunk"]
    g = torch.Generator(device=DEV)
    g.manual_seed(cfg["seed"])
    q = W.randn_device_sliced((b, hq, 1, d), "bf16", g, DEV)
    k = W.randn_device_sliced((b, hkv, nk, d), "bf16", g, DEV)
    v = W.randn_device_sliced((b, hkv, nk, d), "bf16", g, DEV)
    c = -(-nk // chunk)
    pm = torch.empty((b, hq, 1, c), dtype=torch.float32, device=DEV)
    pl = torch.empty_like(pm)
    pa = torch.empty((b, hq, 1, c, d), dtype=torch.float32, device=DEV)
    o = torch.empty((b, hq, 1, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((b, hq, 1), dtype=torch.float32, device=DEV)
    scale = W.scale_f32(d)
    split = lambda: sattn_fwd_split(q, k, v, chunk, scale, part_m=pm, part_l=pl, part_acc=pa)  # noqa: E731
    merge = lambda: sattn_merge(pm, pl, pa, torch.bfloat16, out=o, lse=lse)  # noqa: E731
    # gate: 4 rows
    split()
    merge()
    torch.cuda.synchronize()
    for flat in (0, 137, 300, 511):
        bb, h = divmod(flat, hq)
        gate_rows(o[bb, h].cpu(), lse[bb, h].cpu(), q[bb, h], k[bb, h], v[bb, h], scale, False,
                  torch.tensor([0]), None, torch.bfloat16, "gate decode")
    t_split = time_launches(split, steps, 2)
    t_merge = time_launches(merge, steps, 2)
    kv_bytes = 2 * b * hkv * nk * d * 2
    part_bytes = b * hq * c * (d + 2) * 4
    io_bytes = b * hq * d * 2 * 2 + b * hq * 4
    split_bytes = kv_bytes + b * hq * d * 2 + part_bytes
    merge_bytes = part_bytes + b * hq * d * 2 + b * hq * 4
    ms_split, ms_merge = float(np.mean(t_split)), float(np.mean(t_merge))
    total_bytes = kv_bytes + 2 * part_bytes + io_bytes
    out = {"workload": "splitkv_decode_16x32x131072x128_bf16 (chunk 4096, 32 partials per row)",
           "split_ms_mean": ms_split, "merge_ms_mean": ms_merge,
           "split_GBps": split_bytes / ms_split / 1e6, "merge_GBps": merge_bytes / ms_merge / 1e6,
           "end_to_end_GBps": total_bytes / (ms_split + ms_merge) / 1e6,
           "split_frac_of_hbm_peak": split_bytes / ms_split / 1e6 / PEAK_HBM_GBS,
           "algorithmic_bytes_split": split_bytes, "algorithmic_bytes_merge": merge_bytes}
    out["chunk_sweep"] = chunk_sweep(q, k, v, scale, o, lse, steps)
    if host_rows is not None:
        for flat in (0, 511):
            bb, h = divmod(flat, hq)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            qs, ks, vs = q[bb, h].cpu(), k[bb, h].cpu(), v[bb, h].cpu()
            host_rows[flat] = (qs, ks, vs, time.perf_counter() - t0)
    del q, k, v
    torch.cuda.empty_cache()
    return out


def chunk_sweep(q, k, v, scale, o_ref, lse_ref, steps):
    """Split width against end-to-end decode bandwidth (split + merge) on the
    same resident K/V: narrow chunks launch more workgroups and write more
    partials, wide ones leave CUs idle. Each width's output is checked
    against the 4096-wide result (both lie within the bf16 tolerance of the
    exact value, so they differ by at most twice it)."""
    from exact_tiled_attention_sattn_amd import sattn_fwd_split, sattn_merge
    b, hq, _, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    kv_bytes = 2 * b * hkv * nk * d * 2
    res = []
    for chunk in (1024, 2048, 4096, 8192, 16384, 32768, 131072):
        c = -(-nk // chunk)
        pm = torch.empty((b, hq, 1, c), dtype=torch.float32, device=DEV)
        pl = torch.empty_like(pm)
        pa = torch.empty((b, hq, 1, c, d), dtype=torch.float32, device=DEV)
        o = torch.empty_like(o_ref)
        lse = torch.empty_like(lse_ref)

        def both():
            sattn_fwd_split(q, k, v, chunk, scale, part_m=pm, part_l=pl, part_acc=pa)
            sattn_merge(pm, pl, pa, torch.bfloat16, out=o, lse=lse)
        both()
        torch.cuda.synchronize()
        err = (o.float() - o_ref.float()).abs()
        if not bool((err <= 2e-2 + 2e-2 * o_ref.float().abs()).all()) or \
                float((lse - lse_ref).abs().max()) > 2e-3:
            raise RuntimeError("chunk sweep: chunk %d disagrees with the 4096-wide result" % chunk)
        t = float(np.mean(time_launches(both, steps, 2)))
        part_bytes = b * hq * c * (d + 2) * 4
        total = kv_bytes + 2 * part_bytes + b * hq * d * 2 * 2 + b * hq * 4
        res.append({"chunk": chunk, "partials_per_row": c, "split_workgroups": b * hq * c, "ms": t,
                    "end_to_end_GBps": total / t / 1e6})
        del pm, pl, pa
    return res


def varlen_extra(steps):
    from exact_tiled_attention_sattn_amd import sattn_fwd_varlen
    cfg = W.WORKLOADS["varlen_gqa_8seq_32q8kv_128_bf16_causal"]
    lengths = W.varlen_lengths(cfg["seed"], cfg["S"], cfg["max_len"])
    hq, hkv, d = cfg["Hq"], cfg["Hkv"], cfg["D"]
    t = int(lengths.sum())
    q, k, v = W.qkv((t, hq, d), (t, hkv, d), "bf16", cfg["seed"])
    q, k, v = (x.to(DEV) for x in (q, k, v))
    cu = torch.from_numpy(W.cu_seqlens_of(lengths)).to(DEV)
    mx = int(lengths.max())
    scale = W.scale_f32(d)
    o = torch.empty_like(q)
    lse = torch.empty((hq, t), dtype=torch.float32, device=DEV)
    fn = lambda: sattn_fwd_varlen(q, k, v, cu, max_seqlen=mx, causal=True, scale=scale, out=o, lse=lse)  # noqa
    ms = float(np.mean(time_launches(fn, steps, 2)))
    flops = sum(2 * int(L) * int(L) * d * hq for L in lengths)
    return {"workload": "varlen_gqa_8seq_32q8kv_128_bf16_causal", "lengths": lengths.tolist(), "T": t,
            "ms_mean": ms, "TFLOPs": flops / ms / 1e9, "frac_of_bf16_peak": flops / ms / 1e9 / PEAK_BF16_TFLOPS,
            "flop": flops}


def prefill_extra(steps):
    """One 2048-query chunk of a chunked prefill against a 16384-token K/V
    cache (query i at position i + 14336), 32 query heads on 8 KV heads,
    bf16, causal. FLOPs count eligible (query, key) pairs at 4*D each, with
    the diagonal term dropped as in the dense convention."""
    from exact_tiled_attention_sattn_amd import sattn_fwd_cache
    b, hq, hkv, nq, nk, d = 1, 32, 8, 2048, 16384, 128
    q, k, v = (x.to(DEV) for x in W.qkv((b, hq, nq, d), (b, hkv, nk, d), "bf16", 7))
    scale = W.scale_f32(d)
    o = torch.empty_like(q)
    lse = torch.empty((b, hq, nq), dtype=torch.float32, device=DEV)
    fn = lambda: sattn_fwd_cache(q, k, v, causal=True, scale=scale, out=o, lse=lse)  # noqa: E731
    fn()
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1000, nq - 1])
    oc, lc = o.cpu(), lse.cpu()
    for h in (0, 13, 31):
        gate_rows(oc[0, h], lc[0, h], q[0, h], k[0, h // 4], v[0, h // 4], scale, True, rows, rows + nk - nq,
                  torch.bfloat16, "gate prefill")
    ms = float(np.mean(time_launches(fn, steps, 2)))
    off = nk - nq
    flops = 4 * d * (nq * off + nq * nq // 2) * b * hq
    del q, k, v, o
    torch.cuda.empty_cache()
    return {"workload": "chunked prefill: 2048 queries vs 16384-token cache, 32q/8kv heads, D=128 bf16 causal",
            "ms_mean": ms, "TFLOPs": flops / ms / 1e9, "frac_of_bf16_peak": flops / ms / 1e9 / PEAK_BF16_TFLOPS,
            "flop": flops}


def gqa_decode_extra(steps):
    """Causal decode of 4 new tokens per sequence against a 32768-token K/V
    cache: B=8, 32 query heads on 8 KV heads, D=128 bf16, chunks of 2048
    (causal split partials, then the merge). Bytes count K/V once."""
    from exact_tiled_attention_sattn_amd import sattn_fwd_split_cache, sattn_merge
    b, hq, hkv, nq, nk, d, chunk = 8, 32, 8, 4, 32768, 128, 2048
    g = torch.Generator(device=DEV)
    g.manual_seed(8)
    q = W.randn_device_sliced((b, hq, nq, d), "bf16", g, DEV)
    k = W.randn_device_sliced((b, hkv, nk, d), "bf16", g, DEV)
    v = W.randn_device_sliced((b, hkv, nk, d), "bf16", g, DEV)
    c = -(-nk // chunk)
    pm = torch.empty((b, hq, nq, c), dtype=torch.float32, device=DEV)
    pl = torch.empty_like(pm)
    pa = torch.empty((b, hq, nq, c, d), dtype=torch.float32, device=DEV)
    o = torch.empty((b, hq, nq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((b, hq, nq), dtype=torch.float32, device=DEV)
    scale = W.scale_f32(d)
    split = lambda: sattn_fwd_split_cache(q, k, v, chunk, causal=True, scale=scale,  # noqa: E731
                                          part_m=pm, part_l=pl, part_acc=pa)
    merge = lambda: sattn_merge(pm, pl, pa, torch.bfloat16, out=o, lse=lse)  # noqa: E731
    split()
    merge()
    torch.cuda.synchronize()
    rows = torch.arange(nq)
    for bb, h in ((0, 0), (5, 17), (7, 31)):
        gate_rows(o[bb, h].cpu(), lse[bb, h].cpu(), q[bb, h], k[bb, h // 4], v[bb, h // 4], scale, True, rows,
                  rows + nk - nq, torch.bfloat16, "gate gqa decode")
    t_split = time_launches(split, steps, 2)
    t_merge = time_launches(merge, steps, 2)
    kv_bytes = 2 * b * hkv * nk * d * 2
    part_bytes = b * hq * nq * c * (d + 2) * 4
    split_bytes = kv_bytes + b * hq * nq * d * 2 + part_bytes
    ms_split, ms_merge = float(np.mean(t_split)), float(np.mean(t_merge))
    del q, k, v
    torch.cuda.empty_cache()
    return {"workload": "causal GQA decode: 4 queries vs 32768-token cache, B=8, 32q/8kv heads, D=128 bf16, "
                        "chunk 2048",
            "split_ms_mean": ms_split, "merge_ms_mean": ms_merge, "split_GBps": split_bytes / ms_split / 1e6,
            "split_frac_of_hbm_peak": split_bytes / ms_split / 1e6 / PEAK_HBM_GBS,
            "algorithmic_bytes_split": split_bytes}


def strided_extra(steps):
    """Transposed inputs: q, k, v stored [B, N, H, D] (B=4, H=16, N=4096,
    D=128 bf16) and viewed as [B, H, N, D]. Loaded in place by
    sattn_fwd_strided, against copying them to [B, H, N, D] first and running
    the same kernel on the copies (the copy inside the timing, as in the
    pages' strided-input comparison)."""
    from exact_tiled_attention_sattn_amd import sattn_fwd_strided, sattn_fwd_cache
    b, h, n, d = 4, 16, 4096, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    q, k, v = (W.randn_device_sliced((b, n, h, d), "bf16", g, DEV).permute(0, 2, 1, 3) for _ in range(3))
    scale = W.scale_f32(d)
    o = torch.empty((b, h, n, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=DEV)
    res = {"workload": "transposed [B,N,H,D] inputs viewed as [B,H,N,D], 4x16x4096x128 bf16"}
    for causal in (False, True):
        direct = lambda: sattn_fwd_strided(q, k, v, causal=causal, scale=scale, out=o, lse=lse)  # noqa: E731
        direct()
        torch.cuda.synchronize()
        r = torch.tensor([0, 2047, n - 1])
        gate_rows(o[1, 5].cpu(), lse[1, 5].cpu(), q[1, 5], k[1, 5], v[1, 5], scale, causal, r, r, torch.bfloat16,
                  "gate strided")

        def copied():
            sattn_fwd_cache(q.contiguous(), k.contiguous(), v.contiguous(), causal=causal, scale=scale, out=o, lse=lse)
        ms_d = float(np.mean(time_launches(direct, steps, 2)))
        ms_c = float(np.mean(time_launches(copied, steps, 2)))
        fl = dense_flops(b, h, n, d, causal)
        tag = "causal" if causal else "noncausal"
        res[tag] = {"direct_ms": ms_d, "copy_then_kernel_ms": ms_c, "direct_TFLOPs": fl / ms_d / 1e9,
                    "copy_then_kernel_TFLOPs": fl / ms_c / 1e9}
    del q, k, v
    torch.cuda.empty_cache()
    return res


def sparse_extra(steps):
    """Changed operators (lessons 06 and 07): work counts kept (query, key)
    pairs at 4*D FLOP each.
    * causal sliding window of 2048 keys united with 64 global tokens,
      B=1, H=16, N=16384, D=128 bf16;
    * block-sparse, non-causal, 64x64 blocks, a seeded per-head mask with a
      quarter of the blocks active, B=1, H=16, N=8192, D=128 bf16."""
    from exact_tiled_attention_sattn_amd import sattn_fwd_sparse
    res = {}
    h, d = 16, 128
    scale = W.scale_f32(d)
    # -- window + globals
    n, w, ng = 16384, 2048, 64
    q, k, v = (x.to(DEV) for x in W.qkv((1, h, n, d), (1, h, n, d), "bf16", 10))
    o = torch.empty_like(q)
    lse = torch.empty((1, h, n), dtype=torch.float32, device=DEV)
    fn = lambda: sattn_fwd_sparse(q, k, v, causal=True, window=(w - 1, -1), n_global=ng, scale=scale,  # noqa: E731
                                  out=o, lse=lse)
    fn()
    torch.cuda.synchronize()
    rows = torch.tensor([0, 63, 64, 5000, n - 1])
    j = torch.arange(n)[None, :]
    p = rows[:, None]
    allowed = (j <= p) & ((j >= p - (w - 1)) | (j < ng) | (p < ng))
    gate_rows(o[0, 3].cpu(), lse[0, 3].cpu(), q[0, 3], k[0, 3], v[0, 3], scale, False, rows, None, torch.bfloat16,
              "gate window", allowed=allowed)
    ms = float(np.mean(time_launches(fn, steps, 2)))
    pairs = sum((i + 1) if i < ng else min(i + 1, w) + ng - max(0, ng - max(0, i - w + 1)) for i in range(n)) * h
    res["causal_window2048_global64_16x16384x128_bf16"] = {
        "ms_mean": ms, "kept_pairs": pairs, "TFLOPs": 4 * d * pairs / ms / 1e9,
        "frac_of_bf16_peak": 4 * d * pairs / ms / 1e9 / PEAK_BF16_TFLOPS}
    del q, k, v, o
    # -- block sparse
    n = 8192
    q, k, v = (x.to(DEV) for x in W.qkv((1, h, n, d), (1, h, n, d), "bf16", 11))
    gen = torch.Generator().manual_seed(11)
    bm = (torch.rand((h, n // 64, n // 64), generator=gen) < 0.25).to(torch.uint8)
    bmd = bm.to(DEV)
    o = torch.empty_like(q)
    lse = torch.empty((1, h, n), dtype=torch.float32, device=DEV)
    fn = lambda: sattn_fwd_sparse(q, k, v, block_mask=bmd, block_q=64, block_k=64, scale=scale,  # noqa: E731
                                  out=o, lse=lse)
    fn()
    torch.cuda.synchronize()
    rows = torch.tensor([0, 4000, n - 1])
    allowed = bm[5][rows // 64].repeat_interleave(64, dim=1).bool()
    ok = allowed.any(dim=1)
    gate_rows(o[0, 5].cpu(), lse[0, 5].cpu(), q[0, 5], k[0, 5], v[0, 5], scale, False, rows[ok], None,
              torch.bfloat16, "gate block-sparse", allowed=allowed[ok])
    ms = float(np.mean(time_launches(fn, steps, 2)))
    pairs = int(bm.sum()) * 64 * 64
    res["block_sparse_quarter_64x64_16x8192x128_bf16"] = {
        "ms_mean": ms, "active_block_pairs": int(bm.sum()), "kept_pairs": pairs,
        "TFLOPs": 4 * d * pairs / ms / 1e9, "frac_of_bf16_peak": 4 * d * pairs / ms / 1e9 / PEAK_BF16_TFLOPS}
    del q, k, v, o
    torch.cuda.empty_cache()
    return res


def backward_extra(steps):
    """Backward (dQ, dK, dV) of the batched 4x16x4096x128 bf16 workload,
    causal and non-causal, on the forward's own O and lse. FLOPs follow the
    usual convention of five N^2*D products (2.5x the forward: 10*N^2*D per
    head non-causal, 5*N^2*D causal); the two-kernel schedule here executes
    seven (S and dP are recomputed by both kernels), also reported."""
    from exact_tiled_attention_sattn_amd import sattn_fwd, sattn_bwd
    b, h, n, d = 4, 16, 4096, 128
    q, k, v = (x.to(DEV) for x in W.qkv((b, h, n, d), (b, h, n, d), "bf16", 3))
    do = W.randn((b, h, n, d), "bf16", torch.Generator().manual_seed(33)).to(DEV)
    scale = W.scale_f32(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((b, h, n), dtype=torch.float32, device=DEV)
    res = {"workload": "backward of batched_4x16x4096x128_bf16",
           "flop_convention": "10*N^2*D per head noncausal, 5*N^2*D causal (2.5x forward)"}
    for causal in (False, True):
        o, lse = sattn_fwd(q, k, v, causal=causal, scale=scale)
        fn = lambda: sattn_bwd(q, k, v, o, do, lse, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv,  # noqa: E731
                               delta=delta)
        fn()
        torch.cuda.synchronize()
        assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()
        ms = float(np.mean(time_launches(fn, steps, 2)))
        fl = 2.5 * dense_flops(b, h, n, d, causal)
        res["causal" if causal else "noncausal"] = {
            "ms_mean": ms, "TFLOPs": fl / ms / 1e9, "frac_of_bf16_peak": fl / ms / 1e9 / PEAK_BF16_TFLOPS,
            "executed_TFLOPs": 3.5 * dense_flops(b, h, n, d, causal) / ms / 1e9}
    del q, k, v, do, dq, dk, dv
    torch.cuda.empty_cache()
    return res


def varlen_backward_extra(steps):
    """Backward of the packed varlen GQA workload (8 seeded sequence lengths,
    32 query heads on 8 KV heads, D = 128, bf16, causal) on the forward's own
    O and lse. FLOPs: 2.5x the forward's causal count, as for the batched
    backward."""
    from exact_tiled_attention_sattn_amd import sattn_fwd_varlen, sattn_bwd_varlen
    cfg = W.WORKLOADS["varlen_gqa_8seq_32q8kv_128_bf16_causal"]
    lengths = W.varlen_lengths(cfg["seed"], cfg["S"], cfg["max_len"])
    hq, hkv, d = cfg["Hq"], cfg["Hkv"], cfg["D"]
    t = int(lengths.sum())
    q, k, v = (x.to(DEV) for x in W.qkv((t, hq, d), (t, hkv, d), "bf16", cfg["seed"]))
    do = W.randn((t, hq, d), "bf16", torch.Generator().manual_seed(cfg["seed"] + 1)).to(DEV)
    cu = torch.from_numpy(W.cu_seqlens_of(lengths)).to(DEV)
    mx = int(lengths.max())
    scale = W.scale_f32(d)
    o, lse = sattn_fwd_varlen(q, k, v, cu, max_seqlen=mx, causal=True, scale=scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((hq, t), dtype=torch.float32, device=DEV)
    fn = lambda: sattn_bwd_varlen(q, k, v, o, do, lse, cu, max_seqlen=mx, causal=True, scale=scale,  # noqa: E731
                                  dq=dq, dk=dk, dv=dv, delta=delta)
    fn()
    torch.cuda.synchronize()
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()
    ms = float(np.mean(time_launches(fn, steps, 2)))
    flops = 2.5 * sum(2 * int(L) * int(L) * d * hq for L in lengths)
    del q, k, v, do, dq, dk, dv, o
    torch.cuda.empty_cache()
    return {"workload": "backward of varlen_gqa_8seq_32q8kv_128_bf16_causal", "T": t, "ms_mean": ms,
            "TFLOPs": flops / ms / 1e9, "frac_of_bf16_peak": flops / ms / 1e9 / PEAK_BF16_TFLOPS,
            "flop_convention": "2.5x the forward's causal 2*L^2*D per query head"}


def sparse_backward_extra(steps):
    """Backward of the causal sliding window (2048 keys) united with 64
    global tokens, B=1, H=16, N=16384, D=128 bf16, on the forward's own O and
    lse. FLOPs: 2.5x the forward's kept-pair count at 4*D each."""
    from exact_tiled_attention_sattn_amd import sattn_fwd_sparse, sattn_bwd_sparse
    h, d, n, w, ng = 16, 128, 16384, 2048, 64
    scale = W.scale_f32(d)
    q, k, v = (x.to(DEV) for x in W.qkv((1, h, n, d), (1, h, n, d), "bf16", 10))
    do = W.randn((1, h, n, d), "bf16", torch.Generator().manual_seed(12)).to(DEV)
    o, lse = sattn_fwd_sparse(q, k, v, causal=True, window=(w - 1, -1), n_global=ng, scale=scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((1, h, n), dtype=torch.float32, device=DEV)
    fn = lambda: sattn_bwd_sparse(q, k, v, o, do, lse, causal=True, window=(w - 1, -1), n_global=ng,  # noqa: E731
                                  scale=scale, dq=dq, dk=dk, dv=dv, delta=delta)
    fn()
    torch.cuda.synchronize()
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()
    ms = float(np.mean(time_launches(fn, steps, 2)))
    pairs = sum((i + 1) if i < ng else min(i + 1, w) + ng - max(0, ng - max(0, i - w + 1)) for i in range(n)) * h
    del q, k, v, do, dq, dk, dv, o
    torch.cuda.empty_cache()
    fl = 2.5 * 4 * d * pairs
    return {"workload": "backward of causal_window2048_global64_16x16384x128_bf16", "ms_mean": ms,
            "TFLOPs": fl / ms / 1e9, "frac_of_bf16_peak": fl / ms / 1e9 / PEAK_BF16_TFLOPS,
            "flop_convention": "2.5x the forward's kept pairs at 4*D"}


def cpu_baseline(budget_s):
    """The FP64 oracle on sampled query rows of the batched workload, both
    variants, on the host cores, scaled to TFLOP/s by the sampled fraction."""
    from oracle import dense
    b, h, n, d = 4, 16, 4096, 128
    q, k, v = W.qkv((b, h, n, d), (b, h, n, d), "bf16", W.WORKLOADS["batched_4x16x4096x128_bf16"]["seed"])
    qh, kh, vh = W.to_f64(q), W.to_f64(k), W.to_f64(v)
    scale = W.scale_f32(d)
    rows_done = 0
    t0 = time.perf_counter()
    per = 64
    heads_done = 0
    while True:
        bh = heads_done % (b * h)
        bi, hi = divmod(bh, h)
        r = W.sample_rows(1000 + heads_done, n, per)[0]
        for causal in (False, True):
            dense.attention(qh[bi, hi][r], kh[bi, hi], vh[bi, hi], scale, causal, q_pos=r)
        rows_done += per
        heads_done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    frac = rows_done / float(b * h * n)     # fraction of all query rows, both variants each
    step_flop = dense_flops(b, h, n, d, False) + dense_flops(b, h, n, d, True)
    value = frac * step_flop / el / 1e12
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": value, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": "numpy float64 dense oracle on %d seeded query rows (64 per head per draw, heads in turn; each "
                      "row against all 4096 keys, computed both noncausal and causal) of the 4x16x4096x128 workload "
                      "in %.1f s; that is %.3f times the query rows of one step, and value = that share of one "
                      "step's FLOPs / time" % (rows_done, el, frac),
            "host_cores_visible": len(os.sched_getaffinity(0)), "cpu_model": cpu_model}


def cpu_oracle_per_workload(decode_rows, budget_rows_varlen=64):
    """The FP64 oracle on each workload, timed on the host cores: the two
    small shapes in full (median of 5), the decode on the rows copied to the
    host (per row, and the device-to-host time of their slices), the packed
    varlen workload on seeded rows per (sequence, query head), scaled to the
    full workload by FLOPs and labelled as an estimate."""
    from oracle import dense

    def med_ms(fn, reps=5):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append((time.perf_counter() - t0) * 1e3)
        return float(np.median(ts)), ts

    out = {}
    q, k, v = W.qkv((1, 1, 129, 32), (1, 1, 129, 32), "fp16", W.WORKLOADS["single_head_129x32_fp16_causal"]["seed"])
    qh, kh, vh = W.to_f64(q), W.to_f64(k), W.to_f64(v)
    sc = W.scale_f32(32)
    m, ts = med_ms(lambda: dense.attention_bhnd(qh, kh, vh, sc, True))
    out["129x32_fp16_causal"] = {"oracle_ms_median": m, "oracle_ms_samples": ts, "rows": "all 129"}
    q, k, v = W.qkv((1, 1, 512, 64), (1, 1, 512, 64), "fp16", W.WORKLOADS["single_head_512x64_fp16"]["seed"])
    kh, vh = W.to_f64(k), W.to_f64(v)
    sc = W.scale_f32(64)
    for qmul in (1.0, 16.0):
        qh = W.to_f64(q) * qmul
        for causal in (True, False):
            m, ts = med_ms(lambda: dense.attention_bhnd(qh, kh, vh, sc, causal))
            out["512x64_fp16_%s%s" % ("causal" if causal else "noncausal", "_q16" if qmul != 1.0 else "")] = {
                "oracle_ms_median": m, "oracle_ms_samples": ts, "rows": "all 512"}
    if decode_rows:
        sc = W.scale_f32(128)
        per_row, d2h = [], []
        for flat, (qs, ks, vs, t_copy) in sorted(decode_rows.items()):
            qd, kd, vd = W.to_f64(qs), W.to_f64(ks), W.to_f64(vs)
            t0 = time.perf_counter()
            dense.attention(qd, kd, vd, sc, False)
            per_row.append((time.perf_counter() - t0) * 1e3)
            d2h.append(t_copy * 1e3)
        out["splitkv_decode_16x32x131072x128_bf16"] = {
            "oracle_ms_per_row": per_row, "rows": sorted(decode_rows),
            "d2h_ms_per_row_slice": d2h, "d2h_bytes_per_row_slice": 2 * 131072 * 128 * 2 + 128 * 2,
            "estimate_all_512_rows_s": float(np.mean(per_row)) * 512 / 1e3,
            "note": "estimate = mean per-row oracle time x 512 rows, D2H excluded"}
    cfg = W.WORKLOADS["varlen_gqa_8seq_32q8kv_128_bf16_causal"]
    lengths = W.varlen_lengths(cfg["seed"], cfg["S"], cfg["max_len"])
    hq, hkv, d = cfg["Hq"], cfg["Hkv"], cfg["D"]
    t = int(lengths.sum())
    q, k, v = W.qkv((t, hq, d), (t, hkv, d), "bf16", cfg["seed"])
    qh, kh, vh = W.to_f64(q), W.to_f64(k), W.to_f64(v)
    cu = W.cu_seqlens_of(lengths)
    rows, flop_s = {}, 0.0
    for si, L in enumerate(lengths):
        for h in range(hq):
            r = W.sample_rows(2000 + si * hq + h, int(L), min(budget_rows_varlen, int(L)))[0]
            rows[(si, h)] = r
            flop_s += float(np.sum(4.0 * (r + 1) * d))     # QK^T and PV over the eligible keys
    t0 = time.perf_counter()
    dense.varlen_gqa(qh, kh, vh, cu, W.scale_f32(d), True, rows=rows)
    el = time.perf_counter() - t0
    flop_full = float(sum(2 * int(L) * int(L) * d * hq for L in lengths))
    out["varlen_gqa_8seq_32q8kv_128_bf16_causal"] = {
        "oracle_s": el, "rows": "%d seeded rows per (sequence, query head), %d in all" % (
            budget_rows_varlen, sum(len(r) for r in rows.values())),
        "oracle_TFLOPs": flop_s / el / 1e12, "estimate_full_s": flop_full / (flop_s / el),
        "note": "estimate = the workload's FLOPs at the sampled rows' rate"}
    return out


def load_traffic(src_hash, launch_bytes):
    """HBM traffic of the dominant kernel from the committed counter summary,
    only if it was taken on the current kernel sources."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    try:
        with open(PMC_SUMMARY) as fh:
            s = json.load(fh)
    except (OSError, ValueError):
        return None
    if s.get("kernel_source_sha256") != src_hash:
        return None
    return s.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-gate", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this attention path runs whole on a single MI355X "
              "(sharding across GPUs is described in the design notes, not run). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    from exact_tiled_attention_sattn_amd import sattn_fwd, library
    library()

    # A plain copy of known size (the counter-scaling reference for --pmc runs).
    cal = torch.empty(64 << 20, dtype=torch.float32, device=DEV)
    cal2 = torch.empty_like(cal)
    cal2.copy_(cal)
    torch.cuda.synchronize()
    del cal, cal2

    b, h, n, d = 4, 16, 4096, 128
    seed = W.WORKLOADS["batched_4x16x4096x128_bf16"]["seed"]
    log("generating inputs")
    q, k, v = W.qkv((b, h, n, d), (b, h, n, d), "bf16", seed)
    q, k, v = (x.to(DEV) for x in (q, k, v))
    scale = W.scale_f32(d)
    gates = {}
    if not args.no_gate:
        for causal in (False, True):
            log("correctness gate causal=%s" % causal)
            gates["causal" if causal else "noncausal"] = gate_dense(
                sattn_fwd, q, k, v, scale, causal, 16, seed, torch.bfloat16)
    o_nc = torch.empty_like(q)
    o_c = torch.empty_like(q)
    l_nc = torch.empty((b, h, n), dtype=torch.float32, device=DEV)
    l_c = torch.empty_like(l_nc)

    # Warm the GPU on the same step before the counted warmup steps: from
    # idle the chip takes tens of milliseconds of load to reach its steady
    # clock, and five steps (about 4 ms) time it partly ramping (measured on
    # one box: 1062-1070 TFLOP/s noncausal after 5 warmup steps, 1162 after
    # 200). Untimed; the timed region below is still exactly `steps` steps.
    preheat_steps = 0
    t_pre = time.perf_counter()
    while time.perf_counter() - t_pre < PREHEAT_S:
        for _ in range(8):
            sattn_fwd(q, k, v, causal=False, scale=scale, out=o_nc, lse=l_nc)
            sattn_fwd(q, k, v, causal=True, scale=scale, out=o_c, lse=l_c)
        preheat_steps += 8
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        sattn_fwd(q, k, v, causal=False, scale=scale, out=o_nc, lse=l_nc)
        sattn_fwd(q, k, v, causal=True, scale=scale, out=o_c, lse=l_c)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log("timing %d steps" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        sattn_fwd(q, k, v, causal=False, scale=scale, out=o_nc, lse=l_nc)
        e[1].record()
        e[2].record()
        sattn_fwd(q, k, v, causal=True, scale=scale, out=o_c, lse=l_c)
        e[3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_nc = [e[0].elapsed_time(e[1]) for e in ev]
    ms_c = [e[2].elapsed_time(e[3]) for e in ev]
    ms_step = wall * 1000.0 / args.steps
    f_nc, f_c = dense_flops(b, h, n, d, False), dense_flops(b, h, n, d, True)
    value = (f_nc + f_c) / (ms_step / 1000.0) / 1e12
    tf_nc = f_nc / (np.mean(ms_nc) / 1000.0) / 1e12
    tf_c = f_c / (np.mean(ms_c) / 1000.0) / 1e12
    src_hash = kernel_source_hash()
    traffic = load_traffic(src_hash, None)
    roofline = {"bound": "mfma", "achieved": tf_nc, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": tf_nc / PEAK_BF16_TFLOPS, "traffic": traffic,
                "kernel": "fwd_kernel<Bf16, D=128, BN=64, 8 waves, noncausal, dense>",
                "algorithmic_flop_per_launch": f_nc,
                "launch_ms_mean": float(np.mean(ms_nc))}
    decode_rows = {}   # host copies of decode rows for the CPU leg
    extras = {"noncausal_TFLOPs": tf_nc, "causal_TFLOPs": tf_c,
              "noncausal_frac_of_bf16_peak": tf_nc / PEAK_BF16_TFLOPS,
              "causal_frac_of_bf16_peak": tf_c / PEAK_BF16_TFLOPS,
              "noncausal_launch_ms": {"mean": float(np.mean(ms_nc)), "min": float(min(ms_nc)),
                                      "max": float(max(ms_nc))},
              "causal_launch_ms": {"mean": float(np.mean(ms_c)), "min": float(min(ms_c)), "max": float(max(ms_c))},
              "gate": gates, "kernel_source_sha256": src_hash}
    del q, k, v, o_nc, o_c
    torch.cuda.empty_cache()
    if not args.no_extras:
        log("small-shape latency")
        extras["latency_512x64_fp16_causal"] = small_latency(sattn_fwd, 512, 64, "fp16", 2, True)
        extras["latency_512x64_fp16_causal"]["pages_context"] = PAGES_CONTEXT["512x64"]
        extras["latency_512x64_fp16_noncausal"] = small_latency(sattn_fwd, 512, 64, "fp16", 2, False)
        extras["latency_129x32_fp16_causal"] = small_latency(sattn_fwd, 129, 32, "fp16", 1, True)
        extras["latency_129x32_fp16_causal"]["pages_context"] = PAGES_CONTEXT["129x32"]
        log("split-KV decode")
        extras["splitkv_decode"] = decode_extra(max(3, min(args.steps, 10)),
                                                host_rows=None if args.no_cpu_baseline else decode_rows)
        log("varlen GQA")
        extras["varlen_gqa"] = varlen_extra(max(3, min(args.steps, 10)))
        log("chunked prefill against a K/V cache")
        extras["cache_prefill"] = prefill_extra(max(3, min(args.steps, 10)))
        log("causal GQA decode against a K/V cache")
        extras["cache_gqa_decode"] = gqa_decode_extra(max(3, min(args.steps, 10)))
        log("strided (transposed) inputs")
        extras["strided_transposed"] = strided_extra(max(3, min(args.steps, 10)))
        log("sparse: window + globals, block mask")
        extras["sparse"] = sparse_extra(max(3, min(args.steps, 10)))
        log("backward")
        extras["backward"] = backward_extra(max(3, min(args.steps, 10)))
        log("backward: packed varlen GQA")
        extras["varlen_backward"] = varlen_backward_extra(max(3, min(args.steps, 10)))
        log("backward: sliding window + global tokens")
        extras["sparse_backward"] = sparse_backward_extra(max(3, min(args.steps, 10)))
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(args.cpu_budget_s)
        log("cpu oracle per workload")
        cpu["per_workload"] = cpu_oracle_per_workload(decode_rows)
    line = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "batched_4x16x4096x128_bf16: one noncausal + one causal forward per step",
                       "B": b, "H": h, "N": n, "D": d, "flop_per_step": f_nc + f_c,
                       "flop_convention": "4*N^2*D per head noncausal, 2*N^2*D causal",
                       "parallelism": "single GPU"},
            "frac_of_bf16_peak": value / PEAK_BF16_TFLOPS,
            "preheat": {"seconds": PREHEAT_S, "steps": preheat_steps,
                        "note": "untimed load on the same step before the warmup steps (clock settling)"},
            "roofline": roofline, "cpu_baseline": cpu, "extras": extras}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

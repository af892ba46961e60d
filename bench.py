#!/usr/bin/env python3
"""Throughput benchmark of the exact streaming attention forward on one MI355X.

One step = the batched multi-head forward B=4, H=16, N=4096, D=128 in bf16,
run once noncausal and once causal on the same resident inputs. FLOPs are
counted per head as 4*N^2*D noncausal and 2*N^2*D causal; ``value`` is the
step's FLOPs over its wall time (TFLOP/s).

Method, after the pages' timing rules ("Intermediate and advanced extension",
code review and execution gates, item 5; "Intermediate and advanced workshop
validation", measured examples): every timed call passes a correctness gate
first (its rows against a plain float64 computation of the definition on the
host; the FP64 oracle itself runs only in the CPU-baseline leg). The headline
step is timed with a HIP event pair around every launch, between device
synchronizations, after untimed warmup. Every other workload ("extras") is
timed as two separate experiments, with 5 warmup calls per variant and then 7
samples of 20 calls in a variant order shuffled per sample: eager calls
between HIP events, and a HIP graph of the 20 calls replayed between events.
Every raw sample is kept.

Output: one JSON line on stdout (progress goes to stderr).

Other modes:
  --variants        also time the design-variant libraries against the
                    product on the headline workload (evidence for the
                    design choices; build them with the package's build).
  --trace-summary D reads a rocprofv3 --kernel-trace --stats output
                    directory D (with --bench-log, the log of the bench run
                    it traced) and prints a markdown summary of the headline
                    kernels' timed dispatches.
  --pmc-summary F W reads FETCH_SIZE (F) and WRITE_SIZE (W) counter CSVs of
                    two bench runs (their logs: --bench-log twice, in that
                    order) and writes the traffic summary
                    profiles/fwd_kernel_batched_4x16x4096x128_bf16_pmc.{md,json}.
  --read-ceiling    times a bare streaming read of an 8 GiB device buffer
                    (libsattn_probe.so) and prints one JSON line: the read
                    bandwidth the split-KV decode is set against.
  --sq-summary D    reads a --pmc pass over the SQ counters listed in
                    SQ_COUNTERS (with --bench-log) and prints a markdown
                    summary (MFMA busy of the headline and every kernel).
"""
import argparse
import csv
import glob
import gzip
import hashlib
import json
import math
import os
import random
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "attention fwd TFLOP/s and % of bf16 MFMA peak; µs latency at N,D=512×64"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
KERNEL_SOURCES = ["exact_tiled_attention_sattn_amd/csrc/fwd_kernel.hpp",
                  "exact_tiled_attention_sattn_amd/csrc/common.hpp",
                  "exact_tiled_attention_sattn_amd/csrc/fwd_small.hpp",
                  "exact_tiled_attention_sattn_amd/csrc/fwd_decode.hpp",
                  "exact_tiled_attention_sattn_amd/csrc/launch.hpp",
                  "exact_tiled_attention_sattn_amd/csrc/k_fwd_dense.hip",
                  "exact_tiled_attention_sattn_amd/csrc/sattn.hip"]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "fwd_kernel_batched_4x16x4096x128_bf16_pmc.json")
HEADLINE_KERNELS = {"noncausal": "fwd_kernel<Bf16, 128, 64, 8, false, 0>",
                    "causal": "fwd_kernel<Bf16, 128, 64, 8, true, 0>"}
DEV = "cuda:0"
PREHEAT_S = 0.5   # untimed load on the benchmark step before its warmup steps
CALLS, SAMPLES, WARMUP = 20, 7, 5   # the pages' method: 7 samples x 20 calls, 5 warmup calls
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


def stats(xs):
    xs = [float(x) for x in xs]
    return {"median": float(statistics.median(xs)), "mean": float(statistics.fmean(xs)), "min": min(xs),
            "max": max(xs), "samples": xs}


# ------------------------------------------------------------------ timing
def time_variants(fns, calls=CALLS, samples=SAMPLES, warmup=WARMUP, graph=True, seed=0, min_warm_s=0.2):
    """The pages' timing method for a set of named variants (no-argument
    callables writing into preallocated outputs). Warmup: ``warmup`` calls of
    each, then more until ``min_warm_s`` of load has passed (clock settling).
    Experiment 1 (event): per sample, HIP events around ``calls`` eager calls
    of each variant, variant order shuffled per sample. Experiment 2 (graph):
    the ``calls`` calls of each variant captured in one HIP graph, replayed
    between events, order shuffled per sample. Returns per-variant per-call
    microseconds (median, min, max, every sample)."""
    import torch
    for fn in fns.values():
        for _ in range(warmup):
            fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_warm_s:
        for fn in fns.values():
            fn()
        torch.cuda.synchronize()
    rng = random.Random(seed)
    names = list(fns)
    ev = {n: [] for n in names}
    for _ in range(samples):
        order = names[:]
        rng.shuffle(order)
        for n in order:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(calls):
                fns[n]()
            b.record()
            b.synchronize()
            ev[n].append(a.elapsed_time(b) * 1000.0 / calls)
    out = {n: {"event_us": stats(ev[n])} for n in names}
    if not graph:
        return out
    graphs = {}
    side = torch.cuda.Stream()
    for n in names:
        g = torch.cuda.CUDAGraph()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fns[n]()
            side.synchronize()
            with torch.cuda.graph(g, stream=side):
                for _ in range(calls):
                    fns[n]()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs[n] = g
    for g in graphs.values():
        g.replay()
    torch.cuda.synchronize()
    gr = {n: [] for n in names}
    for _ in range(samples):
        order = names[:]
        rng.shuffle(order)
        for n in order:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            graphs[n].replay()
            b.record()
            b.synchronize()
            gr[n].append(a.elapsed_time(b) * 1000.0 / calls)
    for n in names:
        out[n]["graph_us"] = stats(gr[n])
    del graphs
    return out


def replay_matches(fn, outs):
    """A graph of one call of ``fn`` replays bit-identically to the eager
    result already in ``outs`` (outputs refilled with NaN in between)."""
    import torch
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    ok = True
    for _ in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ok = ok and all(torch.equal(a, b) for a, b in zip(outs, ref))
    del g
    return ok


# ------------------------------------------------------------------ gates
def gate_rows(o, lse, q, k, v, scale, causal, rows, pos, dtype, what, allowed=None):
    """Correctness gate for one (batch, head) slice: the GPU's rows ``rows``
    (query indices) against float64 torch on the host, computed directly from
    the definition for those rows only (``pos``: their logical positions,
    keys j <= pos eligible when causal; ``allowed``: an optional [R, Nk]
    eligibility; every gated row has an eligible key)."""
    import torch
    from tests.parity import check_attention
    qh = q[rows].detach().cpu().double()
    kh, vh = k.detach().cpu().double(), v.detach().cpu().double()
    s = scale * (qh @ kh.T)
    if causal:
        s = s.masked_fill(torch.arange(kh.shape[0])[None, :] > torch.as_tensor(pos)[:, None], -math.inf)
    if allowed is not None:
        s = s.masked_fill(~allowed, -math.inf)
    lse_ref = torch.logsumexp(s, dim=-1)
    o_ref = torch.exp(s - lse_ref[:, None]) @ vh
    return check_attention(o[rows], lse[rows], o_ref.numpy(), lse_ref.numpy(), dtype, what)


def worst(results):
    out = {}
    for res in results:
        for key, val in res.items():
            out[key] = max(out.get(key, 0.0), val)
    return out


def gate_dense(o, lse, q, k, v, scale, causal, heads, rows_per_head, seed, dtype, what="gate"):
    """Seeded sampled rows of the given (b, h) slices."""
    import torch
    n = q.shape[2]
    oc, lc = o.cpu(), lse.cpu()
    res = []
    for i, (b, h) in enumerate(heads):
        r = torch.from_numpy(W.sample_rows(seed * 100 + i, n, rows_per_head)[0])
        res.append(gate_rows(oc[b, h], lc[b, h], q[b, h], k[b, h], v[b, h], scale, causal, r, r, dtype, what))
    return worst(res)


def ref_grads(q, k, v, do, scale, allowed):
    """float64 gradients of sum(dO*O) for query rows q [R, D] against keys
    k, v [C, D] with eligibility ``allowed`` [R, C], from the definition:
    P = softmax over eligible keys, dP = dO V^T, Delta = rowsum(P*dP),
    dS = P*(dP - Delta), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
    dK/dV are complete only for keys whose every eligible query is a row."""
    s = np.where(allowed, scale * (q @ k.T), -np.inf)
    mx = s.max(axis=1, keepdims=True)
    p = np.exp(s - np.where(np.isfinite(mx), mx, 0.0))
    tot = p.sum(axis=1, keepdims=True)
    p = np.where(tot > 0, p / np.where(tot > 0, tot, 1.0), 0.0)
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return scale * (ds @ k), scale * (ds.T @ q), p.T @ do


def gate_grads(slices, dtype, what):
    """Backward gate. ``slices``: per KV head checked, a list of per-query-
    head tuples (q, k, v, do, o, allowed, dq_gpu, dk_gpu, dv_gpu, key_sel)
    with float64 numpy q/k/v/do/o, the GPU gradients of those rows (dq) and
    of the candidate keys (dk, dv, summed over the group by the kernel), and
    ``key_sel`` the keys whose gradients are complete. Bounds as in the GPU
    parity tests (relative rounding of the products plus the underflow
    floor)."""
    from tests.parity import grad_bounds, check_grad
    res = {}
    for group in slices:
        gq = []
        rdk = rdv = bdk = bdv = adk = adv = None
        for (q, k, v, do, o, allowed, sc, dq_g, dk_g, dv_g, key_sel) in group:
            rq, rk, rv = ref_grads(q, k, v, do, sc, allowed)
            (bq, bk, bv), (aq, ak, av) = grad_bounds(q, k, v, do, o, sc, False, allowed.astype(np.float64))
            gq.append(check_grad(dq_g, rq, bq, aq, dtype, what + " dq", verbose=False))
            if rdk is None:
                rdk, rdv, bdk, bdv, adk, adv = rk, rv, bk, bv, ak, av
            else:
                rdk, rdv, bdk, bdv, adk, adv = rdk + rk, rdv + rv, bdk + bk, bdv + bv, adk + ak, adv + av
        ks = group[0][10]
        dk_g, dv_g = group[0][8], group[0][9]
        rk_ = check_grad(dk_g[ks], rdk[ks], bdk[ks], adk[ks], dtype, what + " dk", verbose=False)
        rv_ = check_grad(dv_g[ks], rdv[ks], bdv[ks], adv[ks], dtype, what + " dv", verbose=False)
        for key, val in (("dq_err_over_bound", max(gq)), ("dk_err_over_bound", rk_), ("dv_err_over_bound", rv_)):
            res[key] = max(res.get(key, 0.0), val)
    return res


# ------------------------------------------------------------------ extras
def small_latency(fwd):
    """129x32 causal and the four 512x64 variants (causal, noncausal, each
    with Q and with Q x 16), fp16, every row gated, then timed together."""
    import torch
    fns, res = {}, {}
    for tag, n, d, seed, causal, qmul in (("129x32_fp16_causal", 129, 32, 1, True, 1.0),
                                          ("512x64_fp16_causal", 512, 64, 2, True, 1.0),
                                          ("512x64_fp16_noncausal", 512, 64, 2, False, 1.0),
                                          ("512x64_fp16_causal_q16", 512, 64, 2, True, 16.0),
                                          ("512x64_fp16_noncausal_q16", 512, 64, 2, False, 16.0)):
        q, k, v = W.qkv((1, 1, n, d), (1, 1, n, d), "fp16", seed)
        if qmul != 1.0:
            q = (q.float() * qmul).to(q.dtype)
        q, k, v = (x.to(DEV) for x in (q, k, v))
        scale = W.scale_f32(d)
        o = torch.empty_like(q)
        lse = torch.empty((1, 1, n), dtype=torch.float32, device=DEV)
        fn = (lambda q=q, k=k, v=v, causal=causal, scale=scale, o=o, lse=lse:
              fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse))
        fn()
        torch.cuda.synchronize()
        r = torch.arange(n)
        res[tag] = {"gate": gate_rows(o[0, 0].cpu(), lse[0, 0].cpu(), q[0, 0], k[0, 0], v[0, 0], scale, causal,
                                      r, r, torch.float16, "gate " + tag),
                    "graph_replay_bitwise": replay_matches(fn, [o, lse])}
        fns[tag] = fn
    t = time_variants(fns, seed=1)
    for tag in fns:
        res[tag].update(t[tag])
        res[tag]["graph_us_median"] = t[tag]["graph_us"]["median"]
        res[tag]["event_us_median"] = t[tag]["event_us"]["median"]
    res["129x32_fp16_causal"]["pages_context"] = PAGES_CONTEXT["129x32"]
    res["512x64_fp16_causal"]["pages_context"] = PAGES_CONTEXT["512x64"]
    res["512x64_q16_over_q1_graph"] = {c: res["512x64_fp16_%s_q16" % c]["graph_us_median"] /
                                       res["512x64_fp16_%s" % c]["graph_us_median"] for c in ("causal", "noncausal")}
    return res


def batched_fp16_extra(fwd):
    """The batched shape in fp16, 4x16x4096x128, N(0,1) inputs and the
    large-logit variant (Q x 16, exact in fp16), causal and noncausal:
    the cost of a changing maximum at scale."""
    import torch
    b, h, n, d = 4, 16, 4096, 128
    q, k, v = (x.to(DEV) for x in W.qkv((b, h, n, d), (b, h, n, d), "fp16", 13))
    q16 = (q.float() * 16.0).to(torch.float16)
    scale = W.scale_f32(d)
    fns, res = {}, {}
    for qtag, qq in (("q1", q), ("q16", q16)):
        for causal in (False, True):
            tag = "%s_%s" % ("causal" if causal else "noncausal", qtag)
            o = torch.empty_like(q)
            lse = torch.empty((b, h, n), dtype=torch.float32, device=DEV)
            fn = (lambda qq=qq, causal=causal, o=o, lse=lse:
                  fwd(qq, k, v, causal=causal, scale=scale, out=o, lse=lse))
            fn()
            torch.cuda.synchronize()
            res[tag] = {"gate": gate_dense(o, lse, qq, k, v, scale, causal, [(0, 0), (1, 7), (3, 15)], 24, 13,
                                           torch.float16, "gate fp16 " + tag)}
            fns[tag] = fn
    t = time_variants(fns, seed=2)
    for tag in fns:
        fl = dense_flops(b, h, n, d, tag.startswith("causal"))
        res[tag].update(t[tag])
        res[tag]["TFLOPs_graph"] = fl / t[tag]["graph_us"]["median"] / 1e6
        res[tag]["TFLOPs_event"] = fl / t[tag]["event_us"]["median"] / 1e6
        res[tag]["frac_of_fp16_peak"] = res[tag]["TFLOPs_graph"] / PEAK_BF16_TFLOPS
    res["q16_over_q1_time"] = {c: t["%s_q16" % c]["graph_us"]["median"] / t["%s_q1" % c]["graph_us"]["median"]
                               for c in ("noncausal", "causal")}
    res["workload"] = "batched_4x16x4096x128_fp16, N(0,1) (q1) and Q x 16 (q16), seed 13"
    return res


def decode_extra(cpu_leg):
    """Split-KV decode B=16, Hq=Hkv=32, Nk=131072, D=128, chunks of 4096:
    one call = sattn_fwd_split + sattn_merge. With ``cpu_leg`` the FP64
    oracle also runs on all 512 rows, each row's q, K and V slices streamed
    to the host (that is the CPU-baseline leg for this workload)."""
    import torch
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

    def both():
        split()
        merge()
    both()
    torch.cuda.synchronize()
    picks = np.random.default_rng(cfg["seed"]).choice(b * hq, size=16, replace=False)
    gate = worst(gate_rows(o[bb, h].cpu(), lse[bb, h].cpu(), q[bb, h], k[bb, h], v[bb, h], scale, False,
                           torch.tensor([0]), None, torch.bfloat16, "gate decode row %d" % f)
                 for f in picks for bb, h in [divmod(int(f), hq)])
    replay_ok = replay_matches(both, [o, lse])
    t = time_variants({"split+merge": both, "split": split, "merge": merge}, seed=3)
    kv_bytes = 2 * b * hkv * nk * d * 2
    part_bytes = b * hq * c * (d + 2) * 4
    split_bytes = kv_bytes + b * hq * d * 2 + part_bytes
    merge_bytes = part_bytes + b * hq * d * 2 + b * hq * 4
    total_bytes = kv_bytes + 2 * part_bytes + b * hq * d * 2 * 2 + b * hq * 4
    gbps = lambda by, us: by / us / 1e3  # noqa: E731
    out = {"workload": "splitkv_decode_16x32x131072x128_bf16 (chunk 4096, 32 partials per row)",
           "gate_16_rows": gate, "graph_replay_bitwise": replay_ok, "timing": t,
           "algorithmic_bytes_split": split_bytes, "algorithmic_bytes_merge": merge_bytes,
           "algorithmic_bytes_call": total_bytes}
    for exp in ("graph_us", "event_us"):
        ms = {n: t[n][exp]["median"] for n in t}
        out[exp.split("_")[0]] = {"call_GBps": gbps(total_bytes, ms["split+merge"]),
                                  "split_GBps": gbps(split_bytes, ms["split"]),
                                  "merge_GBps": gbps(merge_bytes, ms["merge"]),
                                  "split_frac_of_hbm_peak": gbps(split_bytes, ms["split"]) / PEAK_HBM_GBS,
                                  "call_frac_of_hbm_peak": gbps(total_bytes, ms["split+merge"]) / PEAK_HBM_GBS}
    out["chunk_sweep"] = chunk_sweep(q, k, v, scale, o, lse, picks[:4])
    if cpu_leg:
        out["cpu_oracle_all_rows"] = cpu_oracle_decode(q, k, v, o, lse, scale)
    del q, k, v
    torch.cuda.empty_cache()
    return out


def chunk_sweep(q, k, v, scale, o_ref, lse_ref, picks):
    """Split width against end-to-end decode bandwidth (split + merge) on the
    same resident K/V: narrow chunks launch more workgroups and write more
    partials, wide ones leave CUs idle. Each width is gated on seeded rows
    against float64 host rows and compared with the 4096-wide result (both
    lie within the bf16 tolerance of the exact value, so they differ by at
    most twice it)."""
    import torch
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
        gate = worst(gate_rows(o[bb, h].cpu(), lse[bb, h].cpu(), q[bb, h], k[bb, h], v[bb, h], scale, False,
                               torch.tensor([0]), None, torch.bfloat16, "gate chunk %d row %d" % (chunk, f))
                     for f in picks for bb, h in [divmod(int(f), hq)])
        t = time_variants({"call": both}, calls=5, samples=5, warmup=2, seed=4, min_warm_s=0.05)["call"]
        part_bytes = b * hq * c * (d + 2) * 4
        total = kv_bytes + 2 * part_bytes + b * hq * d * 2 * 2 + b * hq * 4
        res.append({"chunk": chunk, "partials_per_row": c, "split_workgroups": b * hq * c, "gate": gate,
                    "timing": t, "end_to_end_GBps_graph": total / t["graph_us"]["median"] / 1e3,
                    "end_to_end_GBps_event": total / t["event_us"]["median"] / 1e3})
        del pm, pl, pa
    return res


def varlen_extra():
    """Packed variable-length causal GQA forward (8 seeded lengths, 32 query
    heads on 8 KV heads, D = 128, bf16); the host copy of cu_seqlens is
    passed so that a call does not synchronize."""
    import torch
    from exact_tiled_attention_sattn_amd import sattn_fwd_varlen
    cfg = W.WORKLOADS["varlen_gqa_8seq_32q8kv_128_bf16_causal"]
    lengths = W.varlen_lengths(cfg["seed"], cfg["S"], cfg["max_len"])
    hq, hkv, d = cfg["Hq"], cfg["Hkv"], cfg["D"]
    t = int(lengths.sum())
    q, k, v = W.qkv((t, hq, d), (t, hkv, d), "bf16", cfg["seed"])
    q, k, v = (x.to(DEV) for x in (q, k, v))
    cu_h = W.cu_seqlens_of(lengths)
    cu = torch.from_numpy(cu_h).to(DEV)
    mx = int(lengths.max())
    scale = W.scale_f32(d)
    o = torch.empty_like(q)
    lse = torch.empty((hq, t), dtype=torch.float32, device=DEV)
    fn = lambda: sattn_fwd_varlen(q, k, v, cu, max_seqlen=mx, causal=True, scale=scale, out=o, lse=lse,  # noqa
                                  cu_seqlens_host=cu_h)
    fn()
    torch.cuda.synchronize()
    oc, lc = o.cpu(), lse.cpu()
    res = []
    for s, L in enumerate(lengths):
        a = int(cu_h[s])
        for h in (0, 13, 31):
            r = torch.from_numpy(W.sample_rows(5000 + s * 64 + h, int(L), 16)[0])
            res.append(gate_rows(oc[a:a + L, h], lc[h, a:a + L], q[a:a + L, h], k[a:a + L, h // 4],
                                 v[a:a + L, h // 4], scale, True, r, r, torch.bfloat16, "gate varlen"))
    replay_ok = replay_matches(fn, [o, lse])
    tm = time_variants({"call": fn}, seed=5)["call"]
    flops = sum(2 * int(L) * int(L) * d * hq for L in lengths)
    return {"workload": "varlen_gqa_8seq_32q8kv_128_bf16_causal", "lengths": lengths.tolist(), "T": t,
            "gate": worst(res), "graph_replay_bitwise": replay_ok, "timing": tm, "flop": flops,
            "TFLOPs_graph": flops / tm["graph_us"]["median"] / 1e6,
            "TFLOPs_event": flops / tm["event_us"]["median"] / 1e6,
            "frac_of_bf16_peak": flops / tm["graph_us"]["median"] / 1e6 / PEAK_BF16_TFLOPS}


def prefill_extra():
    """One 2048-query chunk of a chunked prefill against a 16384-token K/V
    cache (query i at position i + 14336), 32 query heads on 8 KV heads,
    bf16, causal. FLOPs count eligible (query, key) pairs at 4*D each, with
    the diagonal term dropped as in the dense convention."""
    import torch
    from exact_tiled_attention_sattn_amd import sattn_fwd_cache
    b, hq, hkv, nq, nk, d = 1, 32, 8, 2048, 16384, 128
    q, k, v = (x.to(DEV) for x in W.qkv((b, hq, nq, d), (b, hkv, nk, d), "bf16", 7))
    scale = W.scale_f32(d)
    o = torch.empty_like(q)
    lse = torch.empty((b, hq, nq), dtype=torch.float32, device=DEV)
    fn = lambda: sattn_fwd_cache(q, k, v, causal=True, scale=scale, out=o, lse=lse)  # noqa: E731
    fn()
    torch.cuda.synchronize()
    oc, lc = o.cpu(), lse.cpu()
    res = []
    for h in (0, 13, 31):
        rows = torch.from_numpy(W.sample_rows(700 + h, nq, 12)[0])
        res.append(gate_rows(oc[0, h], lc[0, h], q[0, h], k[0, h // 4], v[0, h // 4], scale, True, rows,
                             rows + nk - nq, torch.bfloat16, "gate prefill"))
    replay_ok = replay_matches(fn, [o, lse])
    tm = time_variants({"call": fn}, seed=6)["call"]
    off = nk - nq
    flops = 4 * d * (nq * off + nq * nq // 2) * b * hq
    del q, k, v, o
    torch.cuda.empty_cache()
    return {"workload": "chunked prefill: 2048 queries vs 16384-token cache, 32q/8kv heads, D=128 bf16 causal",
            "gate": worst(res), "graph_replay_bitwise": replay_ok, "timing": tm, "flop": flops,
            "TFLOPs_graph": flops / tm["graph_us"]["median"] / 1e6,
            "TFLOPs_event": flops / tm["event_us"]["median"] / 1e6,
            "frac_of_bf16_peak": flops / tm["graph_us"]["median"] / 1e6 / PEAK_BF16_TFLOPS}


def read_ceiling(gib=8, grids=(1024, 2048, 4096, 8192)):
    """A bare streaming read of a resident ``gib`` GiB device buffer (the
    probe library's 16-byte nontemporal loads, one contiguous slice per
    workgroup), graph- and
    event-timed like the extras: the bandwidth the split-KV decode is set
    against. Nothing of the attention path runs here."""
    import ctypes
    import torch
    from exact_tiled_attention_sattn_amd.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        raise SystemExit("%s is missing: build the package first" % PROBE_LIB)
    lib = ctypes.CDLL(PROBE_LIB)
    lib.sattn_probe_read.restype = ctypes.c_int
    lib.sattn_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_void_p]
    nbytes = gib << 30
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
    out = torch.empty(max(grids) * 256, dtype=torch.int32, device=DEV)
    fns = {}
    for g in grids:
        def fn(g=g):
            rc = lib.sattn_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
                                      out.numel(), g, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError("sattn_probe_read failed (%d)" % rc)
        fns["grid %d" % g] = fn
    t = time_variants(fns, seed=3)
    res = {"workload": "streaming read of a resident %d GiB buffer, 16-byte nontemporal loads" % gib,
           "bytes": nbytes, "timing": t}
    res["GBps_graph"] = {n: nbytes / t[n]["graph_us"]["median"] / 1e3 for n in fns}
    res["best_GBps_graph"] = max(res["GBps_graph"].values())
    res["best_frac_of_hbm_peak"] = res["best_GBps_graph"] / PEAK_HBM_GBS
    del buf, out
    torch.cuda.empty_cache()
    return res


def gqa_token_decode_extra():
    """Single-token decode with grouped KV heads: 1 query per head against a
    32768-token K/V cache, B=16, 32 query heads on 8 KV heads, D=128 bf16,
    chunks of 2048 (split partials, then the merge). Bytes count K/V once."""
    import torch
    from exact_tiled_attention_sattn_amd import sattn_fwd_split, sattn_merge
    b, hq, hkv, nq, nk, d, chunk = 16, 32, 8, 1, 32768, 128, 2048
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
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
    split = lambda: sattn_fwd_split(q, k, v, chunk, scale, part_m=pm, part_l=pl, part_acc=pa)  # noqa: E731
    merge = lambda: sattn_merge(pm, pl, pa, torch.bfloat16, out=o, lse=lse)  # noqa: E731

    def both():
        split()
        merge()
    both()
    torch.cuda.synchronize()
    rows = torch.arange(nq)
    grp = hq // hkv
    gate = worst(gate_rows(o[bb, h].cpu(), lse[bb, h].cpu(), q[bb, h], k[bb, h // grp], v[bb, h // grp], scale,
                           False, rows, rows + nk - nq, torch.bfloat16, "gate gqa token decode")
                 for bb, h in ((0, 0), (6, 13), (15, 31)))
    replay_ok = replay_matches(both, [o, lse])
    t = time_variants({"split+merge": both, "split": split, "merge": merge}, seed=9)
    kv_bytes = 2 * b * hkv * nk * d * 2
    part_bytes = b * hq * nq * c * (d + 2) * 4
    split_bytes = kv_bytes + b * hq * nq * d * 2 + part_bytes
    del q, k, v
    torch.cuda.empty_cache()
    return {"workload": "GQA single-token decode: 1 query per head vs 32768-token cache, B=16, 32q/8kv heads, "
                        "D=128 bf16, chunk 2048",
            "gate": gate, "graph_replay_bitwise": replay_ok, "timing": t, "algorithmic_bytes_split": split_bytes,
            "split_GBps_graph": split_bytes / t["split"]["graph_us"]["median"] / 1e3,
            "split_frac_of_hbm_peak": split_bytes / t["split"]["graph_us"]["median"] / 1e3 / PEAK_HBM_GBS,
            "merge_us_graph": t["merge"]["graph_us"]["median"]}


def gqa_decode_extra():
    """Causal decode of 4 new tokens per sequence against a 32768-token K/V
    cache: B=8, 32 query heads on 8 KV heads, D=128 bf16, chunks of 2048
    (causal split partials, then the merge). Bytes count K/V once."""
    import torch
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

    def both():
        split()
        merge()
    both()
    torch.cuda.synchronize()
    rows = torch.arange(nq)
    gate = worst(gate_rows(o[bb, h].cpu(), lse[bb, h].cpu(), q[bb, h], k[bb, h // 4], v[bb, h // 4], scale, True,
                           rows, rows + nk - nq, torch.bfloat16, "gate gqa decode")
                 for bb, h in ((0, 0), (5, 17), (7, 31)))
    replay_ok = replay_matches(both, [o, lse])
    t = time_variants({"split+merge": both, "split": split, "merge": merge}, seed=7)
    kv_bytes = 2 * b * hkv * nk * d * 2
    part_bytes = b * hq * nq * c * (d + 2) * 4
    split_bytes = kv_bytes + b * hq * nq * d * 2 + part_bytes
    del q, k, v
    torch.cuda.empty_cache()
    return {"workload": "causal GQA decode: 4 queries vs 32768-token cache, B=8, 32q/8kv heads, D=128 bf16, "
                        "chunk 2048",
            "gate": gate, "graph_replay_bitwise": replay_ok, "timing": t, "algorithmic_bytes_split": split_bytes,
            "split_GBps_graph": split_bytes / t["split"]["graph_us"]["median"] / 1e3,
            "split_frac_of_hbm_peak": split_bytes / t["split"]["graph_us"]["median"] / 1e3 / PEAK_HBM_GBS,
            "merge_us_graph": t["merge"]["graph_us"]["median"]}


def strided_extra():
    """Transposed inputs: q, k, v stored [B, N, H, D] (B=4, H=16, N=4096,
    D=128 bf16) and viewed as [B, H, N, D]. Loaded in place by
    sattn_fwd_strided, against copying them to [B, H, N, D] first and running
    the same kernel on the copies (the copy inside the timing, as in the
    pages' strided-input comparison)."""
    import torch
    from exact_tiled_attention_sattn_amd import sattn_fwd_strided, sattn_fwd_cache
    b, h, n, d = 4, 16, 4096, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    q, k, v = (W.randn_device_sliced((b, n, h, d), "bf16", g, DEV).permute(0, 2, 1, 3) for _ in range(3))
    scale = W.scale_f32(d)
    res = {"workload": "transposed [B,N,H,D] inputs viewed as [B,H,N,D], 4x16x4096x128 bf16"}
    fns = {}
    for causal in (False, True):
        tag = "causal" if causal else "noncausal"
        o = torch.empty((b, h, n, d), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((b, h, n), dtype=torch.float32, device=DEV)
        o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
        direct = (lambda causal=causal, o=o, lse=lse:
                  sattn_fwd_strided(q, k, v, causal=causal, scale=scale, out=o, lse=lse))
        copied = (lambda causal=causal, o=o2, lse=lse2:
                  sattn_fwd_cache(q.contiguous(), k.contiguous(), v.contiguous(), causal=causal, scale=scale,
                                  out=o, lse=lse))
        direct()
        copied()
        torch.cuda.synchronize()
        r = torch.from_numpy(W.sample_rows(900, n, 12)[0])
        res[tag] = {"gate_direct": gate_rows(o[1, 5].cpu(), lse[1, 5].cpu(), q[1, 5], k[1, 5], v[1, 5], scale,
                                             causal, r, r, torch.bfloat16, "gate strided"),
                    "direct_equals_copy_bitwise": bool(torch.equal(o, o2) and torch.equal(lse, lse2))}
        fns["direct_" + tag] = direct
        fns["copy_then_kernel_" + tag] = copied
    t = time_variants(fns, seed=8)
    for causal in (False, True):
        tag = "causal" if causal else "noncausal"
        fl = dense_flops(b, h, n, d, causal)
        res[tag].update({"direct": t["direct_" + tag], "copy_then_kernel": t["copy_then_kernel_" + tag],
                         "direct_TFLOPs_graph": fl / t["direct_" + tag]["graph_us"]["median"] / 1e6,
                         "copy_then_kernel_TFLOPs_graph": fl / t["copy_then_kernel_" + tag]["graph_us"]["median"]
                         / 1e6})
    del q, k, v
    torch.cuda.empty_cache()
    return res


def window_pairs(n, w, ng):
    """Kept (query, key) pairs of a causal window of w keys united with ng
    global tokens, per head."""
    tot = 0
    for i in range(n):
        if i < ng:
            tot += i + 1
        else:
            lo = max(0, i - w + 1)
            tot += (i - lo + 1) + min(ng, lo)
    return tot


def window_allowed(rows, keys, w, ng):
    """Eligibility of the causal window + global tokens rule."""
    import torch
    j = torch.as_tensor(keys)[None, :]
    p = torch.as_tensor(rows)[:, None]
    return (j <= p) & ((j >= p - (w - 1)) | (j < ng) | (p < ng))


def sparse_extra():
    """Changed operators (lessons 06 and 07): work counts kept (query, key)
    pairs at 4*D FLOP each.
    * causal sliding window of 2048 keys united with 64 global tokens,
      B=1, H=16, N=16384, D=128 bf16;
    * block-sparse, non-causal, 64x64 blocks, a seeded per-head mask with a
      quarter of the blocks active, B=1, H=16, N=8192, D=128 bf16."""
    import torch
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
    rows = torch.tensor([0, 63, 64, 5000, 9999, n - 1])
    gate = gate_rows(o[0, 3].cpu(), lse[0, 3].cpu(), q[0, 3], k[0, 3], v[0, 3], scale, False, rows, None,
                     torch.bfloat16, "gate window", allowed=window_allowed(rows, np.arange(n), w, ng))
    replay_ok = replay_matches(fn, [o, lse])
    tm = time_variants({"call": fn}, seed=9)["call"]
    pairs = window_pairs(n, w, ng) * h
    res["causal_window2048_global64_16x16384x128_bf16"] = {
        "gate": gate, "graph_replay_bitwise": replay_ok, "timing": tm, "kept_pairs": pairs,
        "TFLOPs_graph": 4 * d * pairs / tm["graph_us"]["median"] / 1e6,
        "frac_of_bf16_peak": 4 * d * pairs / tm["graph_us"]["median"] / 1e6 / PEAK_BF16_TFLOPS}
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
    rows = torch.tensor([0, 1000, 4000, 7777, n - 1])
    allowed = bm[5][rows // 64].repeat_interleave(64, dim=1).bool()
    ok = allowed.any(dim=1)
    gate = gate_rows(o[0, 5].cpu(), lse[0, 5].cpu(), q[0, 5], k[0, 5], v[0, 5], scale, False, rows[ok], None,
                     torch.bfloat16, "gate block-sparse", allowed=allowed[ok])
    replay_ok = replay_matches(fn, [o, lse])
    tm = time_variants({"call": fn}, seed=10)["call"]
    pairs = int(bm.sum()) * 64 * 64
    res["block_sparse_quarter_64x64_16x8192x128_bf16"] = {
        "gate": gate, "graph_replay_bitwise": replay_ok, "timing": tm, "active_block_pairs": int(bm.sum()),
        "kept_pairs": pairs, "TFLOPs_graph": 4 * d * pairs / tm["graph_us"]["median"] / 1e6,
        "frac_of_bf16_peak": 4 * d * pairs / tm["graph_us"]["median"] / 1e6 / PEAK_BF16_TFLOPS}
    del q, k, v, o
    torch.cuda.empty_cache()
    return res


def _f64(x):
    return W.to_f64(x)


def backward_extra():
    """Backward (dQ, dK, dV) of the batched 4x16x4096x128 bf16 workload,
    causal and non-causal, on the forward's own O and lse. Gate: one whole
    head per variant against float64 gradients from the definition. FLOPs
    follow the usual convention of five N^2*D products (2.5x the forward:
    10*N^2*D per head non-causal, 5*N^2*D causal); the two-kernel schedule
    here executes seven (S and dP are recomputed by both kernels)."""
    import torch
    from exact_tiled_attention_sattn_amd import sattn_fwd, sattn_bwd
    b, h, n, d = 4, 16, 4096, 128
    q, k, v = (x.to(DEV) for x in W.qkv((b, h, n, d), (b, h, n, d), "bf16", 3))
    do = W.randn((b, h, n, d), "bf16", torch.Generator().manual_seed(33)).to(DEV)
    scale = W.scale_f32(d)
    res = {"workload": "backward of batched_4x16x4096x128_bf16",
           "flop_convention": "10*N^2*D per head noncausal, 5*N^2*D causal (2.5x forward)"}
    fns = {}
    for causal in (False, True):
        tag = "causal" if causal else "noncausal"
        o, lse = sattn_fwd(q, k, v, causal=causal, scale=scale)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty((b, h, n), dtype=torch.float32, device=DEV)
        fn = (lambda o=o, lse=lse, causal=causal, dq=dq, dk=dk, dv=dv, delta=delta:
              sattn_bwd(q, k, v, o, do, lse, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv, delta=delta))
        fn()
        torch.cuda.synchronize()
        bi, hi = (1, 5) if causal else (2, 9)
        allowed = np.tril(np.ones((n, n), dtype=bool)) if causal else np.ones((n, n), dtype=bool)
        sl = [(_f64(q[bi, hi]), _f64(k[bi, hi]), _f64(v[bi, hi]), _f64(do[bi, hi]), _f64(o[bi, hi]), allowed,
               scale, dq[bi, hi], _f64(dk[bi, hi]), _f64(dv[bi, hi]), slice(None))]
        res[tag] = {"gate_head_%d_%d" % (bi, hi): gate_grads([sl], torch.bfloat16, "gate bwd " + tag),
                    "graph_replay_bitwise": replay_matches(fn, [dq, dk, dv])}
        fns[tag] = fn
    t = time_variants(fns, seed=11)
    for causal in (False, True):
        tag = "causal" if causal else "noncausal"
        fl = 2.5 * dense_flops(b, h, n, d, causal)
        us = t[tag]["graph_us"]["median"]
        res[tag].update({"timing": t[tag], "TFLOPs_graph": fl / us / 1e6,
                         "frac_of_bf16_peak": fl / us / 1e6 / PEAK_BF16_TFLOPS,
                         "executed_TFLOPs_graph": 3.5 * dense_flops(b, h, n, d, causal) / us / 1e6})
    del q, k, v, do
    torch.cuda.empty_cache()
    return res


def varlen_backward_extra():
    """Backward of the packed varlen GQA workload (8 seeded sequence lengths,
    32 query heads on 8 KV heads, D = 128, bf16, causal) on the forward's own
    O and lse. Gate: KV head 3 (query heads 12-15) of two sequences, whole,
    against float64 gradients. FLOPs: 2.5x the forward's causal count."""
    import torch
    from exact_tiled_attention_sattn_amd import sattn_fwd_varlen, sattn_bwd_varlen
    cfg = W.WORKLOADS["varlen_gqa_8seq_32q8kv_128_bf16_causal"]
    lengths = W.varlen_lengths(cfg["seed"], cfg["S"], cfg["max_len"])
    hq, hkv, d = cfg["Hq"], cfg["Hkv"], cfg["D"]
    t = int(lengths.sum())
    q, k, v = (x.to(DEV) for x in W.qkv((t, hq, d), (t, hkv, d), "bf16", cfg["seed"]))
    do = W.randn((t, hq, d), "bf16", torch.Generator().manual_seed(cfg["seed"] + 1)).to(DEV)
    cu_h = W.cu_seqlens_of(lengths)
    cu = torch.from_numpy(cu_h).to(DEV)
    mx = int(lengths.max())
    scale = W.scale_f32(d)
    o, lse = sattn_fwd_varlen(q, k, v, cu, max_seqlen=mx, causal=True, scale=scale, cu_seqlens_host=cu_h)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((hq, t), dtype=torch.float32, device=DEV)
    fn = lambda: sattn_bwd_varlen(q, k, v, o, do, lse, cu, max_seqlen=mx, causal=True, scale=scale,  # noqa: E731
                                  dq=dq, dk=dk, dv=dv, delta=delta, cu_seqlens_host=cu_h)
    fn()
    torch.cuda.synchronize()
    groups = []
    g = 3
    for s in (2, 7):
        a, e = int(cu_h[s]), int(cu_h[s + 1])
        L = e - a
        allowed = np.tril(np.ones((L, L), dtype=bool))
        groups.append([(_f64(q[a:e, hh]), _f64(k[a:e, g]), _f64(v[a:e, g]), _f64(do[a:e, hh]), _f64(o[a:e, hh]),
                        allowed, scale, dq[a:e, hh], _f64(dk[a:e, g]), _f64(dv[a:e, g]), slice(None))
                       for hh in range(4 * g, 4 * g + 4)])
    gate = gate_grads(groups, torch.bfloat16, "gate varlen bwd")
    replay_ok = replay_matches(fn, [dq, dk, dv])
    tm = time_variants({"call": fn}, seed=12)["call"]
    flops = 2.5 * sum(2 * int(L) * int(L) * d * hq for L in lengths)
    del q, k, v, do, dq, dk, dv, o
    torch.cuda.empty_cache()
    return {"workload": "backward of varlen_gqa_8seq_32q8kv_128_bf16_causal", "T": t,
            "gate_kv_head_3_seqs_2_7": gate, "graph_replay_bitwise": replay_ok, "timing": tm,
            "TFLOPs_graph": flops / tm["graph_us"]["median"] / 1e6,
            "frac_of_bf16_peak": flops / tm["graph_us"]["median"] / 1e6 / PEAK_BF16_TFLOPS,
            "flop_convention": "2.5x the forward's causal 2*L^2*D per query head"}


def sparse_backward_extra():
    """Backward of the causal sliding window (2048 keys) united with 64
    global tokens, B=1, H=16, N=16384, D=128 bf16, on the forward's own O and
    lse. Gate (head 6): dK/dV of keys [8192, 8448) and dQ of every query that
    sees them, queries [8192, 10495), against float64 gradients over all of
    those queries' eligible keys. FLOPs: 2.5x the forward's kept pairs."""
    import torch
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
    k0, kb = 8192, 256
    rows = np.arange(k0, k0 + kb + w - 1)
    cand = np.concatenate([np.arange(ng), np.arange(k0 - (w - 1), rows[-1] + 1)])
    allowed = window_allowed(rows, cand, w, ng).numpy()
    sel = np.nonzero((cand >= k0) & (cand < k0 + kb))[0]
    hh = 6
    r_t, c_t = torch.from_numpy(rows), torch.from_numpy(cand)
    hq_ = lambda x: x[0, hh].cpu()  # noqa: E731
    sl = [(_f64(hq_(q)[r_t]), _f64(hq_(k)[c_t]), _f64(hq_(v)[c_t]), _f64(hq_(do)[r_t]), _f64(hq_(o)[r_t]),
           allowed, scale, hq_(dq)[r_t], _f64(hq_(dk)[c_t]), _f64(hq_(dv)[c_t]), sel)]
    gate = gate_grads([sl], torch.bfloat16, "gate sparse bwd")
    replay_ok = replay_matches(fn, [dq, dk, dv])
    tm = time_variants({"call": fn}, seed=13)["call"]
    pairs = window_pairs(n, w, ng) * h
    del q, k, v, do, dq, dk, dv, o
    torch.cuda.empty_cache()
    fl = 2.5 * 4 * d * pairs
    return {"workload": "backward of causal_window2048_global64_16x16384x128_bf16", "gate_head_6": gate,
            "graph_replay_bitwise": replay_ok, "timing": tm, "TFLOPs_graph": fl / tm["graph_us"]["median"] / 1e6,
            "frac_of_bf16_peak": fl / tm["graph_us"]["median"] / 1e6 / PEAK_BF16_TFLOPS,
            "flop_convention": "2.5x the forward's kept pairs at 4*D"}


# ------------------------------------------------------------------ variants
def variants_leg():
    """Design variants against the product on the headline workload: each
    variant library (one design choice changed, built beside the product) is
    loaded with ctypes, gated (bit-equality with the product where the
    arithmetic order is the same, else sampled rows against float64), and
    timed with the product in one shuffled order, both experiments."""
    import ctypes
    import torch
    from exact_tiled_attention_sattn_amd import LIB_PATH
    from exact_tiled_attention_sattn_amd import build as B
    libs = {"product": LIB_PATH}
    for name in B.VARIANTS:
        if os.path.exists(B.variant_path(name)):
            libs[name] = B.variant_path(name)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    handles = {}
    for name, path in libs.items():
        lib = ctypes.CDLL(path)
        lib.sattn_fwd.restype = ctypes.c_int
        lib.sattn_fwd.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                  ctypes.c_float, vp]
        handles[name] = lib
    b, h, n, d = 4, 16, 4096, 128
    seed = W.WORKLOADS["batched_4x16x4096x128_bf16"]["seed"]
    q, k, v = (x.to(DEV) for x in W.qkv((b, h, n, d), (b, h, n, d), "bf16", seed))
    scale = W.scale_f32(d)

    def caller(lib, causal, o, lse):
        def fn():
            rc = lib.sattn_fwd(1, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), b, h, n,
                               d, int(causal), scale, vp(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError("variant call failed: %d" % rc)
        return fn
    res = {"workload": "batched_4x16x4096x128_bf16", "libraries": {k_: os.path.basename(p) for k_, p in libs.items()}}
    for causal in (False, True):
        tag = "causal" if causal else "noncausal"
        fns, outs = {}, {}
        for name, lib in handles.items():
            o = torch.empty_like(q)
            lse = torch.empty((b, h, n), dtype=torch.float32, device=DEV)
            fns[name] = caller(lib, causal, o, lse)
            fns[name]()
            outs[name] = (o, lse)
        torch.cuda.synchronize()
        gates = {}
        o0, l0 = outs["product"]
        for name, (o, lse) in outs.items():
            gates[name] = {"bitwise_equal_to_product": bool(torch.equal(o, o0) and torch.equal(lse, l0)),
                           "max_abs_diff_o": float((o.float() - o0.float()).abs().max()),
                           "max_abs_diff_lse": float((lse - l0).abs().max())}
            try:
                gates[name]["gate"] = gate_dense(o, lse, q, k, v, scale, causal, [(0, 0), (3, 15)], 16, seed,
                                                 torch.bfloat16, "gate variant " + name)
            except AssertionError as exc:     # a failed variant is reported, never timed
                if name == "product":
                    raise
                gates[name]["gate_failed"] = str(exc)
                log("variant %s failed its gate: %s" % (name, exc))
                fns.pop(name)
        t = time_variants(fns, seed=20 + int(causal), samples=12)
        fl = dense_flops(b, h, n, d, causal)
        res[tag] = {name: {"gate": gates[name], "timing": t[name],
                           "TFLOPs_graph": fl / t[name]["graph_us"]["median"] / 1e6,
                           "TFLOPs_event": fl / t[name]["event_us"]["median"] / 1e6,
                           "vs_product_graph": t["product"]["graph_us"]["median"] / t[name]["graph_us"]["median"]}
                    for name in fns}
        res[tag].update({name: {"gate": gates[name]} for name in gates if name not in fns})
        log("variants %s: %s" % (tag, ", ".join("%s %.0f" % (nm, r["TFLOPs_graph"]) for nm, r in res[tag].items()
                                                if "TFLOPs_graph" in r)))
    return res


# ------------------------------------------------------------------ CPU leg
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


def cpu_oracle_decode(q, k, v, o, lse, scale):
    """CPU-baseline leg of the split-KV decode: the FP64 oracle on every one
    of the 512 rows, each row's q, K and V slices (64 MiB) streamed from the
    device to the host in turn; also compares each row with the GPU result."""
    import torch
    from oracle import dense
    from tests.parity import TOL, LSE_ATOL
    atol, rtol = TOL[torch.bfloat16]
    b, hq = q.shape[0], q.shape[1]
    t_d2h = t_conv = t_orc = 0.0
    worst_ratio = worst_lse = 0.0
    oc, lc = o.float().cpu().numpy(), lse.cpu().numpy()
    for bb in range(b):
        for h in range(hq):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            qs, ks, vs = q[bb, h].cpu(), k[bb, h].cpu(), v[bb, h].cpu()
            t1 = time.perf_counter()
            qd, kd, vd = W.to_f64(qs), W.to_f64(ks), W.to_f64(vs)
            t2 = time.perf_counter()
            o_ref, l_ref = dense.attention(qd, kd, vd, scale, False)
            t3 = time.perf_counter()
            t_d2h, t_conv, t_orc = t_d2h + t1 - t0, t_conv + t2 - t1, t_orc + t3 - t2
            err = np.abs(oc[bb, h] - o_ref)
            worst_ratio = max(worst_ratio, float((err / (atol + rtol * np.abs(o_ref))).max()))
            worst_lse = max(worst_lse, float(np.abs(lc[bb, h] - l_ref).max()))
    rows = b * hq
    if worst_ratio > 1.0 or worst_lse > LSE_ATOL:
        raise RuntimeError("decode: a row disagrees with the oracle (err/bound %.3f, lse %.3g)"
                           % (worst_ratio, worst_lse))
    return {"rows": rows, "oracle_s": t_orc, "oracle_ms_per_row": t_orc * 1e3 / rows,
            "bf16_to_f64_s": t_conv, "d2h_s": t_d2h, "d2h_bytes": rows * (2 * 131072 * 128 * 2 + 128 * 2),
            "all_rows_o_err_over_bound": worst_ratio, "all_rows_lse_max_err": worst_lse,
            "note": "oracle time excludes the device-to-host copy and the exact bf16 -> float64 conversion, "
                    "reported apart"}


def cpu_oracle_per_workload(budget_rows_varlen=64):
    """The FP64 oracle on the other workloads, timed on the host cores: the
    two small shapes in full (median of 5), the packed varlen workload on
    seeded rows per (sequence, query head), scaled to the full workload by
    FLOPs and labelled as an estimate. (The decode runs in full inside the
    decode extra, while its K/V are resident.)"""
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


def load_traffic(src_hash):
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


# ------------------------------------------------------------ profile summaries
def _read_csv(pattern):
    """Rows of the first file matching ``pattern`` or ``pattern + '.gz'``."""
    files = sorted(glob.glob(pattern, recursive=True) + glob.glob(pattern + ".gz", recursive=True))
    if not files:
        raise SystemExit("no file matches %s" % pattern)
    opener = gzip.open if files[0].endswith(".gz") else open
    with opener(files[0], "rt") as fh:
        return list(csv.DictReader(fh)), files[0]


def _kname(name):
    """A kernel name as the traces print it, without namespaces and spaces."""
    return name.replace("sattn::", "").replace(" ", "")


def _disp(name):
    """A kernel name for the summaries' tables: no namespace, return type or
    parameter list."""
    n = name.replace("sattn::", "")
    n = n[5:] if n.startswith("void ") else n
    return n.split("(")[0].replace("|", "/")[:110]


def _dispatches(per, key):
    """(dispatch id, value) of every kernel whose name contains ``key``."""
    k_ = _kname(key)
    return sorted(x for name, xs in per.items() if k_ in _kname(name) for x in xs)


def _bench_line(path):
    with open(path) as fh:
        for line in fh:
            if line.startswith('{"metric"'):
                return json.loads(line)
    raise SystemExit("no bench JSON line in %s" % path)


def trace_summary(trace_dir, bench_log, command):
    """Markdown summary of a rocprofv3 kernel trace of one bench.py run: the
    headline kernels' timed dispatches (identified by their order: the JSON
    line records how many launches of each came before the timed steps),
    against the same run's HIP-event figures, plus every kernel's stats."""
    rows, path = _read_csv(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    line = _bench_line(bench_log)
    ex = line["extras"]
    steps = line["steps"]
    per = {}
    for r in rows:
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    out = ["# Kernel trace of one bench.py run: batched 4x16x4096x128 bf16 forward", "",
           "Command (MI355X, one GPU):", "", "    " + command, "",
           "kernel_source_sha256: `%s`" % ex["kernel_source_sha256"], "",
           "## Headline kernels, timed dispatches only", "",
           "The bench line records how many launches of each headline kernel came before its timed steps "
           "(correctness gate, preheat, warmup); the timed dispatches are the next `steps` = %d of that kernel "
           "in dispatch order." % steps, "",
           "| launch | kernel | timed dispatches | trace mean us | trace median us | bench events mean us | "
           "bench events median us | trace TFLOP/s (mean) | frac of 2.5 PFLOP/s |", "|---|---|---|---|---|---|---|---|---|"]
    summ = {}
    for tag, kname in HEADLINE_KERNELS.items():
        ds = _dispatches(per, kname)
        skip = ex["launches_before_timing"][tag]
        timed = [us for _, us in ds[skip:skip + steps]]
        if len(timed) != steps:
            raise SystemExit("trace has %d timed dispatches of %s, expected %d" % (len(timed), kname, steps))
        ev = ex["%s_launch_ms" % tag]
        fl = line["config"]["flop_per_launch"][tag]
        tm = statistics.fmean(timed)
        summ[tag] = {"mean": tm, "median": statistics.median(timed), "samples": timed}
        out.append("| %s | `%s` | %d | %.2f | %.2f | %.2f | %.2f | %.1f | %.4f |" % (
            tag, kname, steps, tm, statistics.median(timed), ev["mean"] * 1e3, ev["median"] * 1e3,
            fl / tm / 1e6, fl / tm / 1e6 / PEAK_BF16_TFLOPS))
    step_sum = [a + b for a, b in zip(summ["noncausal"]["samples"], summ["causal"]["samples"])]
    out += ["", "Per step, the two timed kernels sum to %.2f us on average (max %.2f); the bench's ms_per_step "
            "(wall clock over the timed steps, between synchronizations) is %.2f us." % (
                statistics.fmean(step_sum), max(step_sum), line["ms_per_step"] * 1e3),
            "The bench line's roofline: achieved %.1f TFLOP/s, frac %.4f (events, mean over the timed launches)." % (
                line["roofline"]["achieved"], line["roofline"]["frac"]), "",
            "## Every kernel of the run (all dispatches, warm-up included)", "",
            "| kernel | dispatches | mean us | median us | min us | max us |", "|---|---|---|---|---|---|"]
    for kname, ds in sorted(per.items(), key=lambda kv: -sum(u for _, u in kv[1])):
        us = [u for _, u in ds]
        out.append("| `%s` | %d | %.2f | %.2f | %.2f | %.2f |" % (_disp(kname), len(us),
                                                                 statistics.fmean(us), statistics.median(us),
                                                                 min(us), max(us)))
    out += ["", "Source: `%s` (rocprofv3 --kernel-trace --stats)." % os.path.relpath(path, trace_dir)]
    return "\n".join(out) + "\n"


def _counter_per_kernel(d, counter):
    """{kernel name: [(dispatch id, value)]} of one counter in a rocprofv3
    --pmc output directory."""
    rows, _ = _read_csv(os.path.join(d, "**", "*counter_collection.csv"))
    per = {}
    for r in rows:
        if r["Counter_Name"] == counter:
            per.setdefault(r["Kernel_Name"], []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return per


# Kernels of the extras whose algorithmic bytes the bench line records:
# (workload, kernel, (extras leg, key)). The chunk-width sweep launches the
# split kernel at other widths too; those read the same K/V bytes.
EXTRA_TRAFFIC = [
    ("split-KV decode partials 16x32x131072x128 bf16", "split_row_kernel<Bf16, 128, false>",
     ("splitkv_decode", "algorithmic_bytes_split")),
    ("GQA single-token decode partials, 1 q vs 32768 cached, B=16, 32q/8kv", "fwd_kernel<Bf16, 128, 64, 4, false, 2>",
     ("gqa_token_decode", "algorithmic_bytes_split")),
    ("causal GQA decode partials, 4 q vs 32768 cached, B=8, 32q/8kv", "fwd_kernel<Bf16, 128, 64, 4, true, 2>",
     ("cache_gqa_decode", "algorithmic_bytes_split")),
]
SQ_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
               "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"]
SIMDS = 1024   # 256 CUs x 4 SIMDs
XCDS = 8


def sq_summary(sq_dir, bench_log, command):
    """Markdown summary of one rocprofv3 --pmc pass over the SQ counters
    (SQ_COUNTERS) of a bench run: the headline kernels' timed dispatches and
    the MFMA busy share of every kernel of the run."""
    line = _bench_line(bench_log)
    ex = line["extras"]
    per = {c: _counter_per_kernel(sq_dir, c) for c in SQ_COUNTERS}

    def busy(mfma, grbm):   # GRBM_GUI_ACTIVE sums the XCDs' active cycles
        return mfma / (grbm / XCDS * SIMDS)
    md = ["# SQ counters: batched 4x16x4096x128 bf16 forward, and every kernel of the run", "",
          "Command (MI355X, one GPU):", "", "    " + command, "",
          "kernel_source_sha256: `%s`" % ex["kernel_source_sha256"], "",
          "Medians over the timed dispatches (the bench line records how many launches came before them). MFMA busy "
          "= SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / %d XCDs x %d SIMDs): the share of SIMD cycles the matrix "
          "cores were busy at the clock the chip ran, not a share of the 2.4 GHz peak." % (XCDS, SIMDS), "",
          "| counter | " + " | ".join(HEADLINE_KERNELS) + " |", "|---|" + "---|" * len(HEADLINE_KERNELS)]
    med = {}
    for tag, kname in HEADLINE_KERNELS.items():
        skip = ex["launches_before_timing"][tag]
        med[tag] = {}
        for c in SQ_COUNTERS:
            vals = [v for _, v in _dispatches(per[c], kname)[skip:skip + line["steps"]]]
            if len(vals) != line["steps"]:
                raise SystemExit("%s: %d timed dispatches of %s" % (c, len(vals), kname))
            med[tag][c] = statistics.median(vals)
    for c in SQ_COUNTERS:
        md.append("| %s | " % c + " | ".join("%.4g" % med[tag][c] for tag in HEADLINE_KERNELS) + " |")
    md.append("| MFMA busy | " + " | ".join("%.1f%%" % (100 * busy(med[t]["SQ_VALU_MFMA_BUSY_CYCLES"],
                                                                  med[t]["GRBM_GUI_ACTIVE"])) for t in HEADLINE_KERNELS) + " |")
    md += ["", "## MFMA busy of every kernel of the run (medians over all dispatches, warm-up included)", "",
           "| kernel | dispatches | MFMA busy | SQ_INSTS_MFMA | SQ_LDS_BANK_CONFLICT |", "|---|---|---|---|---|"]
    for kname in sorted(per["SQ_VALU_MFMA_BUSY_CYCLES"], key=lambda k_: -statistics.median(
            [v for _, v in per["GRBM_GUI_ACTIVE"].get(k_, [(0, 0)])])):
        m = statistics.median([v for _, v in per["SQ_VALU_MFMA_BUSY_CYCLES"][kname]])
        g = statistics.median([v for _, v in per["GRBM_GUI_ACTIVE"].get(kname, [(0, 0)])])
        if g <= 0:
            continue
        md.append("| `%s` | %d | %.1f%% | %.4g | %.4g |" % (
            _disp(kname), len(per["SQ_VALU_MFMA_BUSY_CYCLES"][kname]), 100 * busy(m, g),
            statistics.median([v for _, v in per["SQ_INSTS_MFMA"].get(kname, [(0, 0)])]),
            statistics.median([v for _, v in per["SQ_LDS_BANK_CONFLICT"].get(kname, [(0, 0)])])))
    return "\n".join(md) + "\n"


def pmc_summary(fetch_dir, write_dir, bench_logs, commands, out=PMC_SUMMARY):
    """HBM traffic of the headline kernels from FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for the
    bench's plain 256 MiB device copy; medians over the timed dispatches.
    Each counter comes from a bench run of its own, whose log (in the order
    FETCH_SIZE, WRITE_SIZE) says which dispatches were timed. Writes the
    committed summary (.md and .json; ``out`` names the .json)."""
    if len(bench_logs) != 2:
        raise SystemExit("--pmc-summary needs two --bench-log files: the FETCH_SIZE run's, then the WRITE_SIZE run's")
    lines = [_bench_line(b) for b in bench_logs]
    if lines[0]["extras"]["kernel_source_sha256"] != lines[1]["extras"]["kernel_source_sha256"]:
        raise SystemExit("the two counter runs were taken on different kernel sources")
    line = lines[0]
    ex = line["extras"]
    res, pers = {}, {}
    for name, d, counter, run in (("fetch", fetch_dir, "FETCH_SIZE", lines[0]), ("write", write_dir, "WRITE_SIZE",
                                                                                 lines[1])):
        per = pers[name] = _counter_per_kernel(d, counter)
        copies = sorted(x for k_, vs in per.items() if "copyBuffer" in k_ for x in vs)
        if not copies:
            raise SystemExit("no device copy kernel in the %s run" % counter)
        cal_kib = copies[0][1]    # the bench's 256 MiB calibration copy is the run's first device copy
        scale = (256 * 1024) / cal_kib
        res[name] = {"calibration_kib": cal_kib, "scale": scale}
        for tag, kname in HEADLINE_KERNELS.items():
            ds = _dispatches(per, kname)
            skip = run["extras"]["launches_before_timing"][tag]
            vals = [v for _, v in ds[skip:skip + run["steps"]]]
            if len(vals) != run["steps"]:
                raise SystemExit("%s run: %d timed dispatches of %s" % (counter, len(vals), kname))
            res[name][tag] = statistics.median(vals) * scale * 1024
    algo = line["config"]["algorithmic_bytes_per_launch"]
    js = {"kernel_source_sha256": ex["kernel_source_sha256"],
          "hbm_bytes_per_launch": res["fetch"]["noncausal"] + res["write"]["noncausal"],
          "per_launch": {tag: {"fetch_bytes": res["fetch"][tag], "write_bytes": res["write"][tag],
                               "algorithmic_bytes": algo, "ratio": (res["fetch"][tag] + res["write"][tag]) / algo}
                         for tag in HEADLINE_KERNELS},
          "counter_scale": {"FETCH_SIZE": res["fetch"]["scale"], "WRITE_SIZE": res["write"]["scale"]},
          "commands": commands}
    md = ["# HBM traffic: batched 4x16x4096x128 bf16 forward (FETCH_SIZE, WRITE_SIZE)", "", "Commands (MI355X; each "
          "counter in a run of its own):", ""] + ["    " + c for c in commands] + [
          "", "kernel_source_sha256: `%s`" % ex["kernel_source_sha256"], "",
          "Each counter is scaled by what it reads for the bench's plain 256 MiB device copy (FETCH_SIZE %.0f KiB -> "
          "x%.4f, WRITE_SIZE %.0f KiB -> x%.4f). FETCH_SIZE counts L2 misses sent to the fabric, an upper bound "
          "on HBM reads. Medians over the timed dispatches." % (
              res["fetch"]["calibration_kib"], res["fetch"]["scale"], res["write"]["calibration_kib"],
              res["write"]["scale"]), "",
          "| launch | fetch MB | write MB | algorithmic MB | (fetch + write) / algorithmic |", "|---|---|---|---|---|"]
    for tag in HEADLINE_KERNELS:
        p = js["per_launch"][tag]
        md.append("| %s | %.1f | %.1f | %.1f | %.2f |" % (tag, p["fetch_bytes"] / 1e6, p["write_bytes"] / 1e6,
                                                         algo / 1e6, p["ratio"]))
    # Every kernel of the runs (the extras too, when the runs had them):
    # medians over all dispatches, warm-up included.
    known = {}
    for what, kname, (leg, key) in EXTRA_TRAFFIC:
        if leg in lines[0]["extras"] and leg in lines[1]["extras"]:
            known[_kname(kname)] = (what, lines[0]["extras"][leg][key])
    md += ["", "## Every kernel of the runs (medians over all dispatches, warm-up included)", "",
           "| kernel | dispatches | fetch MB | write MB | algorithmic MB | ratio |", "|---|---|---|---|---|---|"]
    js["per_kernel"] = {}
    for kname in sorted(set(pers["fetch"]) & set(pers["write"]),
                        key=lambda k_: -statistics.median([v for _, v in pers["fetch"][k_]])):
        fb = statistics.median([v for _, v in pers["fetch"][kname]]) * res["fetch"]["scale"] * 1024
        wb = statistics.median([v for _, v in pers["write"][kname]]) * res["write"]["scale"] * 1024
        kn = _kname(kname)
        what, ab = next((v for k_, v in known.items() if k_ in kn), (None, None))
        js["per_kernel"][kn] = {"dispatches": len(pers["fetch"][kname]), "fetch_bytes": fb, "write_bytes": wb,
                                "algorithmic_bytes": ab, "workload": what}
        md.append("| `%s`%s | %d | %.1f | %.1f | %s | %s |" % (
            _disp(kname), (" (%s)" % what) if what else "", len(pers["fetch"][kname]), fb / 1e6,
            wb / 1e6, "%.1f" % (ab / 1e6) if ab else "", "%.2f" % ((fb + wb) / ab) if ab else ""))
    base = os.path.splitext(out)[0]
    with open(base + ".json", "w") as fh:
        json.dump(js, fh, indent=1)
    with open(base + ".md", "w") as fh:
        fh.write("\n".join(md) + "\n")
    return js


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-gate", action="store_true")
    ap.add_argument("--variants", action="store_true")
    ap.add_argument("--read-ceiling", action="store_true")
    ap.add_argument("--trace-summary", metavar="DIR")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--sq-summary", metavar="DIR")
    ap.add_argument("--bench-log", action="append", default=[])
    ap.add_argument("--command", action="append", default=[])
    args = ap.parse_args()
    if args.trace_summary:
        sys.stdout.write(trace_summary(args.trace_summary, args.bench_log[0], " ".join(args.command)))
        return
    if args.sq_summary:
        sys.stdout.write(sq_summary(args.sq_summary, args.bench_log[0], " ".join(args.command)))
        return
    if args.pmc_summary:
        print(json.dumps(pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.bench_log, args.command)))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this attention path runs whole on a single MI355X "
              "(sharding across GPUs is described in the design notes, not run). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.read_ceiling:
        print(json.dumps(read_ceiling()))
        return
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
    o_nc = torch.empty_like(q)
    o_c = torch.empty_like(q)
    l_nc = torch.empty((b, h, n), dtype=torch.float32, device=DEV)
    l_c = torch.empty_like(l_nc)
    launches = {"noncausal": 0, "causal": 0}

    def run(causal):
        launches["causal" if causal else "noncausal"] += 1
        if causal:
            sattn_fwd(q, k, v, causal=True, scale=scale, out=o_c, lse=l_c)
        else:
            sattn_fwd(q, k, v, causal=False, scale=scale, out=o_nc, lse=l_nc)
    gates = {}
    if not args.no_gate:
        for causal in (False, True):
            log("correctness gate causal=%s" % causal)
            run(causal)
            torch.cuda.synchronize()
            oo, ll = (o_c, l_c) if causal else (o_nc, l_nc)
            heads = [(i, j) for i in range(b) for j in range(h)]
            gates["causal" if causal else "noncausal"] = gate_dense(oo, ll, q, k, v, scale, causal, heads, 16, seed,
                                                                    torch.bfloat16)

    # Warm the GPU on the same step before the counted warmup steps: from
    # idle the chip takes tens of milliseconds of load to reach its steady
    # clock. Untimed; the timed region below is still exactly `steps` steps.
    preheat_steps = 0
    t_pre = time.perf_counter()
    while time.perf_counter() - t_pre < PREHEAT_S:
        for _ in range(8):
            run(False)
            run(True)
        preheat_steps += 8
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        run(False)
        run(True)
    torch.cuda.synchronize()
    before = dict(launches)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log("timing %d steps" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        run(False)
        e[1].record()
        e[2].record()
        run(True)
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
    traffic = load_traffic(src_hash)
    algo_bytes = 4 * b * h * n * d * 2 + b * h * n * 4
    roofline = {"bound": "mfma", "achieved": tf_nc, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": tf_nc / PEAK_BF16_TFLOPS, "traffic": traffic,
                "kernel": "fwd_kernel<Bf16, D=128, BN=64, 8 waves, noncausal, dense>",
                "algorithmic_flop_per_launch": f_nc, "algorithmic_bytes_per_launch": algo_bytes,
                "launch_ms_mean": float(np.mean(ms_nc)), "launch_ms_median": float(np.median(ms_nc)),
                "frac_from_median": f_nc / (np.median(ms_nc) / 1000.0) / 1e12 / PEAK_BF16_TFLOPS}
    extras = {"noncausal_TFLOPs": tf_nc, "causal_TFLOPs": tf_c,
              "noncausal_frac_of_bf16_peak": tf_nc / PEAK_BF16_TFLOPS,
              "causal_frac_of_bf16_peak": tf_c / PEAK_BF16_TFLOPS,
              "noncausal_launch_ms": stats(ms_nc), "causal_launch_ms": stats(ms_c),
              "launches_before_timing": before, "gate": gates, "kernel_source_sha256": src_hash}
    if not args.no_extras:
        log("headline kernels, the pages' method (graph and event)")
        t = time_variants({"noncausal": lambda: run(False), "causal": lambda: run(True)}, seed=0)
        extras["headline_pages_method"] = {
            tag: dict(t[tag], TFLOPs_graph=(f_c if tag == "causal" else f_nc) / t[tag]["graph_us"]["median"] / 1e6,
                      TFLOPs_event=(f_c if tag == "causal" else f_nc) / t[tag]["event_us"]["median"] / 1e6)
            for tag in t}
    del q, k, v, o_nc, o_c
    torch.cuda.empty_cache()
    if not args.no_extras:
        log("small-shape latency")
        extras["latency"] = small_latency(sattn_fwd)
        log("batched fp16: N(0,1) and Q x 16")
        extras["batched_fp16"] = batched_fp16_extra(sattn_fwd)
        log("split-KV decode")
        extras["splitkv_decode"] = decode_extra(cpu_leg=not args.no_cpu_baseline)
        log("varlen GQA")
        extras["varlen_gqa"] = varlen_extra()
        log("chunked prefill against a K/V cache")
        extras["cache_prefill"] = prefill_extra()
        log("causal GQA decode against a K/V cache")
        extras["cache_gqa_decode"] = gqa_decode_extra()
        log("GQA single-token decode")
        extras["gqa_token_decode"] = gqa_token_decode_extra()
        log("strided (transposed) inputs")
        extras["strided_transposed"] = strided_extra()
        log("sparse: window + globals, block mask")
        extras["sparse"] = sparse_extra()
        log("backward")
        extras["backward"] = backward_extra()
        log("backward: packed varlen GQA")
        extras["varlen_backward"] = varlen_backward_extra()
        log("backward: sliding window + global tokens")
        extras["sparse_backward"] = sparse_backward_extra()
    if args.variants:
        log("design variants")
        extras["variants"] = variants_leg()
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(args.cpu_budget_s)
        log("cpu oracle per workload")
        cpu["per_workload"] = cpu_oracle_per_workload()
        if "splitkv_decode" in extras:
            cpu["per_workload"]["splitkv_decode_16x32x131072x128_bf16"] = \
                extras["splitkv_decode"].pop("cpu_oracle_all_rows")
    line = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "batched_4x16x4096x128_bf16: one noncausal + one causal forward per step",
                       "B": b, "H": h, "N": n, "D": d, "flop_per_step": f_nc + f_c,
                       "flop_per_launch": {"noncausal": f_nc, "causal": f_c},
                       "algorithmic_bytes_per_launch": algo_bytes,
                       "flop_convention": "4*N^2*D per head noncausal, 2*N^2*D causal",
                       "parallelism": "single GPU"},
            "frac_of_bf16_peak": value / PEAK_BF16_TFLOPS,
            "preheat": {"seconds": PREHEAT_S, "steps": preheat_steps,
                        "note": "untimed load on the same step before the warmup steps (clock settling)"},
            "roofline": roofline, "cpu_baseline": cpu, "extras": extras}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it only draws inputs, lengths and
sampled row indices from fixed seeds, and converts stored half-precision
tensors to exact float64 copies. Both the oracle side and the HIP side of a
test receive what it produces.

Recipe (the pages fix only "iid N(0,1) from seed"):
  * one ``torch.Generator`` per tensor set, seeded with the workload's seed;
    q, k and v are drawn in that order with ``randn`` in float32 and rounded
    to the workload's dtype (round to nearest even); the rounded values are
    the inputs;
  * very large K/V (the split-KV decode workload, 2 x 16 GiB) are drawn on
    the device in slices with a seeded CUDA generator;
  * packed variable-length lengths: numpy ``default_rng(seed).integers(1,
    8193, 8)``, concatenated in draw order (token-major packing);
  * sampled rows: numpy ``default_rng(seed)`` choice without replacement,
    always including the first and last row.
"""
import numpy as np
import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}

# The five workloads of the pages' hot path, by what they are.
WORKLOADS = {
    "single_head_129x32_fp16_causal": dict(
        kind="dense", B=1, H=1, N=129, D=32, dtype="fp16", causal=(True,), seed=1),
    "single_head_512x64_fp16": dict(
        kind="dense", B=1, H=1, N=512, D=64, dtype="fp16", causal=(True, False), seed=2,
        q_multipliers=(1.0, 16.0)),
    "batched_4x16x4096x128_bf16": dict(
        kind="dense", B=4, H=16, N=4096, D=128, dtype="bf16", causal=(True, False), seed=3,
        sampled_rows_per_head=256),
    "splitkv_decode_16x32x131072x128_bf16": dict(
        kind="split", B=16, Hq=32, Hkv=32, Nq=1, Nk=131072, D=128, dtype="bf16",
        chunk=4096, seed=4),
    "varlen_gqa_8seq_32q8kv_128_bf16_causal": dict(
        kind="varlen", S=8, max_len=8192, Hq=32, Hkv=8, D=128, dtype="bf16", seed=5),
}


def randn(shape, dtype, gen, device="cpu"):
    """iid N(0,1) drawn in float32 from ``gen``, rounded to ``dtype``."""
    return torch.randn(shape, generator=gen, dtype=torch.float32, device=device).to(DTYPES[dtype])


def qkv(q_shape, kv_shape, dtype, seed, device="cpu"):
    """q, k, v drawn in that order from one generator seeded with ``seed``."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q = randn(q_shape, dtype, g, device)
    k = randn(kv_shape, dtype, g, device)
    v = randn(kv_shape, dtype, g, device)
    return q, k, v


def randn_device_sliced(shape, dtype, gen, device, slice_elems=1 << 28):
    """Fill a large device tensor slice by slice (bounded float32 transients)."""
    out = torch.empty(shape, dtype=DTYPES[dtype], device=device)
    flat = out.view(-1)
    n = flat.numel()
    for a in range(0, n, slice_elems):
        b = min(n, a + slice_elems)
        flat[a:b] = torch.randn((b - a,), generator=gen, dtype=torch.float32,
                                device=device).to(DTYPES[dtype])
    return out


def varlen_lengths(seed, count=8, max_len=8192):
    """Sequence lengths drawn uniformly from [1, max_len]."""
    return np.random.default_rng(seed).integers(1, max_len + 1, count).astype(np.int64)


def cu_seqlens_of(lengths):
    """Prefix offsets [0, L0, L0+L1, ...] of packed sequences (int32)."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu.astype(np.int32)


def sample_rows(seed, n, count, groups=1):
    """``groups`` independent draws of ``count`` distinct row indices in
    [0, n), each containing 0 and n-1. Returns int64 [groups, count]."""
    rng = np.random.default_rng(seed)
    count = min(count, n)
    out = np.zeros((groups, count), dtype=np.int64)
    for g in range(groups):
        if n <= count:
            out[g] = np.arange(n)
            continue
        inner = rng.choice(np.arange(1, n - 1), size=count - 2, replace=False)
        out[g] = np.sort(np.concatenate([[0, n - 1], inner]))
    return out


def to_f64(t):
    """Exact float64 copy of a stored fp16/bf16/fp32 tensor (numpy)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def scale_f32(d):
    """1/sqrt(D) rounded to float32: the value the GPU receives."""
    return float(np.float32(1.0 / np.sqrt(np.float64(d))))

"""sattn_bwd_noalloc, the backward entry point that allocates nothing (its
Delta workspace lives in the library's static device array), called through
the C ABI: its gradients must equal sattn_bwd's (same kernels, so bit for
bit), on two calls in a row, the second with a smaller input, each written
over NaN-filled outputs. The smaller call also runs on a side stream and is
checked against the float64 gradients of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from exact_tiled_attention_sattn_amd import library, sattn_fwd, sattn_bwd
from oracle import backward
from tests.parity import grad_bounds, check_grad

DEV = "cuda:0"
pytestmark = pytest.mark.gpu


def _noalloc(q, k, v, o, do, lse, causal, scale, stream):
    lib = library()
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    b, hq, n, d = q.shape
    st = lib.sattn_bwd_noalloc(1 if q.dtype == torch.bfloat16 else 0,
                               *(ctypes.c_void_p(x.data_ptr()) for x in (q, k, v, o, do, lse, dq, dk, dv)),
                               b, hq, k.shape[1], n, d, int(causal), scale, ctypes.c_void_p(stream.cuda_stream))
    assert st == 0, library().sattn_last_error()
    return dq, dk, dv


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_bwd_on_two_calls(order):
    calls = [(2, 8, 2, 1100, 128, "bf16", True, 51), (1, 3, 3, 300, 64, "fp16", False, 52)]
    for i, (b, hq, hkv, n, d, dt, causal, seed) in enumerate(calls):
        print("[noalloc] call", i, (b, hq, hkv, n, d, dt, causal), flush=True)
        q, k, v = W.qkv((b, hq, n, d), (b, hkv, n, d), dt, seed)
        do = W.randn((b, hq, n, d), dt, torch.Generator().manual_seed(seed + 100))
        q, k, v, do = (x.to(DEV) for x in (q, k, v, do))
        scale = W.scale_f32(d)
        o, lse = sattn_fwd(q, k, v, causal=causal, scale=scale) if hq == hkv else \
            _fwd_gqa(q, k, v, causal, scale)
        ref = sattn_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream() if i == 0 else torch.cuda.Stream()
        if i > 0:
            stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            got = _noalloc(q, k, v, o, do, lse, causal, scale, stream)
        stream.synchronize()
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(g, r), "%s differs from sattn_bwd" % name
        if i == 1:
            qf, kf, vf, dof, of = (W.to_f64(x.cpu()) for x in (q, k, v, do, o))
            for h in range(hq):
                refs = backward.attention_backward(qf[0, h], kf[0, h], vf[0, h], dof[0, h], scale, causal)
                rel, und = grad_bounds(qf[0, h], kf[0, h], vf[0, h], dof[0, h], of[0, h], scale, causal)
                for j, name in enumerate(("dq", "dk", "dv")):
                    check_grad(got[j][0, h], refs[j], rel[j], und[j], W.DTYPES[dt], "noalloc %s head %d" % (name, h))
            assert np.isfinite(got[0].float().cpu().numpy()).all()


def _fwd_gqa(q, k, v, causal, scale):
    """The forward for grouped heads (sattn_fwd_cache with Nq = Nk)."""
    from exact_tiled_attention_sattn_amd import sattn_fwd_cache
    return sattn_fwd_cache(q, k, v, causal=causal, scale=scale)

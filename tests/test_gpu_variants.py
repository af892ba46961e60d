"""GPU parity of the design-variant libraries (libsattn_<name>.so): each
rebuilds the dense forward with one design choice changed (tile width,
single buffer, no causal tile skip, no query-tile pairing) so that the
choice can be timed against the product. Their outputs must meet the same
bar against the oracle as the product's. Variants that are not built are
skipped."""
import ctypes
import os

import numpy as np
import pytest
import torch

import workloads as W
from exact_tiled_attention_sattn_amd import build as B
from oracle import dense
from tests.parity import check_attention

DEV = "cuda:0"
pytestmark = pytest.mark.gpu


def _lib(name):
    path = B.variant_path(name)
    if not os.path.exists(path):
        pytest.skip("variant %s not built" % name)
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.sattn_fwd.restype = ctypes.c_int
    lib.sattn_fwd.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float, vp]
    return lib


def _run(lib, q, k, v, causal, scale):
    b, h, n, d = q.shape
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=DEV)
    rc = lib.sattn_fwd(1 if q.dtype == torch.bfloat16 else 0, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                       o.data_ptr(), lse.data_ptr(), b, h, n, d, int(causal), scale,
                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, rc
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("name", sorted(B.VARIANTS))
@pytest.mark.parametrize("causal", [False, True])
def test_variant_full_rows(name, causal):
    """Every row of a ragged three-head problem (several tiles of every
    width, a partial last tile)."""
    print("[variant]", name, causal, flush=True)
    lib = _lib(name)
    q, k, v = W.qkv((1, 3, 777, 128), (1, 3, 777, 128), "bf16", 41)
    scale = W.scale_f32(128)
    o, lse = _run(lib, q, k, v, causal, scale)
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal)
    check_attention(o, lse, o_ref, lse_ref, torch.bfloat16, name)


@pytest.mark.parametrize("name", sorted(B.VARIANTS))
def test_variant_paired_grid_sampled(name):
    """A causal grid large enough for query-tile pairing (odd tile count,
    ragged last tile), sampled rows of every head."""
    print("[variant] paired", name, flush=True)
    lib = _lib(name)
    b, h, n, d = 1, 205, 1270, 128
    q, k, v = W.qkv((b, h, n, d), (b, h, n, d), "fp16", 43)
    scale = W.scale_f32(d)
    o, lse = _run(lib, q, k, v, True, scale)
    rows = W.sample_rows(43, n, 8, groups=b * h).reshape(b, h, -1)
    o_ref, lse_ref = dense.attention_bhnd(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, True, rows=rows)
    idx = torch.from_numpy(rows)
    o_s = torch.stack([torch.stack([o[0, j][idx[0, j]] for j in range(h)])])
    l_s = torch.stack([torch.stack([lse[0, j][idx[0, j]] for j in range(h)])])
    check_attention(o_s, l_s, o_ref, lse_ref, torch.float16, name)
    assert np.isfinite(o.float().numpy()).all()

"""Tolerance checks shared by the GPU parity tests.

Bar (elementwise, allclose semantics): |o - ref| <= atol + rtol * |ref| with
(atol, rtol) = (2e-3, 2e-3) for fp16 and (1e-2, 1e-2) for bf16 outputs, and
|lse - ref| <= 1e-3 for the float32 logsumexp. Partial states of the split
path are fp32 and are compared with the fp32-accumulation bound below.
"""
import numpy as np
import torch

TOL = {torch.float16: (2e-3, 2e-3), torch.bfloat16: (1e-2, 1e-2)}
LSE_ATOL = 1e-3


def _np(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def check_o(o_gpu, o_ref, dtype, what="o"):
    atol, rtol = TOL[dtype]
    a, r = _np(o_gpu), _np(o_ref)
    assert a.shape == r.shape, (what, a.shape, r.shape)
    assert np.isfinite(a).all(), "%s: non-finite values in GPU output" % what
    err = np.abs(a - r)
    bound = atol + rtol * np.abs(r)
    ratio = float((err / bound).max()) if err.size else 0.0
    assert ratio <= 1.0, "%s: max|err|=%.3g, worst err/bound=%.3f at %s" % (
        what, float(err.max()), ratio, np.unravel_index(int(np.argmax(err / bound)), err.shape))
    return float(err.max()) if err.size else 0.0, ratio


def check_lse(lse_gpu, lse_ref, what="lse"):
    a, r = _np(lse_gpu), _np(lse_ref)
    assert a.shape == r.shape, (what, a.shape, r.shape)
    inf_ref = np.isinf(r)
    assert np.array_equal(np.isinf(a), inf_ref) and np.array_equal(a[inf_ref], r[inf_ref]), \
        "%s: -inf pattern differs" % what
    err = np.abs(a[~inf_ref] - r[~inf_ref])
    m = float(err.max()) if err.size else 0.0
    assert m <= LSE_ATOL, "%s: max|err|=%.3g > %.1g" % (what, m, LSE_ATOL)
    return m


def check_attention(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    eo, ratio = check_o(o_gpu, o_ref, dtype, what + " o")
    el = check_lse(lse_gpu, lse_ref, what + " lse")
    return {"o_max_err": eo, "o_err_over_bound": ratio, "lse_max_err": el}

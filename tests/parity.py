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


# Tolerance for gradients, derived from the arithmetic (the pages give none).
# dQ_i = scale * sum_j dS_ij k_j, dK_j = scale * sum_i dS_ij q_i and
# dV_j = sum_i P_ij dO_i are fp32 sums whose other factor (dS or P) enters the
# MFMA rounded to the input dtype (unit roundoff u = 2^-8 bf16, 2^-11 fp16);
# Delta_i = dO_i . O_i uses the output O, itself rounded (|dDelta_i| <=
# u sum_d |dO_id O_id|), which shifts dS_ij by P_ij dDelta_i; the result is
# rounded once more. Because sum_j dS_ij = 0 the sums cancel heavily, so the
# bound is taken on the sums of magnitudes, element by element:
#   |dq - ref| <= K u (scale (|dS| |K| + dDelta . (P |K|)) + |ref|)   (dk alike)
#   |dv - ref| <= K u (P^T |dO| + |ref|)
# with K = 4 for the fp32 accumulation and the rounding of P itself.
GRAD_U = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}
# absolute rounding error of a value below the dtype's normal range (half the
# subnormal spacing): fp16 P and dS values under 2^-14 round to multiples of
# 2^-24; bf16 shares fp32's exponent range, where this never matters here
GRAD_ETA = {torch.bfloat16: 2.0 ** -134, torch.float16: 2.0 ** -25}
GRAD_K = 4.0


def grad_bounds(q, k, v, do, o, scale, causal, allowed=None):
    """Per-element bounds for one head, float64 numpy inputs: the relative
    part (dq, dk, dv), in units of u, and the underflow part (dq, dk, dv), in
    units of the absolute error of one rounded P or dS element. ``allowed``
    (optional) is the eligibility mask; rows without a key get P = 0."""
    n = q.shape[0]
    s = scale * (q @ k.T)
    elig = np.ones((n, k.shape[0]))
    if causal:
        elig = (np.arange(n)[None, :] <= np.arange(n)[:, None]).astype(np.float64)
    if allowed is not None:
        elig = elig * allowed
    s = np.where(elig > 0, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    pm = np.exp(s - np.where(np.isfinite(mx), mx, 0.0))
    tot = pm.sum(axis=1, keepdims=True)
    pm = np.where(tot > 0, pm / np.where(tot > 0, tot, 1.0), 0.0)
    dp = do @ v.T
    ds = pm * (dp - (pm * dp).sum(axis=1, keepdims=True))
    ddel = (np.abs(do) * np.abs(o)).sum(axis=1, keepdims=True)       # per unit roundoff
    bq = scale * (np.abs(ds) @ np.abs(k) + ddel * (pm @ np.abs(k)))
    bk = scale * (np.abs(ds).T @ np.abs(q) + (pm * ddel).T @ np.abs(q))
    bv = pm.T @ np.abs(do)
    aq = scale * (elig @ np.abs(k))          # dS_ij rounded, times |K_j|
    ak = scale * (elig.T @ np.abs(q))
    av = elig.T @ np.abs(do)                  # P_ij rounded, times |dO_i|
    return (bq, bk, bv), (aq, ak, av)


def check_grad(g, ref, bound, abound, dtype, what, verbose=True):
    a = _np(g)
    assert np.isfinite(a).all(), what + ": non-finite gradient"
    u = GRAD_U[dtype]
    err = np.abs(a - ref)
    # relative rounding, plus the absolute floor below the normal range: of
    # the rounded P / dS operands (abound) and of the stored gradient (1)
    lim = GRAD_K * (u * (bound + np.abs(ref)) + GRAD_ETA[dtype] * (abound + 1.0)) + 1e-30
    ratio = float((err / lim).max()) if err.size else 0.0
    if verbose:
        print("[grad] %s max|err| %.3g max bound %.3g worst err/bound %.3f" % (what, float(err.max()),
                                                                               float(lim.max()), ratio), flush=True)
    assert ratio <= 1.0, "%s: worst err/bound %.3f" % (what, ratio)
    return ratio

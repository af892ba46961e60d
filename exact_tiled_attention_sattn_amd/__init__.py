"""Exact streaming attention forward for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libsattn.so`` (declared in
``include/sattn.h``). The functions carry the C names and only marshal
arguments: they check tensor dtype/device/shape/contiguity, allocate outputs
with torch when the caller does not pass them, and hand raw device pointers
and the current HIP stream to the library. Every step of the computation runs
in the HIP kernels; there is no fallback. If the library is missing, every
call raises.
"""
import ctypes
import math
import os

import torch

__all__ = [
    "sattn_fwd", "sattn_fwd_split", "sattn_merge", "sattn_fwd_varlen", "sattn_fwd_cache",
    "sattn_fwd_split_cache", "sattn_fwd_strided", "sattn_fwd_sparse", "sattn_bwd", "sattn_bwd_noalloc",
    "sattn_bwd_cache", "sattn_bwd_varlen", "sattn_bwd_sparse",
    "SattnError", "library", "LIB_PATH", "STATUS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsattn.so")

STATUS = {
    0: "SATTN_OK", 1: "SATTN_ERR_NULL", 2: "SATTN_ERR_SHAPE", 3: "SATTN_ERR_DTYPE",
    4: "SATTN_ERR_UNSUPPORTED", 5: "SATTN_ERR_ALIGN", 6: "SATTN_ERR_ALIAS",
    7: "SATTN_ERR_HIP", 8: "SATTN_ERR_VALUE",
}
_DTYPE_CODE = {torch.float16: 0, torch.bfloat16: 1}

_lib = None


class SattnError(RuntimeError):
    """A libsattn call returned a non-OK status."""

    def __init__(self, status, detail):
        self.status = status
        super().__init__("%s: %s" % (STATUS.get(status, "status %d" % status), detail))


def library():
    """Load libsattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libsattn.so is not built (%s); run "
                           "`python -m exact_tiled_attention_sattn_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, fp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
    lib.sattn_status_string.restype = ctypes.c_char_p
    lib.sattn_status_string.argtypes = [i32]
    lib.sattn_last_error.restype = ctypes.c_char_p
    lib.sattn_last_error.argtypes = []
    lib.sattn_fwd.restype = i32
    lib.sattn_fwd.argtypes = [i32, vp, vp, vp, vp, fp, i64, i64, i64, i64, i32, ctypes.c_float, vp]
    lib.sattn_fwd_split.restype = i32
    lib.sattn_fwd_split.argtypes = [i32, vp, vp, vp, fp, fp, fp, i64, i64, i64, i64, i64, i64, i64,
                                    ctypes.c_float, vp]
    lib.sattn_merge.restype = i32
    lib.sattn_merge.argtypes = [i32, fp, fp, fp, i64, i64, i64, vp, fp, vp]
    lib.sattn_fwd_varlen.restype = i32
    lib.sattn_fwd_varlen.argtypes = [i32, vp, vp, vp, vp, fp, vp, i64, i64, i64, i64, i64, i64, i32,
                                     ctypes.c_float, vp]
    lib.sattn_fwd_cache.restype = i32
    lib.sattn_fwd_cache.argtypes = [i32, vp, vp, vp, vp, fp, i64, i64, i64, i64, i64, i64, i32,
                                    ctypes.c_float, vp]
    lib.sattn_fwd_strided.restype = i32
    lib.sattn_fwd_strided.argtypes = [i32, vp, vp, vp, vp, fp, i64, i64, i64, i64, i64, i64,
                                      ctypes.POINTER(i64), ctypes.POINTER(i64), i32, ctypes.c_float, vp]
    lib.sattn_bwd.restype = i32
    lib.sattn_bwd.argtypes = [i32, vp, vp, vp, vp, vp, fp, fp, vp, vp, vp, i64, i64, i64, i64, i64, i32,
                              ctypes.c_float, vp]
    lib.sattn_bwd_noalloc.restype = i32
    lib.sattn_bwd_noalloc.argtypes = [i32, vp, vp, vp, vp, vp, fp, vp, vp, vp, i64, i64, i64, i64, i64, i32,
                                      ctypes.c_float, vp]
    lib.sattn_bwd_varlen.restype = i32
    lib.sattn_bwd_varlen.argtypes = [i32, vp, vp, vp, vp, vp, fp, fp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                     i64, i32, ctypes.c_float, vp]
    lib.sattn_bwd_cache.restype = i32
    lib.sattn_bwd_cache.argtypes = [i32, vp, vp, vp, vp, vp, fp, fp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32,
                                    ctypes.c_float, vp]
    lib.sattn_bwd_sparse.restype = i32
    lib.sattn_bwd_sparse.argtypes = [i32, vp, vp, vp, vp, vp, fp, fp, vp, vp, vp, i64, i64, i64, i64, i64, i32,
                                     i64, i64, i64, vp, i64, i64, i64, ctypes.c_float, vp]
    lib.sattn_fwd_sparse.restype = i32
    lib.sattn_fwd_sparse.argtypes = [i32, vp, vp, vp, vp, fp, i64, i64, i64, i64, i64, i64, i32, i64, i64, i64,
                                     vp, i64, i64, i64, ctypes.c_float, vp]
    lib.sattn_fwd_split_cache.restype = i32
    lib.sattn_fwd_split_cache.argtypes = [i32, vp, vp, vp, fp, fp, fp, i64, i64, i64, i64, i64, i64, i64,
                                          i32, ctypes.c_float, vp]
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise SattnError(status, library().sattn_last_error().decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev_tensor(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _same_device(*ts):
    dev = ts[0].device
    for t in ts[1:]:
        if t is not None and t.device != dev:
            raise ValueError("all tensors must be on %s" % dev)
    return dev


def _scale(scale, d):
    return float(1.0 / math.sqrt(d)) if scale is None else float(scale)


def sattn_fwd(q, k, v, causal=False, scale=None, out=None, lse=None):
    """Attention forward on [B, H, N, D] tensors (fp16 or bf16).

    Returns (o [B,H,N,D] in q's dtype, lse [B,H,N] float32)."""
    lib = library()
    _dev_tensor(q, "q", ndim=4)
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("q must be float16 or bfloat16")
    _dev_tensor(k, "k", q.dtype, 4)
    _dev_tensor(v, "v", q.dtype, 4)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share shape [B, H, N, D]")
    dev = _same_device(q, k, v, out, lse)
    b, h, n, d = q.shape
    out = torch.empty_like(q) if out is None else _dev_tensor(out, "out", q.dtype, 4)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=dev) if lse is None else \
        _dev_tensor(lse, "lse", torch.float32, 3)
    if out.shape != q.shape or lse.shape != (b, h, n):
        raise ValueError("out/lse shape mismatch")
    with torch.cuda.device(dev):
        _check(lib.sattn_fwd(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                             b, h, n, d, int(bool(causal)), _scale(scale, d), _stream(dev)))
    return out, lse


def split_num_chunks(nk, chunk):
    return -(-nk // chunk)


def _cache_shapes(q, k, v):
    _dev_tensor(q, "q", ndim=4)
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("q must be float16 or bfloat16")
    _dev_tensor(k, "k", q.dtype, 4)
    _dev_tensor(v, "v", q.dtype, 4)
    b, hq, nq, d = q.shape
    if k.shape != v.shape or k.shape[0] != b or k.shape[3] != d:
        raise ValueError("k/v must be [B, Hkv, Nk, D] matching q")
    return b, hq, nq, d, k.shape[1], k.shape[2]


def sattn_fwd_cache(q, k, v, causal=False, scale=None, out=None, lse=None):
    """Queries [B,Hq,Nq,D] against a K/V cache [B,Hkv,Nk,D]; query i sits at
    position i + Nk - Nq (causal: keys j <= i + Nk - Nq).

    Returns (o [B,Hq,Nq,D] in q's dtype, lse [B,Hq,Nq] float32)."""
    lib = library()
    b, hq, nq, d, hkv, nk = _cache_shapes(q, k, v)
    dev = _same_device(q, k, v, out, lse)
    out = torch.empty_like(q) if out is None else _dev_tensor(out, "out", q.dtype, 4)
    lse = torch.empty((b, hq, nq), dtype=torch.float32, device=dev) if lse is None else \
        _dev_tensor(lse, "lse", torch.float32, 3)
    if out.shape != q.shape or lse.shape != (b, hq, nq):
        raise ValueError("out/lse shape mismatch")
    with torch.cuda.device(dev):
        _check(lib.sattn_fwd_cache(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                   b, hq, hkv, nq, nk, d, int(bool(causal)), _scale(scale, d), _stream(dev)))
    return out, lse


def sattn_fwd_strided(q, k, v, causal=False, scale=None, out=None, lse=None):
    """``sattn_fwd_cache`` on strided views: q [B,Hq,Nq,D] and k, v [B,Hkv,Nk,D]
    may be transposed, sliced or expanded (stride 0) views whose last dim is
    contiguous; k and v must have equal strides. They are read in place.

    Returns dense (o [B,Hq,Nq,D], lse [B,Hq,Nq] float32)."""
    lib = library()
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dim() != 4:
            raise ValueError("%s must be a 4-dim GPU tensor" % name)
        if t.shape[3] > 1 and t.stride(3) != 1:
            raise ValueError("%s must have a contiguous last dim" % name)
    if q.dtype not in _DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float16 or bfloat16")
    b, hq, nq, d = q.shape
    if k.shape != v.shape or k.shape[0] != b or k.shape[3] != d:
        raise ValueError("k/v must be [B, Hkv, Nk, D] matching q")
    if k.stride()[:3] != v.stride()[:3]:
        raise ValueError("k and v must have equal strides")
    hkv, nk = k.shape[1], k.shape[2]
    dev = _same_device(q, k, v, out, lse)
    out = torch.empty(q.shape, dtype=q.dtype, device=dev) if out is None else _dev_tensor(out, "out", q.dtype, 4)
    lse = torch.empty((b, hq, nq), dtype=torch.float32, device=dev) if lse is None else \
        _dev_tensor(lse, "lse", torch.float32, 3)
    if out.shape != q.shape or lse.shape != (b, hq, nq):
        raise ValueError("out/lse shape mismatch")
    qs = (ctypes.c_int64 * 3)(*q.stride()[:3])
    ks = (ctypes.c_int64 * 3)(*k.stride()[:3])
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t.numel() > 0 else ctypes.c_void_p(0)  # noqa: E731
    with torch.cuda.device(dev):
        _check(lib.sattn_fwd_strided(_DTYPE_CODE[q.dtype], ptr(q), ptr(k), ptr(v), _ptr(out), _ptr(lse),
                                     b, hq, hkv, nq, nk, d, qs, ks, int(bool(causal)), _scale(scale, d),
                                     _stream(dev)))
    return out, lse


def sattn_bwd(q, k, v, o, dout, lse, causal=False, scale=None, dq=None, dk=None, dv=None, delta=None):
    """Gradients of sum(dout * o) for o, lse = sattn_fwd(q, k, v) (or
    sattn_fwd_cache with Nq = Nk). q, o, dout [B,Hq,N,D]; k, v [B,Hkv,N,D];
    lse [B,Hq,N] float32. ``delta`` is a float32 [B,Hq,N] workspace.

    Returns (dq, dk, dv) in q's dtype."""
    lib = library()
    _dev_tensor(q, "q", ndim=4)
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("q must be float16 or bfloat16")
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _dev_tensor(t, name, q.dtype, 4)
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    if k.shape != (b, hkv, n, d) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q/o/dout must be [B,Hq,N,D] and k/v [B,Hkv,N,D]")
    _dev_tensor(lse, "lse", torch.float32, 3)
    if lse.shape != (b, hq, n):
        raise ValueError("lse must be [B, Hq, N]")
    dev = _same_device(q, k, v, o, dout, lse, dq, dk, dv, delta)
    dq = torch.empty_like(q) if dq is None else _dev_tensor(dq, "dq", q.dtype, 4)
    dk = torch.empty_like(k) if dk is None else _dev_tensor(dk, "dk", q.dtype, 4)
    dv = torch.empty_like(v) if dv is None else _dev_tensor(dv, "dv", q.dtype, 4)
    delta = torch.empty((b, hq, n), dtype=torch.float32, device=dev) if delta is None else \
        _dev_tensor(delta, "delta", torch.float32, 3)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape or delta.shape != (b, hq, n):
        raise ValueError("gradient/workspace shape mismatch")
    with torch.cuda.device(dev):
        _check(lib.sattn_bwd(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                             _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), b, hq, hkv, n, d, int(bool(causal)),
                             _scale(scale, d), _stream(dev)))
    return dq, dk, dv


def sattn_bwd_noalloc(q, k, v, o, dout, lse, causal=False, scale=None, dq=None, dk=None, dv=None):
    """sattn_bwd with its Delta workspace in the library's fixed device array
    (B*Hq*N <= 2^21 rows): the C call allocates nothing. Pass dq, dk, dv to
    keep this binding from allocating them. Calls that overlap on one GPU
    race on the shared array.

    Returns (dq, dk, dv) in q's dtype."""
    lib = library()
    _dev_tensor(q, "q", ndim=4)
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("q must be float16 or bfloat16")
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _dev_tensor(t, name, q.dtype, 4)
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    if k.shape != (b, hkv, n, d) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q/o/dout must be [B,Hq,N,D] and k/v [B,Hkv,N,D]")
    _dev_tensor(lse, "lse", torch.float32, 3)
    if lse.shape != (b, hq, n):
        raise ValueError("lse must be [B, Hq, N]")
    dev = _same_device(q, k, v, o, dout, lse, dq, dk, dv)
    dq = torch.empty_like(q) if dq is None else _dev_tensor(dq, "dq", q.dtype, 4)
    dk = torch.empty_like(k) if dk is None else _dev_tensor(dk, "dk", q.dtype, 4)
    dv = torch.empty_like(v) if dv is None else _dev_tensor(dv, "dv", q.dtype, 4)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("gradient shape mismatch")
    with torch.cuda.device(dev):
        _check(lib.sattn_bwd_noalloc(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                     _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), b, hq, hkv, n, d, int(bool(causal)),
                                     _scale(scale, d), _stream(dev)))
    return dq, dk, dv


def sattn_fwd_sparse(q, k, v, causal=False, window=(-1, -1), n_global=0, block_mask=None, block_q=64, block_k=64,
                     scale=None, out=None, lse=None):
    """Sparse attention: ``sattn_fwd_cache`` restricted to the window
    (left, right) (-1 = unlimited), ``n_global`` global tokens and an optional
    uint8 block mask [Hq or 1, ceil(Nq/block_q), ceil(Nk/block_k)] on the GPU.

    Returns (o [B,Hq,Nq,D], lse [B,Hq,Nq] float32)."""
    lib = library()
    b, hq, nq, d, hkv, nk = _cache_shapes(q, k, v)
    dev = _same_device(q, k, v, out, lse, block_mask)
    heads = 0
    if block_mask is not None:
        _dev_tensor(block_mask, "block_mask", torch.uint8)
        if block_mask.dim() == 2:
            heads = 1
            block_mask = block_mask.unsqueeze(0)
        if block_mask.dim() != 3:
            raise ValueError("block_mask must be [nqb, nkb] or [heads, nqb, nkb]")
        heads = block_mask.shape[0]
        nqb, nkb = -(-nq // int(block_q)), -(-nk // int(block_k))
        if tuple(block_mask.shape[1:]) != (nqb, nkb):
            raise ValueError("block_mask must be [heads, %d, %d]" % (nqb, nkb))
    out = torch.empty_like(q) if out is None else _dev_tensor(out, "out", q.dtype, 4)
    lse = torch.empty((b, hq, nq), dtype=torch.float32, device=dev) if lse is None else \
        _dev_tensor(lse, "lse", torch.float32, 3)
    if out.shape != q.shape or lse.shape != (b, hq, nq):
        raise ValueError("out/lse shape mismatch")
    left, right = (int(x) for x in window)
    with torch.cuda.device(dev):
        _check(lib.sattn_fwd_sparse(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                    b, hq, hkv, nq, nk, d, int(bool(causal)), left, right, int(n_global),
                                    _ptr(block_mask), heads, int(block_q), int(block_k), _scale(scale, d),
                                    _stream(dev)))
    return out, lse


def sattn_fwd_split_cache(q, k, v, chunk, causal=False, scale=None, part_m=None, part_l=None, part_acc=None):
    """Split-KV partial states against a K/V cache, optionally causal (query i
    at position i + Nk - Nq). Same outputs as ``sattn_fwd_split``."""
    return _split(q, k, v, chunk, causal, scale, part_m, part_l, part_acc)


def sattn_fwd_split(q, k, v, chunk, scale=None, part_m=None, part_l=None, part_acc=None):
    """Split-KV partial states (non-causal). q [B,Hq,Nq,D], k/v [B,Hkv,Nk,D].

    Returns (part_m [B,Hq,Nq,C], part_l [B,Hq,Nq,C], part_acc [B,Hq,Nq,C,D]),
    all float32, acc not normalized."""
    return _split(q, k, v, chunk, None, scale, part_m, part_l, part_acc)


def _split(q, k, v, chunk, causal, scale, part_m, part_l, part_acc):
    lib = library()
    b, hq, nq, d, hkv, nk = _cache_shapes(q, k, v)
    dev = _same_device(q, k, v, part_m, part_l, part_acc)
    chunk = int(chunk)
    if chunk <= 0:
        raise ValueError("chunk must be > 0")
    c = split_num_chunks(nk, chunk)
    shp = (b, hq, nq, c)
    f32 = torch.float32
    part_m = torch.empty(shp, dtype=f32, device=dev) if part_m is None else _dev_tensor(part_m, "part_m", f32, 4)
    part_l = torch.empty(shp, dtype=f32, device=dev) if part_l is None else _dev_tensor(part_l, "part_l", f32, 4)
    part_acc = torch.empty(shp + (d,), dtype=f32, device=dev) if part_acc is None else \
        _dev_tensor(part_acc, "part_acc", f32, 5)
    if part_m.shape != shp or part_l.shape != shp or part_acc.shape != shp + (d,):
        raise ValueError("partial buffer shape mismatch")
    with torch.cuda.device(dev):
        if causal is None:
            _check(lib.sattn_fwd_split(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(part_m),
                                       _ptr(part_l), _ptr(part_acc), b, hq, hkv, nq, nk, d, chunk,
                                       _scale(scale, d), _stream(dev)))
        else:
            _check(lib.sattn_fwd_split_cache(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(part_m),
                                             _ptr(part_l), _ptr(part_acc), b, hq, hkv, nq, nk, d, chunk,
                                             int(bool(causal)), _scale(scale, d), _stream(dev)))
    return part_m, part_l, part_acc


def sattn_merge(part_m, part_l, part_acc, dtype, out=None, lse=None):
    """Merge partial states [..., C] / [..., C, D] into (o [..., D] of
    ``dtype``, lse [...] float32)."""
    lib = library()
    f32 = torch.float32
    _dev_tensor(part_m, "part_m", f32)
    _dev_tensor(part_l, "part_l", f32)
    _dev_tensor(part_acc, "part_acc", f32)
    if dtype not in _DTYPE_CODE:
        raise ValueError("dtype must be float16 or bfloat16")
    dev = _same_device(part_m, part_l, part_acc, out, lse)
    lead = tuple(part_m.shape[:-1])
    c = part_m.shape[-1]
    d = part_acc.shape[-1]
    if part_l.shape != part_m.shape or tuple(part_acc.shape[:-1]) != tuple(part_m.shape):
        raise ValueError("partial buffer shape mismatch")
    rows = int(math.prod(lead))
    out = torch.empty(lead + (d,), dtype=dtype, device=dev) if out is None else _dev_tensor(out, "out", dtype)
    lse = torch.empty(lead, dtype=f32, device=dev) if lse is None else _dev_tensor(lse, "lse", f32)
    if tuple(out.shape) != lead + (d,) or tuple(lse.shape) != lead:
        raise ValueError("out/lse shape mismatch")
    with torch.cuda.device(dev):
        _check(lib.sattn_merge(_DTYPE_CODE[dtype], _ptr(part_m), _ptr(part_l), _ptr(part_acc), rows, c, d,
                               _ptr(out), _ptr(lse), _stream(dev)))
    return out, lse


def check_cu_seqlens(cu, total, max_seqlen):
    """Validate a host copy of cu_seqlens: cu[0] = 0, non-decreasing,
    cu[-1] = T, every length <= max_seqlen. Raises ValueError."""
    cu = [int(x) for x in cu]
    if len(cu) < 1 or cu[0] != 0:
        raise ValueError("cu_seqlens must start at 0")
    for a, b in zip(cu[:-1], cu[1:]):
        if b < a:
            raise ValueError("cu_seqlens must be non-decreasing")
        if b - a > max_seqlen:
            raise ValueError("a sequence is longer than max_seqlen")
    if cu[-1] != total:
        raise ValueError("cu_seqlens[-1] must equal T")


def sattn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen=None, causal=True, scale=None, out=None, lse=None,
                     cu_seqlens_host=None):
    """Packed variable-length GQA forward. q [T,Hq,D], k/v [T,Hkv,D];
    cu_seqlens int32 [S+1] (host or device). The table is validated on a host
    copy: pass ``cu_seqlens_host`` (the same offsets, on the host) to skip
    the device-to-host copy, which otherwise synchronizes the stream; the
    device table is then used as given (the kernel still clamps every index
    into [0, T)).

    Returns (o [T,Hq,D], lse [Hq,T] float32)."""
    lib = library()
    _dev_tensor(q, "q", ndim=3)
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("q must be float16 or bfloat16")
    _dev_tensor(k, "k", q.dtype, 3)
    _dev_tensor(v, "v", q.dtype, 3)
    dev = _same_device(q, k, v, out, lse)
    t, hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != t or k.shape[2] != d:
        raise ValueError("k/v must be [T, Hkv, D] matching q")
    hkv = k.shape[1]
    cu_dev, max_seqlen = _cu_device(cu_seqlens, t, max_seqlen, dev, cu_seqlens_host)
    s = cu_dev.numel() - 1
    out = torch.empty_like(q) if out is None else _dev_tensor(out, "out", q.dtype, 3)
    lse = torch.empty((hq, t), dtype=torch.float32, device=dev) if lse is None else \
        _dev_tensor(lse, "lse", torch.float32, 2)
    if out.shape != q.shape or lse.shape != (hq, t):
        raise ValueError("out/lse shape mismatch")
    with torch.cuda.device(dev):
        _check(lib.sattn_fwd_varlen(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                    _ptr(cu_dev), s, t, int(max_seqlen), hq, hkv, d, int(bool(causal)),
                                    _scale(scale, d), _stream(dev)))
    return out, lse


def _cu_device(cu_seqlens, total, max_seqlen, dev, cu_host=None):
    """Host-validated cu_seqlens and its int32 device copy (reused when the
    caller already passes a contiguous int32 tensor on that device). The
    host copy is ``cu_host`` when given, else copied from ``cu_seqlens``."""
    if cu_host is None:
        cu_host = cu_seqlens
    cu_host = cu_host.detach().to("cpu", torch.int64) if isinstance(cu_host, torch.Tensor) else \
        torch.as_tensor(cu_host, dtype=torch.int64)
    lengths = (cu_host[1:] - cu_host[:-1]).tolist()
    if max_seqlen is None:
        max_seqlen = max(lengths) if lengths else 0
    check_cu_seqlens(cu_host.tolist(), total, max_seqlen)
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda and cu_seqlens.dtype == torch.int32 \
            and cu_seqlens.is_contiguous() and cu_seqlens.device == dev:
        if cu_seqlens.numel() != cu_host.numel():
            raise ValueError("cu_seqlens and cu_seqlens_host differ in length")
        return cu_seqlens, int(max_seqlen)
    return cu_host.to(torch.int32).to(dev), int(max_seqlen)


def sattn_bwd_varlen(q, k, v, o, dout, lse, cu_seqlens, max_seqlen=None, causal=True, scale=None, dq=None,
                     dk=None, dv=None, delta=None, cu_seqlens_host=None):
    """Gradients of sum(dout * o) for o, lse = sattn_fwd_varlen(q, k, v,
    cu_seqlens). q, o, dout [T,Hq,D]; k, v [T,Hkv,D]; lse [Hq,T] float32;
    ``delta`` is a float32 [Hq,T] workspace. ``cu_seqlens_host`` as in
    sattn_fwd_varlen.

    Returns (dq, dk, dv) in q's dtype."""
    lib = library()
    _dev_tensor(q, "q", ndim=3)
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("q must be float16 or bfloat16")
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _dev_tensor(t, name, q.dtype, 3)
    t_, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (t_, hkv, d) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q/o/dout must be [T,Hq,D] and k/v [T,Hkv,D]")
    _dev_tensor(lse, "lse", torch.float32, 2)
    if lse.shape != (hq, t_):
        raise ValueError("lse must be [Hq, T]")
    dev = _same_device(q, k, v, o, dout, lse, dq, dk, dv, delta)
    cu_dev, max_seqlen = _cu_device(cu_seqlens, t_, max_seqlen, dev, cu_seqlens_host)
    dq = torch.empty_like(q) if dq is None else _dev_tensor(dq, "dq", q.dtype, 3)
    dk = torch.empty_like(k) if dk is None else _dev_tensor(dk, "dk", q.dtype, 3)
    dv = torch.empty_like(v) if dv is None else _dev_tensor(dv, "dv", q.dtype, 3)
    delta = torch.empty((hq, t_), dtype=torch.float32, device=dev) if delta is None else \
        _dev_tensor(delta, "delta", torch.float32, 2)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape or delta.shape != (hq, t_):
        raise ValueError("gradient/workspace shape mismatch")
    with torch.cuda.device(dev):
        _check(lib.sattn_bwd_varlen(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                    _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_dev),
                                    cu_dev.numel() - 1, t_, max_seqlen, hq, hkv, d, int(bool(causal)),
                                    _scale(scale, d), _stream(dev)))
    return dq, dk, dv


def sattn_bwd_sparse(q, k, v, o, dout, lse, causal=False, window=(-1, -1), n_global=0, block_mask=None,
                     block_q=64, block_k=64, scale=None, dq=None, dk=None, dv=None, delta=None):
    """Gradients of sum(dout * o) for o, lse = sattn_fwd_sparse(q, k, v, ...)
    with Nq = Nk (the same window, n_global, block mask and blocks).
    q, o, dout [B,Hq,N,D]; k, v [B,Hkv,N,D]; lse [B,Hq,N] float32;
    ``delta`` is a float32 [B,Hq,N] workspace.

    Returns (dq, dk, dv) in q's dtype."""
    lib = library()
    _dev_tensor(q, "q", ndim=4)
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("q must be float16 or bfloat16")
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _dev_tensor(t, name, q.dtype, 4)
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    if k.shape != (b, hkv, n, d) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q/o/dout must be [B,Hq,N,D] and k/v [B,Hkv,N,D]")
    _dev_tensor(lse, "lse", torch.float32, 3)
    if lse.shape != (b, hq, n):
        raise ValueError("lse must be [B, Hq, N]")
    dev = _same_device(q, k, v, o, dout, lse, dq, dk, dv, delta, block_mask)
    heads = 0
    if block_mask is not None:
        _dev_tensor(block_mask, "block_mask", torch.uint8)
        if block_mask.dim() == 2:
            block_mask = block_mask.unsqueeze(0)
        nqb, nkb = -(-n // int(block_q)), -(-n // int(block_k))
        if block_mask.dim() != 3 or tuple(block_mask.shape[1:]) != (nqb, nkb):
            raise ValueError("block_mask must be [nqb, nkb] or [heads, %d, %d]" % (nqb, nkb))
        heads = block_mask.shape[0]
    dq = torch.empty_like(q) if dq is None else _dev_tensor(dq, "dq", q.dtype, 4)
    dk = torch.empty_like(k) if dk is None else _dev_tensor(dk, "dk", q.dtype, 4)
    dv = torch.empty_like(v) if dv is None else _dev_tensor(dv, "dv", q.dtype, 4)
    delta = torch.empty((b, hq, n), dtype=torch.float32, device=dev) if delta is None else \
        _dev_tensor(delta, "delta", torch.float32, 3)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape or delta.shape != (b, hq, n):
        raise ValueError("gradient/workspace shape mismatch")
    left, right = window
    with torch.cuda.device(dev):
        _check(lib.sattn_bwd_sparse(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                    _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), b, hq, hkv, n, d,
                                    int(bool(causal)), int(left), int(right), int(n_global), _ptr(block_mask),
                                    heads, int(block_q), int(block_k), _scale(scale, d), _stream(dev)))
    return dq, dk, dv


def sattn_bwd_cache(q, k, v, o, dout, lse, causal=False, scale=None, dq=None, dk=None, dv=None, delta=None):
    """Gradients of sum(dout * o) for o, lse = sattn_fwd_cache(q, k, v):
    q, o, dout [B,Hq,Nq,D]; k, v [B,Hkv,Nk,D] (query i at position
    i + Nk - Nq); lse [B,Hq,Nq] float32; ``delta`` a float32 [B,Hq,Nq]
    workspace.

    Returns (dq, dk, dv) in q's dtype."""
    lib = library()
    b, hq, nq, d, hkv, nk = _cache_shapes(q, k, v)
    for t, name in ((o, "o"), (dout, "dout")):
        _dev_tensor(t, name, q.dtype, 4)
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o/dout must match q")
    _dev_tensor(lse, "lse", torch.float32, 3)
    if lse.shape != (b, hq, nq):
        raise ValueError("lse must be [B, Hq, Nq]")
    dev = _same_device(q, k, v, o, dout, lse, dq, dk, dv, delta)
    dq = torch.empty_like(q) if dq is None else _dev_tensor(dq, "dq", q.dtype, 4)
    dk = torch.empty_like(k) if dk is None else _dev_tensor(dk, "dk", q.dtype, 4)
    dv = torch.empty_like(v) if dv is None else _dev_tensor(dv, "dv", q.dtype, 4)
    delta = torch.empty((b, hq, nq), dtype=torch.float32, device=dev) if delta is None else \
        _dev_tensor(delta, "delta", torch.float32, 3)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape or delta.shape != (b, hq, nq):
        raise ValueError("gradient/workspace shape mismatch")
    with torch.cuda.device(dev):
        _check(lib.sattn_bwd_cache(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                   _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), b, hq, hkv, nq, nk, d,
                                   int(bool(causal)), _scale(scale, d), _stream(dev)))
    return dq, dk, dv

"""The C ABI library loads, exports every symbol the header declares, and
rejects invalid calls before any launch (CPU only: no call here reaches the
HIP runtime; each case fails one of the host-side checks).
"""
import ctypes
import os
import re

import pytest

from exact_tiled_attention_sattn_amd import LIB_PATH, STATUS, library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sattn.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sattn_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        from exact_tiled_attention_sattn_amd import build
        build.build()
    return library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("sattn_fwd", "sattn_fwd_split", "sattn_merge", "sattn_fwd_varlen", "sattn_fwd_cache",
              "sattn_fwd_split_cache", "sattn_status_string", "sattn_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(LIB_PATH)
    for name in _declared_functions():
        assert hasattr(raw, name), "libsattn.so does not export %s" % name


def test_status_strings(lib):
    for code, name in STATUS.items():
        assert lib.sattn_status_string(code).decode() == name
    assert lib.sattn_status_string(99).decode() == "SATTN_ERR_UNKNOWN"


I64 = ctypes.c_int64
F32 = ctypes.c_float
FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: every call below fails validation first
FAKE2 = ctypes.c_void_p(0x20000)
FAKE3 = ctypes.c_void_p(0x30000)
FAKE4 = ctypes.c_void_p(0x40000)
FAKE5 = ctypes.c_void_p(0x50000)
NULL = ctypes.c_void_p(0)


def _fwd(lib, dtype=1, q=FAKE, k=FAKE2, v=FAKE3, o=FAKE4, lse=FAKE5, b=1, h=1, n=8, d=64, causal=0, scale=0.125):
    return lib.sattn_fwd(dtype, q, k, v, o, lse, b, h, n, d, causal, scale, NULL)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=7), "SATTN_ERR_DTYPE"),
    (dict(d=96), "SATTN_ERR_UNSUPPORTED"),
    (dict(d=-1), "SATTN_ERR_SHAPE"),
    (dict(n=-3), "SATTN_ERR_SHAPE"),
    (dict(scale=0.0), "SATTN_ERR_VALUE"),
    (dict(scale=-1.0), "SATTN_ERR_VALUE"),
    (dict(scale=float("nan")), "SATTN_ERR_VALUE"),
    (dict(scale=float("inf")), "SATTN_ERR_VALUE"),
    (dict(q=NULL), "SATTN_ERR_NULL"),
    (dict(lse=NULL), "SATTN_ERR_NULL"),
    (dict(q=ctypes.c_void_p(0x10008)), "SATTN_ERR_ALIGN"),
    (dict(lse=ctypes.c_void_p(0x50002)), "SATTN_ERR_ALIGN"),
    (dict(o=FAKE), "SATTN_ERR_ALIAS"),                          # o == q
    (dict(o=ctypes.c_void_p(0x10000 + 512)), "SATTN_ERR_ALIAS"),  # o inside q's 1 KiB
    (dict(lse=ctypes.c_void_p(0x40000 + 16)), "SATTN_ERR_ALIAS"),  # lse inside o
    (dict(b=1 << 40, h=1 << 40), "SATTN_ERR_SHAPE"),              # element count overflows
    (dict(n=1 << 31), "SATTN_ERR_UNSUPPORTED"),
])
def test_fwd_rejects(lib, kwargs, status):
    st = _fwd(lib, **kwargs)
    assert STATUS[st] == status, (STATUS[st], lib.sattn_last_error())
    assert lib.sattn_last_error().decode() != ""


def test_fwd_zero_size_is_ok_without_pointers(lib):
    assert _fwd(lib, q=NULL, k=NULL, v=NULL, o=NULL, lse=NULL, n=0) == 0
    assert _fwd(lib, q=NULL, k=NULL, v=NULL, o=NULL, lse=NULL, b=0) == 0


def _split(lib, b=1, hq=4, hkv=2, nq=1, nk=100, d=128, chunk=32, q=FAKE, k=FAKE2, v=FAKE3,
           pm=ctypes.c_void_p(0x900000), pl=ctypes.c_void_p(0xA00000), pa=ctypes.c_void_p(0xB00000)):
    return lib.sattn_fwd_split(1, q, k, v, pm, pl, pa, b, hq, hkv, nq, nk, d, chunk, F32(0.1), NULL)


@pytest.mark.parametrize("kwargs,status", [
    (dict(chunk=0), "SATTN_ERR_SHAPE"),
    (dict(chunk=-5), "SATTN_ERR_SHAPE"),
    (dict(hq=6, hkv=4), "SATTN_ERR_SHAPE"),
    (dict(hkv=0), "SATTN_ERR_SHAPE"),
    (dict(nk=0), "SATTN_ERR_SHAPE"),
    (dict(d=48), "SATTN_ERR_UNSUPPORTED"),
    (dict(pa=NULL), "SATTN_ERR_NULL"),
    (dict(pa=ctypes.c_void_p(0xB00004)), "SATTN_ERR_ALIGN"),
    (dict(pm=FAKE2), "SATTN_ERR_ALIAS"),
    (dict(pl=ctypes.c_void_p(0x900000)), "SATTN_ERR_ALIAS"),
])
def test_split_rejects(lib, kwargs, status):
    st = _split(lib, **kwargs)
    assert STATUS[st] == status, (STATUS[st], lib.sattn_last_error())


def test_split_zero_rows_ok(lib):
    assert _split(lib, nq=0, q=NULL, k=NULL, v=NULL, pm=NULL, pl=NULL, pa=NULL) == 0


def test_merge_rejects(lib):
    pm, pl, pa = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000)
    o, lse = ctypes.c_void_p(0x400000), ctypes.c_void_p(0x500000)
    assert STATUS[lib.sattn_merge(1, pm, pl, pa, 4, 0, 128, o, lse, NULL)] == "SATTN_ERR_SHAPE"
    assert STATUS[lib.sattn_merge(1, pm, pl, pa, -1, 2, 128, o, lse, NULL)] == "SATTN_ERR_SHAPE"
    assert STATUS[lib.sattn_merge(2, pm, pl, pa, 4, 2, 128, o, lse, NULL)] == "SATTN_ERR_DTYPE"
    assert STATUS[lib.sattn_merge(1, pm, pl, pa, 4, 2, 128, pa, lse, NULL)] == "SATTN_ERR_ALIAS"
    assert STATUS[lib.sattn_merge(1, pm, pl, NULL, 4, 2, 128, o, lse, NULL)] == "SATTN_ERR_NULL"
    assert lib.sattn_merge(1, NULL, NULL, NULL, 0, 2, 128, NULL, NULL, NULL) == 0


def test_varlen_rejects(lib):
    cu = ctypes.c_void_p(0x600000)

    def call(**kw):
        a = dict(dtype=1, q=FAKE, k=FAKE2, v=FAKE3, o=FAKE4, lse=FAKE5, cu=cu, s=2, t=10, mx=6, hq=4,
                 hkv=2, d=64, causal=1, scale=0.1)
        a.update(kw)
        return STATUS[lib.sattn_fwd_varlen(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["s"],
                                           a["t"], a["mx"], a["hq"], a["hkv"], a["d"], a["causal"],
                                           F32(a["scale"]), NULL)]
    assert call(hq=3) == "SATTN_ERR_SHAPE"
    assert call(mx=11) == "SATTN_ERR_SHAPE"
    assert call(cu=NULL) == "SATTN_ERR_NULL"
    assert call(cu=ctypes.c_void_p(0x600002)) == "SATTN_ERR_ALIGN"
    assert call(o=FAKE) == "SATTN_ERR_ALIAS"
    assert call(lse=cu) == "SATTN_ERR_ALIAS"
    assert call(d=16) == "SATTN_ERR_UNSUPPORTED"
    assert call(t=0, q=NULL, k=NULL, v=NULL, o=NULL, lse=NULL, cu=NULL) == "SATTN_OK"


def test_binding_checks_cu_seqlens_on_host():
    from exact_tiled_attention_sattn_amd import check_cu_seqlens
    check_cu_seqlens([0, 3, 3, 10], 10, 7)
    for bad, t, mx in (([1, 3], 3, 5), ([0, 5, 4], 4, 5), ([0, 4], 5, 5), ([0, 9], 9, 8)):
        with pytest.raises(ValueError):
            check_cu_seqlens(bad, t, mx)


def _cache(lib, b=1, hq=4, hkv=2, nq=8, nk=100, d=128, causal=1, q=FAKE, k=FAKE2, v=FAKE3, o=FAKE4, lse=FAKE5,
           scale=0.1):
    return lib.sattn_fwd_cache(1, q, k, v, o, lse, b, hq, hkv, nq, nk, d, causal, F32(scale), NULL)


@pytest.mark.parametrize("kwargs,status", [
    (dict(hq=6, hkv=4), "SATTN_ERR_SHAPE"),
    (dict(hkv=0), "SATTN_ERR_SHAPE"),
    (dict(nk=-1), "SATTN_ERR_SHAPE"),
    (dict(nq=-1), "SATTN_ERR_SHAPE"),
    (dict(d=80), "SATTN_ERR_UNSUPPORTED"),
    (dict(nk=1 << 31), "SATTN_ERR_UNSUPPORTED"),
    (dict(scale=0.0), "SATTN_ERR_VALUE"),
    (dict(k=NULL), "SATTN_ERR_NULL"),
    (dict(lse=NULL), "SATTN_ERR_NULL"),
    (dict(o=ctypes.c_void_p(0x40008)), "SATTN_ERR_ALIGN"),
    (dict(o=FAKE2), "SATTN_ERR_ALIAS"),                             # o == k
    (dict(lse=ctypes.c_void_p(0x40000 + 64)), "SATTN_ERR_ALIAS"),   # lse inside o
])
def test_cache_rejects(lib, kwargs, status):
    st = _cache(lib, **kwargs)
    assert STATUS[st] == status, (STATUS[st], lib.sattn_last_error())


def test_cache_zero_queries_ok_without_pointers(lib):
    assert _cache(lib, nq=0, q=NULL, k=NULL, v=NULL, o=NULL, lse=NULL) == 0
    assert _cache(lib, hq=0, q=NULL, k=NULL, v=NULL, o=NULL, lse=NULL) == 0


def test_split_cache_rejects(lib):
    pm, pl, pa = ctypes.c_void_p(0x900000), ctypes.c_void_p(0xA00000), ctypes.c_void_p(0xB00000)

    def call(**kw):
        a = dict(b=1, hq=4, hkv=2, nq=3, nk=100, d=128, chunk=32, causal=1, pm=pm)
        a.update(kw)
        return STATUS[lib.sattn_fwd_split_cache(1, FAKE, FAKE2, FAKE3, a["pm"], pl, pa, a["b"], a["hq"], a["hkv"],
                                                a["nq"], a["nk"], a["d"], a["chunk"], a["causal"], F32(0.1),
                                                NULL)]
    assert call(chunk=0) == "SATTN_ERR_SHAPE"
    assert call(hq=3) == "SATTN_ERR_SHAPE"
    assert call(nk=0) == "SATTN_ERR_SHAPE"
    assert call(d=16) == "SATTN_ERR_UNSUPPORTED"
    assert call(pm=FAKE) == "SATTN_ERR_ALIAS"
    assert call(pm=NULL) == "SATTN_ERR_NULL"
    assert call(nq=0, pm=NULL) == "SATTN_OK"


def test_strided_rejects(lib):
    Arr = ctypes.c_int64 * 3

    def call(qs=(8192, 1024, 128), ks=(8192, 1024, 128), **kw):
        a = dict(b=1, hq=4, hkv=2, nq=8, nk=8, d=128, q=FAKE, k=FAKE2, v=FAKE3, o=FAKE4, lse=FAKE5)
        a.update(kw)
        return STATUS[lib.sattn_fwd_strided(1, a["q"], a["k"], a["v"], a["o"], a["lse"], a["b"], a["hq"], a["hkv"],
                                            a["nq"], a["nk"], a["d"], Arr(*qs) if qs else None,
                                            Arr(*ks) if ks else None, 1, F32(0.1), NULL)]
    assert call(qs=(8192, 1024, 130)) == "SATTN_ERR_ALIGN"          # row stride not 16-byte aligned
    assert call(ks=(8192, -1024, 128)) == "SATTN_ERR_ALIGN"         # negative stride
    assert call(ks=(8192, 1024, 0)) == "SATTN_ERR_UNSUPPORTED"      # k/v rows must advance
    assert call(ks=(8192, 1024, 64)) == "SATTN_ERR_UNSUPPORTED"     # ... by at least D
    assert call(ks=(8192, 1024, 1 << 24), nk=100) == "SATTN_ERR_UNSUPPORTED"   # slice spans >= 2 GiB
    assert call(qs=None) == "SATTN_ERR_NULL"
    assert call(o=ctypes.c_void_p(0x10000 + 4096)) == "SATTN_ERR_ALIAS"   # o starts inside q (extent 8 KiB)
    assert call(nq=0, q=NULL, k=NULL, v=NULL, o=NULL, lse=NULL) == "SATTN_OK"


def test_sparse_rejects(lib):
    mask = ctypes.c_void_p(0x700000)

    def call(**kw):
        a = dict(nq=256, nk=256, left=-1, right=-1, g=0, mask=mask, heads=1, bq=64, bk=64, hq=4, o=FAKE4)
        a.update(kw)
        return STATUS[lib.sattn_fwd_sparse(1, FAKE, FAKE2, FAKE3, a["o"], FAKE5, 1, a["hq"], 2, a["nq"], a["nk"], 128,
                                           1, a["left"], a["right"], a["g"], a["mask"], a["heads"], a["bq"],
                                           a["bk"], F32(0.1), NULL)]
    assert call(nk=65537, nq=8) == "SATTN_ERR_UNSUPPORTED"       # longer than the tile list
    assert call(left=-2) == "SATTN_ERR_VALUE"
    assert call(g=-1) == "SATTN_ERR_VALUE"
    assert call(bq=48) == "SATTN_ERR_UNSUPPORTED"                # query blocks: multiples of 32
    assert call(bk=32) == "SATTN_ERR_UNSUPPORTED"                # key blocks: multiples of 64
    assert call(heads=3) == "SATTN_ERR_SHAPE"                    # 1 or Hq
    assert call(o=mask) == "SATTN_ERR_ALIAS"                     # output over the mask


# Backward entry points: q 0x100000, k 0x200000, v 0x300000, o 0x400000,
# dout 0x500000, lse 0x600000, delta 0x700000, dq 0x800000, dk 0x900000,
# dv 0xA00000, cu_seqlens 0xB00000 (each 1 MiB apart; the buffers below are
# a few KiB).
def _bp(x):
    return ctypes.c_void_p(x)


BWD_PTRS = dict(q=0x100000, k=0x200000, v=0x300000, o=0x400000, dout=0x500000, lse=0x600000, delta=0x700000,
                dq=0x800000, dk=0x900000, dv=0xA00000)


def _bwd(lib, dtype=1, b=1, hq=2, hkv=1, n=8, d=64, **ptrs):
    a = dict(BWD_PTRS)
    a.update(ptrs)
    return lib.sattn_bwd(dtype, *(_bp(a[x]) for x in ("q", "k", "v", "o", "dout", "lse", "delta", "dq", "dk", "dv")),
                         b, hq, hkv, n, d, 1, F32(0.125), NULL)


def _bwd_varlen(lib, dtype=1, s=2, t=8, max_seqlen=5, hq=2, hkv=1, d=64, cu=0xB00000, **ptrs):
    a = dict(BWD_PTRS)
    a.update(ptrs)
    return lib.sattn_bwd_varlen(dtype, *(_bp(a[x]) for x in ("q", "k", "v", "o", "dout", "lse", "delta", "dq", "dk",
                                                              "dv")),
                                _bp(cu), s, t, max_seqlen, hq, hkv, d, 1, F32(0.125), NULL)


BWD_REJECTS = [
    (dict(dtype=5), "SATTN_ERR_DTYPE"),
    (dict(d=48), "SATTN_ERR_UNSUPPORTED"),
    (dict(hq=3, hkv=2), "SATTN_ERR_SHAPE"),
    (dict(dq=0), "SATTN_ERR_NULL"),
    (dict(delta=0), "SATTN_ERR_NULL"),
    (dict(dq=0x800008), "SATTN_ERR_ALIGN"),
    (dict(delta=0x700002), "SATTN_ERR_ALIGN"),
    (dict(dq=0x100000), "SATTN_ERR_ALIAS"),          # dq over q
    (dict(dk=0x200000 + 256), "SATTN_ERR_ALIAS"),    # dk inside k
    (dict(dv=0x900000), "SATTN_ERR_ALIAS"),          # dv over dk (two outputs)
    (dict(delta=0x600000), "SATTN_ERR_ALIAS"),       # delta over lse
]


@pytest.mark.parametrize("kwargs,status", BWD_REJECTS + [(dict(n=-1), "SATTN_ERR_SHAPE")])
def test_bwd_rejects(lib, kwargs, status):
    st = _bwd(lib, **kwargs)
    assert STATUS[st] == status, (STATUS[st], lib.sattn_last_error())


@pytest.mark.parametrize("kwargs,status", BWD_REJECTS + [
    (dict(s=-1), "SATTN_ERR_SHAPE"),
    (dict(max_seqlen=9), "SATTN_ERR_SHAPE"),          # longer than T
    (dict(cu=0), "SATTN_ERR_NULL"),
    (dict(cu=0xB00002), "SATTN_ERR_ALIGN"),
    (dict(delta=0xB00000), "SATTN_ERR_ALIAS"),        # delta over cu_seqlens
])
def test_bwd_varlen_rejects(lib, kwargs, status):
    st = _bwd_varlen(lib, **kwargs)
    assert STATUS[st] == status, (STATUS[st], lib.sattn_last_error())


def test_bwd_zero_sizes_ok_without_pointers(lib):
    nulls = {x: 0 for x in BWD_PTRS}
    assert _bwd(lib, n=0, **nulls) == 0
    assert _bwd(lib, b=0, **nulls) == 0
    assert _bwd_varlen(lib, t=0, s=0, max_seqlen=0, cu=0, **nulls) == 0
    assert _bwd_varlen(lib, s=0, cu=0, **nulls) == 0


def _bwd_sparse(lib, left=-1, right=-1, g=0, mask=0x700000 + 4096, heads=1, bq=64, bk=64, hq=2, n=8, **ptrs):
    a = dict(BWD_PTRS)
    a.update(ptrs)
    return lib.sattn_bwd_sparse(1, *(_bp(a[x]) for x in ("q", "k", "v", "o", "dout", "lse", "delta", "dq", "dk",
                                                          "dv")),
                                1, hq, 1, n, 64, 1, left, right, g, _bp(mask), heads, bq, bk, F32(0.125), NULL)


@pytest.mark.parametrize("kwargs,status", [
    (dict(left=-2), "SATTN_ERR_VALUE"),
    (dict(g=-1), "SATTN_ERR_VALUE"),
    (dict(bq=48), "SATTN_ERR_UNSUPPORTED"),
    (dict(bk=96), "SATTN_ERR_UNSUPPORTED"),
    (dict(heads=3), "SATTN_ERR_SHAPE"),
    (dict(delta=0x700000 + 4096), "SATTN_ERR_ALIAS"),     # workspace over the mask
    (dict(dq=0), "SATTN_ERR_NULL"),
    (dict(heads=2, hq=4), "SATTN_ERR_SHAPE"),              # per-head masks must number Hq
])
def test_bwd_sparse_rejects(lib, kwargs, status):
    st = _bwd_sparse(lib, **kwargs)
    assert STATUS[st] == status, (STATUS[st], lib.sattn_last_error())


def test_bwd_sparse_zero_size_ok(lib):
    assert _bwd_sparse(lib, n=0, mask=0, **{x: 0 for x in BWD_PTRS}) == 0


def _bwd_cache(lib, nq=8, nk=16, hq=2, **ptrs):
    a = dict(BWD_PTRS)
    a.update(ptrs)
    return lib.sattn_bwd_cache(1, *(_bp(a[x]) for x in ("q", "k", "v", "o", "dout", "lse", "delta", "dq", "dk", "dv")),
                               1, hq, 1, nq, nk, 64, 1, F32(0.125), NULL)


@pytest.mark.parametrize("kwargs,status", [
    (dict(nk=-1), "SATTN_ERR_SHAPE"),
    (dict(dk=0), "SATTN_ERR_NULL"),                      # keys exist: dk needed
    (dict(dk=0x200000 + 1024), "SATTN_ERR_ALIAS"),       # dk inside k (16 keys x 64 x 2 B = 2 KiB)
    (dict(nk=1 << 31), "SATTN_ERR_UNSUPPORTED"),
])
def test_bwd_cache_rejects(lib, kwargs, status):
    st = _bwd_cache(lib, **kwargs)
    assert STATUS[st] == status, (STATUS[st], lib.sattn_last_error())


def test_bwd_cache_zero_queries_ok(lib):
    assert _bwd_cache(lib, nq=0, **{x: 0 for x in BWD_PTRS}) == 0


def _bwd_noalloc(lib, dtype=1, b=1, hq=2, hkv=1, n=8, d=64, **ptrs):
    a = dict(BWD_PTRS)
    a.update(ptrs)
    return lib.sattn_bwd_noalloc(dtype, *(_bp(a[x]) for x in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv")),
                                 b, hq, hkv, n, d, 1, F32(0.125), NULL)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=5), "SATTN_ERR_DTYPE"),
    (dict(d=48), "SATTN_ERR_UNSUPPORTED"),
    (dict(hq=3, hkv=2), "SATTN_ERR_SHAPE"),
    (dict(n=-1), "SATTN_ERR_SHAPE"),
    (dict(dq=0), "SATTN_ERR_NULL"),
    (dict(dq=0x800008), "SATTN_ERR_ALIGN"),
    (dict(dq=0x100000), "SATTN_ERR_ALIAS"),
    # more query rows than the static scratch holds (2^21): rejected before
    # any pointer is used or the HIP runtime is reached
    (dict(b=64, hq=64, n=1024, q=0, k=0, v=0, o=0, dout=0, lse=0, dq=0, dk=0, dv=0), "SATTN_ERR_UNSUPPORTED"),
])
def test_bwd_noalloc_rejects(lib, kwargs, status):
    st = _bwd_noalloc(lib, **kwargs)
    assert STATUS[st] == status, (STATUS[st], lib.sattn_last_error())
    if status == "SATTN_ERR_UNSUPPORTED" and kwargs.get("b") == 64:
        assert b"static scratch" in lib.sattn_last_error()


def test_bwd_noalloc_zero_size_ok_without_pointers(lib):
    nulls = {x: 0 for x in BWD_PTRS}
    assert _bwd_noalloc(lib, n=0, **nulls) == 0
    assert _bwd_noalloc(lib, b=0, **nulls) == 0


PROBE_HEADER = os.path.join(ROOT, "include", "sattn_probe.h")


def test_probe_library_exports_its_header_and_rejects_bad_arguments(lib):
    """The bandwidth probe (libsattn_probe.so, used by bench.py --read-ceiling)
    exports what its header declares and refuses invalid calls before any
    launch."""
    from exact_tiled_attention_sattn_amd.build import PROBE_LIB
    assert os.path.exists(PROBE_LIB), "libsattn_probe.so is built beside libsattn.so"
    src = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(sattn_[a-z_]+)\s*\(", src)))
    assert names == ["sattn_probe_read"]
    probe = ctypes.CDLL(PROBE_LIB)
    probe.sattn_probe_read.restype = ctypes.c_int
    probe.sattn_probe_read.argtypes = [ctypes.c_void_p, I64, ctypes.c_void_p, I64, ctypes.c_int, ctypes.c_void_p]
    ok = dict(buf=FAKE, nbytes=1 << 20, out=FAKE2, count=1024 * 256, grid=1024)
    for bad in (dict(buf=NULL), dict(out=NULL), dict(nbytes=0), dict(nbytes=100), dict(buf=ctypes.c_void_p(0x10008)),
                dict(grid=0), dict(grid=70000), dict(count=1023 * 256)):
        a = dict(ok, **bad)
        assert probe.sattn_probe_read(a["buf"], a["nbytes"], a["out"], a["count"], a["grid"], NULL) == -1, bad

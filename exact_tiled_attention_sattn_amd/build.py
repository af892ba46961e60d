"""Build libsattn.so (HIP, gfx950) in-tree with hipcc.

Each kernel family is its own translation unit (csrc/k_*.hip) next to the C
ABI layer (csrc/sattn.hip); they compile in parallel into objects under
``_build/`` and link into ``libsattn.so``.

Design-variant libraries (``libsattn_<name>.so``) rebuild only the dense
forward unit and the C ABI layer with one design choice changed, and link
them with the product's other objects. They exist to time a design choice
against the product on the same box (``bench.py --variants``); nothing else
loads them.

Usage: python -m exact_tiled_attention_sattn_amd.build [-v] [--no-variants]
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsattn.so")
# The bandwidth probe behind `bench.py --read-ceiling` (not part of the
# attention path; its own library).
PROBE_LIB = os.path.join(PKG, "libsattn_probe.so")
UNITS = ["sattn", "k_fwd_dense", "k_fwd_varlen", "k_fwd_split", "k_fwd_cache", "k_fwd_sparse",
         "k_bwd_dense", "k_bwd_varlen", "k_bwd_sparse"]
ARCH = "gfx950"

# Packed fp32 VALU forms are switched off for all device code.
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]

# One design choice each, changed against the product (see the dense
# forward kernel): 32- or 128-key tiles, one K/V tile buffer instead of two,
# causal key tiles after the diagonal visited and masked instead of skipped,
# causal query tiles not paired.
VARIANTS = {
    "bn32": ["-DSATTN_DENSE_BN=32"],
    "bn128": ["-DSATTN_DENSE_BN=128"],
    "single_buffer": ["-DSATTN_SINGLE_BUFFER=1"],
    "no_causal_skip": ["-DSATTN_NO_CAUSAL_SKIP=1"],
    "no_pair": ["-DSATTN_NO_PAIR=1"],
}
VARIANT_UNITS = ["sattn", "k_fwd_dense"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsattn.so)")


def variant_path(name):
    return os.path.join(PKG, "libsattn_%s.so" % name)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s\n%s\n%s" % (res.returncode, " ".join(cmd), res.stdout,
                                                                res.stderr))


def _compile(unit, tag, extra, verbose):
    out = os.path.join(OBJ, "%s%s.o" % (unit, tag))
    _run([hipcc()] + HIPCC_FLAGS + extra + ["-c", "-o", out, os.path.join(CSRC, unit + ".hip")], verbose)
    return out


def _link(objs, path, verbose):
    fd, tmp = tempfile.mkstemp(prefix=os.path.basename(path) + ".", suffix=".tmp", dir=PKG)
    os.close(fd)
    try:
        _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
        os.replace(tmp, path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return path


def build(verbose=False, variants=True, jobs=None):
    """Compile the library (always recompiles every unit), and the
    design-variant libraries unless ``variants`` is false. Returns the
    library path."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(16, os.cpu_count() or 4)
    tasks = [(u, "", []) for u in UNITS] + [("probe_read", "", [])]
    if variants:
        tasks += [(u, "." + name, flags) for name, flags in VARIANTS.items() for u in VARIANT_UNITS]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {ex.submit(_compile, u, tag, extra, verbose): (u, tag) for u, tag, extra in tasks}
        objs = {}
        for f in cf.as_completed(futs):
            objs[futs[f]] = f.result()
    lib = _link([objs[(u, "")] for u in UNITS], LIB, verbose)
    _link([objs[("probe_read", "")]], PROBE_LIB, verbose)
    if variants:
        for name in VARIANTS:
            parts = [objs[(u, "." + name)] if u in VARIANT_UNITS else objs[(u, "")] for u in UNITS]
            _link(parts, variant_path(name), verbose)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, variants="--no-variants" not in sys.argv))

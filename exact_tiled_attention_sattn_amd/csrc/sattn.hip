// libsattn: C ABI host layer. Validates every argument before any launch,
// picks the kernel instance for (dtype, D, causal, mode), and enqueues it on
// the caller's stream. Allocates nothing; keeps no mutable global state
// except a thread-local error message.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "sattn.h"
#include "launch.hpp"

// Workspace of the allocation-free backward entry point (see
// scratch_on_current_device below): 2^21 floats.
static __device__ __align__(256) float scratch[int64_t(1) << 21];

namespace {

using namespace sattn;

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return SATTN_OK;
}

// Positions inside one sequence or slice are kept in 32-bit registers.
constexpr int64_t kMaxLen = int64_t(1) << 30;
// K/V tiles are fetched with buffer loads whose byte offset within one slice
// (or one packed sequence) is 32-bit.
constexpr int64_t kMaxSpan = int64_t(1) << 31;

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

bool product(std::initializer_list<int64_t> xs, int64_t* out) {
  int64_t acc = 1;
  for (int64_t x : xs)
    if (!mul_ok(acc, x, &acc)) return false;
  *out = acc;
  return true;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  const char* name;
};

bool overlap(const Range& a, const Range& b) {
  if (a.hi <= a.lo || b.hi <= b.lo) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

Range range_of(const void* p, int64_t bytes, const char* name) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes), name};
}

// Outputs must not overlap inputs or each other.
int check_alias(const Range* ins, int nin, const Range* outs, int nout) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j]))
        return fail(SATTN_ERR_ALIAS, "output %s overlaps input %s", outs[i].name, ins[j].name);
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j]))
        return fail(SATTN_ERR_ALIAS, "output %s overlaps output %s", outs[i].name, outs[j].name);
  }
  return SATTN_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_common(int dtype, int64_t D, float scale) {
  if (dtype != SATTN_F16 && dtype != SATTN_BF16) return fail(SATTN_ERR_DTYPE, "dtype %d is not F16/BF16", dtype);
  if (D < 0) return fail(SATTN_ERR_SHAPE, "negative D");
  if (D != 32 && D != 64 && D != 128) return fail(SATTN_ERR_UNSUPPORTED, "head dim D=%lld not in {32,64,128}", (long long)D);
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(SATTN_ERR_VALUE, "scale must be finite and > 0");
  return SATTN_OK;
}

int launch_status() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Query rows per workgroup of each mode of the streaming kernel.
template <int MODE>
int tile_m(int64_t D) {
  switch (D) {
    case 32: return Tile<32, MODE>::BM;
    case 64: return Tile<64, MODE>::BM;
    default: return Tile<128, MODE>::BM;
  }
}

// Causal dense workgroups take a pair of query tiles (equal work per
// workgroup) once the grid has enough tiles that pairing still leaves
// several workgroups per CU (a build-time knob for the design-variant
// builds; the library pairs).
#ifdef SATTN_NO_PAIR
constexpr bool kPairCausal = false;
#else
constexpr bool kPairCausal = true;
#endif

FwdParams blank_params(float scale) {
  FwdParams p{};
  p.c = scale * kLog2e;
  return p;
}

// Scratch of the allocation-free backward entry point: the Delta rows live
// in this file-scope device array (each GPU the library runs on holds its own
// copy until the process ends). Host code must never pass `scratch` itself
// to a kernel: its host-side name is only a handle; the device address comes
// from hipGetSymbolAddress, taken once per device with that device current.
constexpr int64_t kScratchFloats = sizeof(scratch) / sizeof(float);   // 8 MiB: up to 2^21 query rows

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (cached per
// device). Returns SATTN_OK or SATTN_ERR_HIP.
int scratch_on_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SATTN_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SATTN_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(SATTN_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return SATTN_OK;
}

}  // namespace

extern "C" {

const char* sattn_status_string(int status) {
  switch (status) {
    case SATTN_OK: return "SATTN_OK";
    case SATTN_ERR_NULL: return "SATTN_ERR_NULL";
    case SATTN_ERR_SHAPE: return "SATTN_ERR_SHAPE";
    case SATTN_ERR_DTYPE: return "SATTN_ERR_DTYPE";
    case SATTN_ERR_UNSUPPORTED: return "SATTN_ERR_UNSUPPORTED";
    case SATTN_ERR_ALIGN: return "SATTN_ERR_ALIGN";
    case SATTN_ERR_ALIAS: return "SATTN_ERR_ALIAS";
    case SATTN_ERR_HIP: return "SATTN_ERR_HIP";
    case SATTN_ERR_VALUE: return "SATTN_ERR_VALUE";
    default: return "SATTN_ERR_UNKNOWN";
  }
}

const char* sattn_last_error(void) { return g_err; }

int sattn_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
              int64_t N, int64_t D, int causal, float scale, void* stream) {
  int st = check_common(dtype, D, scale);
  if (st) return st;
  if (B < 0 || H < 0 || N < 0) return fail(SATTN_ERR_SHAPE, "negative size");
  int64_t heads, rows, elems;
  if (!product({B, H}, &heads) || !product({heads, N}, &rows) || !product({rows, D, 2}, &elems))
    return fail(SATTN_ERR_SHAPE, "size overflow");
  if (N >= kMaxLen || heads >= kMaxLen) return fail(SATTN_ERR_UNSUPPORTED, "N or B*H too large");
  if (rows == 0) return ok();
  if (!q || !k || !v || !o || !lse) return fail(SATTN_ERR_NULL, "null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return fail(SATTN_ERR_ALIGN, "q/k/v/o need 16-byte and lse 4-byte alignment");
  const int64_t bytes = elems;  // rows * D * 2
  Range ins[3] = {range_of(q, bytes, "q"), range_of(k, bytes, "k"), range_of(v, bytes, "v")};
  Range outs[2] = {range_of(o, bytes, "o"), range_of(lse, rows * 4, "lse")};
  if ((st = check_alias(ins, 3, outs, 2))) return st;

  if (N * D * 2 >= kMaxSpan) return fail(SATTN_ERR_UNSUPPORTED, "K/V slice larger than 2 GiB");
  // Small problems (at most one workgroup of 32 rows per CU): split each
  // head's keys between the waves of a workgroup to shorten the serial chain.
  const int64_t nq32 = (N + 31) / 32;
  if (D <= 64 && heads * nq32 <= 256) {
    FwdParams p = blank_params(scale);
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.o = (uint16_t*)o;
    p.lse = lse;
    p.heads = (int)heads;
    p.n = (int)N;
    p.nqt = (int)nq32;
    // 8 waves when a query tile may see more than 4 key tiles, else 4.
    const bool wide = (N + 63) / 64 > 4;
    launch_fwd_small(dtype, (int)D, causal != 0, wide, p, heads * nq32, (hipStream_t)stream);
    return launch_status();
  }
  const int bm = tile_m<MODE_DENSE>(D);
  const int64_t nqt = (N + bm - 1) / bm;
  // Causal workgroups take a pair of query tiles (equal work per workgroup)
  // once the grid has enough tiles that pairing still leaves several
  // workgroups per CU.
  const bool pair = kPairCausal && causal && nqt * heads >= 1024;
  const int64_t grid = (pair ? (nqt + 1) / 2 : nqt) * heads;
  if (grid >= (int64_t(1) << 31)) return fail(SATTN_ERR_UNSUPPORTED, "grid too large");
  FwdParams p = blank_params(scale);
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.heads = (int)heads;
  p.n = (int)N;
  p.nqt = (int)nqt;
  p.pair = pair ? 1 : 0;
  launch_fwd_dense(dtype, (int)D, causal != 0, p, grid, (hipStream_t)stream);
  return launch_status();
}

static int split_impl(int dtype, const void* q, const void* k, const void* v, float* part_m, float* part_l,
                      float* part_acc, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                      int64_t chunk, bool causal, float scale, void* stream) {
  int st = check_common(dtype, D, scale);
  if (st) return st;
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0) return fail(SATTN_ERR_SHAPE, "negative size");
  if (chunk <= 0) return fail(SATTN_ERR_SHAPE, "chunk must be > 0");
  if (Hq > 0 && (Hkv <= 0 || Hq % Hkv != 0)) return fail(SATTN_ERR_SHAPE, "Hq must be a multiple of Hkv");
  int64_t qrows, kvrows, qbytes, kvbytes;
  if (!product({B, Hq, Nq}, &qrows) || !product({B, Hkv, Nk}, &kvrows) || !product({qrows, D, 2}, &qbytes) ||
      !product({kvrows, D, 2}, &kvbytes))
    return fail(SATTN_ERR_SHAPE, "size overflow");
  if (qrows == 0) return ok();
  if (Nk == 0) return fail(SATTN_ERR_SHAPE, "Nk must be > 0 (a row with no keys has no partials)");
  if (Nq >= kMaxLen || Nk >= kMaxLen || B * Hq >= kMaxLen) return fail(SATTN_ERR_UNSUPPORTED, "size too large");
  if (Nk * D * 2 >= kMaxSpan) return fail(SATTN_ERR_UNSUPPORTED, "K/V slice larger than 2 GiB");
  const int64_t C = (Nk + chunk - 1) / chunk;
  int64_t prow, mbytes, abytes;
  if (!product({qrows, C}, &prow) || !product({prow, 4}, &mbytes) || !product({prow, D, 4}, &abytes))
    return fail(SATTN_ERR_SHAPE, "size overflow");
  if (!q || !k || !v || !part_m || !part_l || !part_acc) return fail(SATTN_ERR_NULL, "null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(part_acc, 16) || !aligned(part_m, 4) ||
      !aligned(part_l, 4))
    return fail(SATTN_ERR_ALIGN, "q/k/v/part_acc need 16-byte, part_m/part_l 4-byte alignment");
  Range ins[3] = {range_of(q, qbytes, "q"), range_of(k, kvbytes, "k"), range_of(v, kvbytes, "v")};
  Range outs[3] = {range_of(part_m, mbytes, "part_m"), range_of(part_l, mbytes, "part_l"),
                   range_of(part_acc, abytes, "part_acc")};
  if ((st = check_alias(ins, 3, outs, 3))) return st;

  const int bm = tile_m<MODE_SPLIT>(D);
  // Few queries per head (decode) with grouped KV heads: one slice per
  // (batch, KV head) holding the group's rows, so each chunk of the cache is
  // read once per group instead of once per query head.
  const bool pack = Hq > Hkv && Nq <= 64;
  const int64_t slices = pack ? B * Hkv : B * Hq;
  const int64_t slice_rows = pack ? (Hq / Hkv) * Nq : Nq;
  const int64_t nqt = (slice_rows + bm - 1) / bm;
  const int64_t grid = slices * nqt * C;
  if (grid >= (int64_t(1) << 31) || C >= kMaxLen) return fail(SATTN_ERR_UNSUPPORTED, "grid too large");
  FwdParams p = blank_params(scale);
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.part_m = part_m;
  p.part_l = part_l;
  p.part_acc = part_acc;
  p.heads = (int)(B * Hq);
  p.hq = (int)Hq;
  p.hkv = (int)Hkv;
  p.n = (int)Nq;
  p.nk = (int)Nk;
  p.chunk = (int)(chunk < Nk ? chunk : Nk);  // chunk >= Nk: one chunk holds every key
  p.nchunks = (int)C;
  p.nqt = (int)nqt;
  p.off = (int)(Nk - Nq);
  p.pack = pack ? 1 : 0;
  launch_fwd_split(dtype, (int)D, causal, p, grid, (hipStream_t)stream);
  return launch_status();
}

int sattn_fwd_split(int dtype, const void* q, const void* k, const void* v, float* part_m, float* part_l,
                    float* part_acc, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                    int64_t chunk, float scale, void* stream) {
  return split_impl(dtype, q, k, v, part_m, part_l, part_acc, B, Hq, Hkv, Nq, Nk, D, chunk, false, scale, stream);
}

int sattn_fwd_split_cache(int dtype, const void* q, const void* k, const void* v, float* part_m, float* part_l,
                          float* part_acc, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                          int64_t chunk, int causal, float scale, void* stream) {
  return split_impl(dtype, q, k, v, part_m, part_l, part_acc, B, Hq, Hkv, Nq, Nk, D, chunk, causal != 0, scale,
                    stream);
}

// Window / global-token / block-mask restriction of the sparse entry point.
struct SparseSpec {
  int64_t left, right, n_global;
  const uint8_t* mask;
  int64_t mask_heads, block_q, block_k;
};

// Queries against a K/V cache with explicit element strides (batch, head,
// row) for q and for k/v; o and lse are dense [B, Hq, Nq, D] / [B, Hq, Nq].
// With a sparse spec the same walk is restricted to it (MODE_SPARSE).
static int cache_impl(int dtype, const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                      int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, const int64_t* qs,
                      const int64_t* ks, int causal, float scale, void* stream, const SparseSpec* sp = nullptr) {
  int st = check_common(dtype, D, scale);
  if (st) return st;
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0) return fail(SATTN_ERR_SHAPE, "negative size");
  if (Hq > 0 && (Hkv <= 0 || Hq % Hkv != 0)) return fail(SATTN_ERR_SHAPE, "Hq must be a multiple of Hkv");
  for (int i = 0; i < 3; ++i)
    if (qs[i] < 0 || ks[i] < 0 || qs[i] % 8 != 0 || ks[i] % 8 != 0)
      return fail(SATTN_ERR_ALIGN, "strides must be >= 0 and multiples of 8 elements (16 bytes)");
  int64_t qrows, obytes;
  if (!product({B, Hq, Nq}, &qrows) || !product({qrows, D, 2}, &obytes)) return fail(SATTN_ERR_SHAPE, "size overflow");
  if (qrows == 0) return ok();
  if (Nq >= kMaxLen || Nk >= kMaxLen || B * Hq >= kMaxLen) return fail(SATTN_ERR_UNSUPPORTED, "size too large");
  // k/v rows must not overlap: a tile's buffer range ends at its last row,
  // and reads past it return zeros
  if (Nk > 0 && ks[2] < D) return fail(SATTN_ERR_UNSUPPORTED, "k/v row stride must be >= D elements");
  // extent of a strided tensor: last element offset + 1, in elements
  int64_t qext = D, kext = 0;
  {
    int64_t a, b2, c;
    if (!product({B - 1, qs[0]}, &a) || !product({Hq - 1, qs[1]}, &b2) || !product({Nq - 1, qs[2]}, &c))
      return fail(SATTN_ERR_SHAPE, "size overflow");
    qext += a + b2 + c;
    if (Nk > 0) {
      if (!product({B - 1, ks[0]}, &a) || !product({Hkv - 1, ks[1]}, &b2) || !product({Nk - 1, ks[2]}, &c))
        return fail(SATTN_ERR_SHAPE, "size overflow");
      kext = a + b2 + c + D;
    }
    if (qext < 0 || kext < 0 || qext > (int64_t(1) << 61) || kext > (int64_t(1) << 61))
      return fail(SATTN_ERR_SHAPE, "size overflow");
  }
  if (Nk * ks[2] * 2 >= kMaxSpan) return fail(SATTN_ERR_UNSUPPORTED, "K/V slice spans 2 GiB or more");
  if (!q || !o || !lse || (kext > 0 && (!k || !v))) return fail(SATTN_ERR_NULL, "null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return fail(SATTN_ERR_ALIGN, "q/k/v/o need 16-byte and lse 4-byte alignment");
  int64_t nkb = 0, mbytes = 0;
  if (sp) {
    if (Nk > int64_t(64) * kSparseMaxTiles)
      return fail(SATTN_ERR_UNSUPPORTED, "sparse attention supports Nk <= %d", 64 * kSparseMaxTiles);
    if (sp->left < -1 || sp->right < -1 || sp->n_global < 0 || sp->left >= kMaxLen || sp->right >= kMaxLen ||
        sp->n_global >= kMaxLen)
      return fail(SATTN_ERR_VALUE, "window bounds must be >= -1 and n_global >= 0");
    if (sp->mask) {
      if (sp->block_q <= 0 || sp->block_q % 32 != 0 || sp->block_k <= 0 || sp->block_k % 64 != 0 ||
          sp->block_q >= kMaxLen || sp->block_k >= kMaxLen)
        return fail(SATTN_ERR_UNSUPPORTED, "block_q must be a positive multiple of 32 and block_k of 64");
      if (sp->mask_heads != 1 && sp->mask_heads != Hq) return fail(SATTN_ERR_SHAPE, "mask_heads must be 1 or Hq");
      const int64_t nqb = (Nq + sp->block_q - 1) / sp->block_q;
      nkb = (Nk + sp->block_k - 1) / sp->block_k;
      if (!product({sp->mask_heads, nqb, nkb}, &mbytes)) return fail(SATTN_ERR_SHAPE, "size overflow");
    }
  }
  Range ins[4] = {range_of(q, qext * 2, "q"), range_of(k, kext * 2, "k"), range_of(v, kext * 2, "v"),
                  range_of(sp ? sp->mask : nullptr, mbytes, "block_mask")};
  Range outs[2] = {range_of(o, obytes, "o"), range_of(lse, qrows * 4, "lse")};
  if ((st = check_alias(ins, 4, outs, 2))) return st;
  // causal with Nk < 2 Nq: the diagonal makes 256-row tiles uneven (9% slower
  // at Nq = Nk = 4096), so only non-causal calls and prefill-like chunks
  const bool wide = !sp && D == 128 && Nq >= kCacheWideRows && (!causal || Nk >= 2 * Nq);
  const int bm = sp ? tile_m<MODE_SPARSE>(D) : (wide ? 256 : tile_m<MODE_CACHE>(D));
  const int64_t nqt = (Nq + bm - 1) / bm;
  const int64_t grid = B * Hq * nqt;
  if (grid >= (int64_t(1) << 31)) return fail(SATTN_ERR_UNSUPPORTED, "grid too large");
  FwdParams p = blank_params(scale);
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.heads = (int)(B * Hq);
  p.hq = (int)Hq;
  p.hkv = (int)Hkv;
  p.n = (int)Nq;
  p.nk = (int)Nk;
  p.off = (int)(Nk - Nq);
  p.nqt = (int)nqt;
  p.qs_b = qs[0];
  p.qs_h = qs[1];
  p.qs_n = qs[2];
  p.ks_b = ks[0];
  p.ks_h = ks[1];
  p.ks_n = ks[2];
  if (sp) {
    p.win_left = (int)sp->left;
    p.win_right = (int)sp->right;
    p.n_global = (int)sp->n_global;
    p.bmask = sp->mask;
    p.bm_q = (int)sp->block_q;
    p.bm_k = (int)sp->block_k;
    p.bm_nkb = (int)nkb;
    p.bm_hstride = (sp->mask && sp->mask_heads > 1) ? mbytes / sp->mask_heads : 0;
    launch_fwd_sparse(dtype, (int)D, causal != 0, p, grid, (hipStream_t)stream);
  } else {
    launch_fwd_cache(dtype, (int)D, causal != 0, wide, p, grid, (hipStream_t)stream);
  }
  return launch_status();
}

int sattn_fwd_cache(int dtype, const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                    int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale,
                    void* stream) {
  if (Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || D < 0) return fail(SATTN_ERR_SHAPE, "negative size");
  int64_t qs[3], ks[3];
  if (!product({Hq, Nq, D}, &qs[0]) || !product({Hkv, Nk, D}, &ks[0])) return fail(SATTN_ERR_SHAPE, "size overflow");
  qs[1] = Nq * D;
  qs[2] = D;
  ks[1] = Nk * D;
  ks[2] = D;
  return cache_impl(dtype, q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, D, qs, ks, causal, scale, stream);
}

int sattn_fwd_sparse(int dtype, const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                     int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, int64_t win_left,
                     int64_t win_right, int64_t n_global, const uint8_t* block_mask, int64_t mask_heads,
                     int64_t block_q, int64_t block_k, float scale, void* stream) {
  if (Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || D < 0) return fail(SATTN_ERR_SHAPE, "negative size");
  int64_t qs[3], ks[3];
  if (!product({Hq, Nq, D}, &qs[0]) || !product({Hkv, Nk, D}, &ks[0])) return fail(SATTN_ERR_SHAPE, "size overflow");
  qs[1] = Nq * D;
  qs[2] = D;
  ks[1] = Nk * D;
  ks[2] = D;
  const SparseSpec sp{win_left, win_right, n_global, block_mask, mask_heads, block_q, block_k};
  return cache_impl(dtype, q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, D, qs, ks, causal, scale, stream, &sp);
}

// Backward on [B, H, N, D] slices: Nq queries at positions i + (Nk - Nq)
// against Nk keys (Nq = Nk for sattn_bwd and the sparse operator).
// With `scratch_ws`, delta is ignored and the library's static scratch
// array serves as the workspace (looked up after every check has passed).
static int bwd_impl(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, float* delta, void* dq, void* dk, void* dv, int64_t B, int64_t Hq,
                    int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale, void* stream,
                    const SparseSpec* sp = nullptr, bool scratch_ws = false) {
  int st = check_common(dtype, D, scale);
  if (st) return st;
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0) return fail(SATTN_ERR_SHAPE, "negative size");
  if (Hq > 0 && (Hkv <= 0 || Hq % Hkv != 0)) return fail(SATTN_ERR_SHAPE, "Hq must be a multiple of Hkv");
  int64_t qrows, kvrows, qbytes, kvbytes;
  if (!product({B, Hq, Nq}, &qrows) || !product({B, Hkv, Nk}, &kvrows) || !product({qrows, D, 2}, &qbytes) ||
      !product({kvrows, D, 2}, &kvbytes))
    return fail(SATTN_ERR_SHAPE, "size overflow");
  if (qrows == 0) return ok();
  if (Nq >= kMaxLen || Nk >= kMaxLen || B * Hq >= kMaxLen) return fail(SATTN_ERR_UNSUPPORTED, "size too large");
  if (Nk * D * 2 >= kMaxSpan) return fail(SATTN_ERR_UNSUPPORTED, "K/V slice larger than 2 GiB");
  // with no key at all (Nk = 0) only dq (all zero) and delta are written
  if (scratch_ws) {
    if (qrows > kScratchFloats)
      return fail(SATTN_ERR_UNSUPPORTED, "B*Hq*N = %lld query rows exceed the %lld-row static scratch of "
                  "sattn_bwd_noalloc; use sattn_bwd with a caller-owned workspace", (long long)qrows,
                  (long long)kScratchFloats);
    delta = nullptr;
  }
  if (!q || !o || !dout || !lse || (!delta && !scratch_ws) || !dq || (kvrows > 0 && (!k || !v || !dk || !dv)))
    return fail(SATTN_ERR_NULL, "null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(delta, 4))
    return fail(SATTN_ERR_ALIGN, "16-bit tensors need 16-byte, lse/delta 4-byte alignment");
  int64_t nkb = 0, mbytes = 0;
  if (sp) {
    if (sp->left < -1 || sp->right < -1 || sp->n_global < 0 || sp->left >= kMaxLen || sp->right >= kMaxLen ||
        sp->n_global >= kMaxLen)
      return fail(SATTN_ERR_VALUE, "window bounds must be >= -1 and n_global >= 0");
    if (sp->mask) {
      if (sp->block_q <= 0 || sp->block_q % 32 != 0 || sp->block_k <= 0 || sp->block_k % 64 != 0 ||
          sp->block_q >= kMaxLen || sp->block_k >= kMaxLen)
        return fail(SATTN_ERR_UNSUPPORTED, "block_q must be a positive multiple of 32 and block_k of 64");
      if (sp->mask_heads != 1 && sp->mask_heads != Hq) return fail(SATTN_ERR_SHAPE, "mask_heads must be 1 or Hq");
      const int64_t nqb = (Nq + sp->block_q - 1) / sp->block_q;
      nkb = (Nk + sp->block_k - 1) / sp->block_k;
      if (!product({sp->mask_heads, nqb, nkb}, &mbytes)) return fail(SATTN_ERR_SHAPE, "size overflow");
    }
  }
  Range ins[7] = {range_of(q, qbytes, "q"),       range_of(k, kvbytes, "k"),          range_of(v, kvbytes, "v"),
                  range_of(o, qbytes, "o"),       range_of(dout, qbytes, "dout"),     range_of(lse, qrows * 4, "lse"),
                  range_of(sp ? sp->mask : nullptr, mbytes, "block_mask")};
  Range outs[4] = {range_of(dq, qbytes, "dq"), range_of(dk, kvbytes, "dk"), range_of(dv, kvbytes, "dv"),
                   range_of(delta, scratch_ws ? 0 : qrows * 4, "delta")};
  if ((st = check_alias(ins, 7, outs, 4))) return st;
  if (scratch_ws && (st = scratch_on_current_device(&delta))) return st;
  BwdParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (const uint16_t*)o;
  p.dout = (const uint16_t*)dout;
  p.lse = lse;
  p.delta = delta;
  p.dq = (uint16_t*)dq;
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.hq = (int)Hq;
  p.hkv = (int)Hkv;
  p.n = (int)Nq;
  p.nk = (int)Nk;
  p.off = (int)(Nk - Nq);
  const int64_t bmq = 32 * bwd_dq_waves((int)D, causal != 0, sp ? BWD_SPARSE : BWD_DENSE);
  p.nqt = (int)((Nq + bmq - 1) / bmq);
  p.nkt = (int)((Nk + 127) / 128);
  p.c = scale * kLog2e;
  p.scale = scale;
  // dQ: BM = bmq rows per workgroup; batched causal grids of at least 1024
  // query tiles pair them (tiles nqt-1-j and j per workgroup)
  p.pair = (!sp && causal && bmq == 256 && B * Hq * p.nqt >= 1024) ? 1 : 0;
  // dK/dV at D = 128 (two roles, one workgroup per CU): batched causal grids
  // of at least 1024 key tiles pair them too (tiles j and nkt-1-j per
  // workgroup). At D = 64 two workgroups share a CU and pairing was slower.
  p.pair_kv = (!sp && causal && D == 128 && B * Hkv * p.nkt >= 1024) ? 1 : 0;
  const int64_t grid_q = B * Hq * (p.pair ? (p.nqt + 1) / 2 : p.nqt);
  const int64_t grid_kv = B * Hkv * (p.pair_kv ? (p.nkt + 1) / 2 : p.nkt);
  if (grid_q >= (int64_t(1) << 31)) return fail(SATTN_ERR_UNSUPPORTED, "grid too large");
  if (sp) {
    p.win_left = (int)sp->left;
    p.win_right = (int)sp->right;
    p.n_global = (int)sp->n_global;
    p.bmask = sp->mask;
    p.bm_q = (int)sp->block_q;
    p.bm_k = (int)sp->block_k;
    p.bm_nkb = (int)nkb;
    p.bm_hstride = (sp->mask && sp->mask_heads > 1) ? mbytes / sp->mask_heads : 0;
    launch_bwd_sparse(dtype, (int)D, causal != 0, p, grid_q, grid_kv, (hipStream_t)stream);
  } else {
    launch_bwd_dense(dtype, (int)D, causal != 0, p, grid_q, grid_kv, (hipStream_t)stream);
  }
  return launch_status();
}

int sattn_bwd(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, float* delta, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
              int64_t N, int64_t D, int causal, float scale, void* stream) {
  return bwd_impl(dtype, q, k, v, o, dout, lse, delta, dq, dk, dv, B, Hq, Hkv, N, N, D, causal, scale, stream);
}

int sattn_bwd_noalloc(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                      int64_t D, int causal, float scale, void* stream) {
  return bwd_impl(dtype, q, k, v, o, dout, lse, nullptr, dq, dk, dv, B, Hq, Hkv, N, N, D, causal, scale, stream,
                  nullptr, true);
}

int sattn_bwd_cache(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, float* delta, void* dq, void* dk, void* dv, int64_t B, int64_t Hq,
                    int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale, void* stream) {
  return bwd_impl(dtype, q, k, v, o, dout, lse, delta, dq, dk, dv, B, Hq, Hkv, Nq, Nk, D, causal, scale, stream);
}

int sattn_bwd_sparse(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, float* delta, void* dq, void* dk, void* dv, int64_t B, int64_t Hq,
                     int64_t Hkv, int64_t N, int64_t D, int causal, int64_t win_left, int64_t win_right,
                     int64_t n_global, const uint8_t* block_mask, int64_t mask_heads, int64_t block_q,
                     int64_t block_k, float scale, void* stream) {
  const SparseSpec sp{win_left, win_right, n_global, block_mask, mask_heads, block_q, block_k};
  return bwd_impl(dtype, q, k, v, o, dout, lse, delta, dq, dk, dv, B, Hq, Hkv, N, N, D, causal, scale, stream, &sp);
}

int sattn_bwd_varlen(int dtype, const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, float* delta, void* dq, void* dk, void* dv, const int32_t* cu_seqlens,
                     int64_t S, int64_t T, int64_t max_seqlen, int64_t Hq, int64_t Hkv, int64_t D, int causal,
                     float scale, void* stream) {
  int st = check_common(dtype, D, scale);
  if (st) return st;
  if (S < 0 || T < 0 || max_seqlen < 0 || Hq < 0 || Hkv < 0) return fail(SATTN_ERR_SHAPE, "negative size");
  if (Hq > 0 && (Hkv <= 0 || Hq % Hkv != 0)) return fail(SATTN_ERR_SHAPE, "Hq must be a multiple of Hkv");
  int64_t qbytes, kvbytes, lbytes;
  if (!product({T, Hq, D, 2}, &qbytes) || !product({T, Hkv, D, 2}, &kvbytes) || !product({Hq, T, 4}, &lbytes))
    return fail(SATTN_ERR_SHAPE, "size overflow");
  if (S == 0 || T == 0 || Hq == 0 || max_seqlen == 0) return ok();
  if (T >= kMaxLen || S >= kMaxLen || Hq >= 65536 || max_seqlen > T)
    return fail(max_seqlen > T ? SATTN_ERR_SHAPE : SATTN_ERR_UNSUPPORTED, "max_seqlen > T or size too large");
  if (max_seqlen * Hkv * D * 2 >= kMaxSpan || 64 * Hq * D * 2 >= kMaxSpan)
    return fail(SATTN_ERR_UNSUPPORTED, "a sequence's K/V span exceeds 2 GiB");
  if (!q || !k || !v || !o || !dout || !lse || !delta || !dq || !dk || !dv || !cu_seqlens)
    return fail(SATTN_ERR_NULL, "null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(delta, 4) ||
      !aligned(cu_seqlens, 4))
    return fail(SATTN_ERR_ALIGN, "16-bit tensors need 16-byte, lse/delta/cu_seqlens 4-byte alignment");
  Range ins[7] = {range_of(q, qbytes, "q"),       range_of(k, kvbytes, "k"),        range_of(v, kvbytes, "v"),
                  range_of(o, qbytes, "o"),       range_of(dout, qbytes, "dout"),   range_of(lse, lbytes, "lse"),
                  range_of(cu_seqlens, (S + 1) * 4, "cu_seqlens")};
  Range outs[4] = {range_of(dq, qbytes, "dq"), range_of(dk, kvbytes, "dk"), range_of(dv, kvbytes, "dv"),
                   range_of(delta, lbytes, "delta")};
  if ((st = check_alias(ins, 7, outs, 4))) return st;
  const int64_t ntile = (max_seqlen + 127) / 128;
  int64_t grid_q, grid_kv;
  if (!product({S, ntile, Hq}, &grid_q) || !product({S, ntile, Hkv}, &grid_kv) || grid_q >= (int64_t(1) << 31))
    return fail(SATTN_ERR_UNSUPPORTED, "grid too large");
  BwdParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (const uint16_t*)o;
  p.dout = (const uint16_t*)dout;
  p.lse = lse;
  p.delta = delta;
  p.dq = (uint16_t*)dq;
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.hq = (int)Hq;
  p.hkv = (int)Hkv;
  p.nqt = (int)ntile;
  p.nkt = (int)ntile;
  p.cu_seqlens = cu_seqlens;
  p.nseq = (int)S;
  p.total = (int)T;
  p.c = scale * kLog2e;
  p.scale = scale;
  launch_bwd_varlen(dtype, (int)D, causal != 0, p, grid_q, grid_kv, (hipStream_t)stream);
  return launch_status();
}

int sattn_fwd_strided(int dtype, const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                      int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, const int64_t* q_strides,
                      const int64_t* kv_strides, int causal, float scale, void* stream) {
  if (!q_strides || !kv_strides) return fail(SATTN_ERR_NULL, "null stride array");
  return cache_impl(dtype, q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, D, q_strides, kv_strides, causal, scale, stream);
}

int sattn_merge(int dtype, const float* part_m, const float* part_l, const float* part_acc, int64_t rows, int64_t C,
                int64_t D, void* o, float* lse, void* stream) {
  int st = check_common(dtype, D, 1.0f);
  if (st) return st;
  if (rows < 0 || C < 0) return fail(SATTN_ERR_SHAPE, "negative size");
  if (rows == 0) return ok();
  if (C == 0) return fail(SATTN_ERR_SHAPE, "C must be > 0");
  int64_t prow, mbytes, abytes, obytes;
  if (!product({rows, C}, &prow) || !product({prow, 4}, &mbytes) || !product({prow, D, 4}, &abytes) ||
      !product({rows, D, 2}, &obytes))
    return fail(SATTN_ERR_SHAPE, "size overflow");
  if (C >= kMaxLen) return fail(SATTN_ERR_UNSUPPORTED, "C too large");
  if (!part_m || !part_l || !part_acc || !o || !lse) return fail(SATTN_ERR_NULL, "null pointer");
  if (!aligned(part_m, 4) || !aligned(part_l, 4) || !aligned(part_acc, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return fail(SATTN_ERR_ALIGN, "misaligned pointer");
  Range ins[3] = {range_of(part_m, mbytes, "part_m"), range_of(part_l, mbytes, "part_l"),
                  range_of(part_acc, abytes, "part_acc")};
  Range outs[2] = {range_of(o, obytes, "o"), range_of(lse, rows * 4, "lse")};
  if ((st = check_alias(ins, 3, outs, 2))) return st;
  if (rows >= (int64_t(1) << 31)) return fail(SATTN_ERR_UNSUPPORTED, "grid too large");  // one workgroup per row
  launch_merge(dtype, (int)D, part_m, part_l, part_acc, rows, (int)C, (uint16_t*)o, lse, (hipStream_t)stream);
  return launch_status();
}

int sattn_fwd_varlen(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                     const int32_t* cu_seqlens, int64_t S, int64_t T, int64_t max_seqlen, int64_t Hq, int64_t Hkv,
                     int64_t D, int causal, float scale, void* stream) {
  int st = check_common(dtype, D, scale);
  if (st) return st;
  if (S < 0 || T < 0 || max_seqlen < 0 || Hq < 0 || Hkv < 0) return fail(SATTN_ERR_SHAPE, "negative size");
  if (Hq > 0 && (Hkv <= 0 || Hq % Hkv != 0)) return fail(SATTN_ERR_SHAPE, "Hq must be a multiple of Hkv");
  int64_t qbytes, kvbytes, lbytes;
  if (!product({T, Hq, D, 2}, &qbytes) || !product({T, Hkv, D, 2}, &kvbytes) || !product({Hq, T, 4}, &lbytes))
    return fail(SATTN_ERR_SHAPE, "size overflow");
  if (S == 0 || T == 0 || Hq == 0 || max_seqlen == 0) return ok();
  if (T >= kMaxLen || S >= kMaxLen || Hq >= 65536 || max_seqlen > T)
    return fail(max_seqlen > T ? SATTN_ERR_SHAPE : SATTN_ERR_UNSUPPORTED, "max_seqlen > T or size too large");
  if (max_seqlen * Hkv * D * 2 >= kMaxSpan) return fail(SATTN_ERR_UNSUPPORTED, "a sequence's K/V span exceeds 2 GiB");
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return fail(SATTN_ERR_NULL, "null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(cu_seqlens, 4))
    return fail(SATTN_ERR_ALIGN, "misaligned pointer");
  Range ins[4] = {range_of(q, qbytes, "q"), range_of(k, kvbytes, "k"), range_of(v, kvbytes, "v"),
                  range_of(cu_seqlens, (S + 1) * 4, "cu_seqlens")};
  Range outs[2] = {range_of(o, qbytes, "o"), range_of(lse, lbytes, "lse")};
  if ((st = check_alias(ins, 4, outs, 2))) return st;
  const int bm = tile_m<MODE_VARLEN>(D);
  const int64_t nqt = (max_seqlen + bm - 1) / bm;
  int64_t grid;
  if (!product({nqt, S, Hq}, &grid) || grid >= (int64_t(1) << 31))
    return fail(SATTN_ERR_UNSUPPORTED, "grid too large");
  FwdParams p = blank_params(scale);
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.hq = (int)Hq;
  p.hkv = (int)Hkv;
  p.nqt = (int)nqt;
  p.nseq = (int)S;
  p.total = (int)T;
  launch_fwd_varlen(dtype, (int)D, causal != 0, p, grid, (hipStream_t)stream);
  return launch_status();
}

}  // extern "C"

// Host-side launchers of the sattn kernels. Each kernel family is compiled in
// its own translation unit (k_*.hip), which instantiates and launches its
// kernels; the C ABI layer (sattn.hip) validates arguments, fills the
// parameter blocks and calls these. All launches go to the caller's stream.
#pragma once

#include "fwd_kernel.hpp"
#include "bwd_kernel.hpp"

namespace sattn {

// Query rows per workgroup (32 per wave) of the streaming forward kernel.
// Dense D = 128 runs 8 waves (256 query rows) per workgroup, one workgroup
// per CU: each K/V tile staged in LDS then serves twice as many queries as
// with 4 waves, and every SIMD still holds two waves. Varlen, split, cache
// and sparse keep 4 waves, whose 128-row granularity wastes fewer rows on
// short sequences and few queries. D = 32 and 64 use 2 waves.
template <int D, int MODE>
struct Tile {
  static constexpr int NW = D == 128 ? (MODE == MODE_DENSE ? 8 : 4) : 2;
  static constexpr int BM = NW * 32;
};

// Keys per tile of the dense streaming kernel (a build-time knob for the
// design-variant builds; the library uses 64).
#ifndef SATTN_DENSE_BN
#define SATTN_DENSE_BN 64
#endif
constexpr int kDenseBN = SATTN_DENSE_BN;

// Cache mode at D = 128 runs 8 waves (256 rows) per workgroup for calls with
// at least this many queries (non-causal, or causal prefill-like chunks).
constexpr int kCacheWideRows = 512;

// Waves of the backward dQ kernel: 8 (256 queries per workgroup) for the
// batched layout at D = 128 (causal grids of enough tiles then pair their
// query tiles, as the forward does), else 4.
constexpr int bwd_dq_waves(int D, bool /* causal: the same either way */, int layout) {
  return (D == 128 && layout == BWD_DENSE) ? 8 : 4;
}

// Whether dK/dV runs in two roles per SIMD (8 waves) rather than one wave
// per 32 keys (4 waves): at D = 128, and causal at D = 64 (non-causal D = 64
// measured 1.4% slower in two roles, causal 7.9% faster).
constexpr bool bwd_dkdv_roles(int D, bool causal) { return D == 128 || (D == 64 && causal); }

template <class E, int D, bool CAUSAL, int LAYOUT>
inline void launch_dkdv(const BwdParams& p, int64_t grid_kv, hipStream_t s) {
  if constexpr (bwd_dkdv_roles(D, CAUSAL))
    hipLaunchKernelGGL((bwd_dkdv_roles_kernel<E, D, CAUSAL, LAYOUT>), dim3((unsigned)grid_kv), dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, CAUSAL, LAYOUT>), dim3((unsigned)grid_kv), dim3(256), 0, s, p);
}

// dtype: 0 = fp16, 1 = bf16 (the C ABI's sattn_dtype_t). D in {32, 64, 128}.
void launch_fwd_dense(int dtype, int D, bool causal, const FwdParams& p, int64_t grid, hipStream_t s);
// Small D <= 64 problems: `wide` selects 8 waves per workgroup, else 4.
void launch_fwd_small(int dtype, int D, bool causal, bool wide, const FwdParams& p, int64_t grid, hipStream_t s);
void launch_fwd_varlen(int dtype, int D, bool causal, const FwdParams& p, int64_t grid, hipStream_t s);
void launch_fwd_split(int dtype, int D, bool causal, const FwdParams& p, int64_t grid, hipStream_t s);
void launch_merge(int dtype, int D, const float* pm, const float* pl, const float* pacc, int64_t rows, int nchunks,
                  uint16_t* o, float* lse, hipStream_t s);
// `wide`: 8 waves (256 query rows) per workgroup at D = 128.
void launch_fwd_cache(int dtype, int D, bool causal, bool wide, const FwdParams& p, int64_t grid, hipStream_t s);
void launch_fwd_sparse(int dtype, int D, bool causal, const FwdParams& p, int64_t grid, hipStream_t s);
// Backward, one launcher per row layout: the dQ launch (which also writes
// Delta), then dK/dV when grid_kv > 0.
void launch_bwd_dense(int dtype, int D, bool causal, const BwdParams& p, int64_t grid_q, int64_t grid_kv,
                      hipStream_t s);
void launch_bwd_varlen(int dtype, int D, bool causal, const BwdParams& p, int64_t grid_q, int64_t grid_kv,
                       hipStream_t s);
void launch_bwd_sparse(int dtype, int D, bool causal, const BwdParams& p, int64_t grid_q, int64_t grid_kv,
                       hipStream_t s);

}  // namespace sattn

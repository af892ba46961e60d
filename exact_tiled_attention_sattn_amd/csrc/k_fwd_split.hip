// Split-KV partial states (optionally causal, cache alignment) and their merge.
#include "launch.hpp"
#include "fwd_decode.hpp"

namespace sattn {

namespace {
template <class E, int D, bool CAUSAL>
void go(const FwdParams& p, int64_t grid, hipStream_t s) {
  if (p.n == 1 && !p.pack) {   // one row per slice: the grid is (row, chunk) already
    hipLaunchKernelGGL((split_row_kernel<E, D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return;
  }
  constexpr int NW = Tile<D, MODE_SPLIT>::NW;
  hipLaunchKernelGGL((fwd_kernel<E, D, 64, NW, CAUSAL, MODE_SPLIT>), dim3((unsigned)grid), dim3(NW * 64), 0, s, p);
}
template <class E, int D>
void go_merge(const float* pm, const float* pl, const float* pacc, int64_t rows, int nchunks, uint16_t* o, float* lse,
              hipStream_t s) {
  hipLaunchKernelGGL((merge_kernel<E, D>), dim3((unsigned)rows), dim3(64), 0, s, pm, pl, pacc, rows, nchunks, o, lse);
}
}  // namespace

void launch_fwd_split(int dtype, int D, bool causal, const FwdParams& p, int64_t grid, hipStream_t s) {
#define SATTN_GO(E_, D_) \
  if (causal) go<E_, D_, true>(p, grid, s); else go<E_, D_, false>(p, grid, s);
  if (dtype == 1) {
    if (D == 32) { SATTN_GO(Bf16, 32) } else if (D == 64) { SATTN_GO(Bf16, 64) } else { SATTN_GO(Bf16, 128) }
  } else {
    if (D == 32) { SATTN_GO(F16, 32) } else if (D == 64) { SATTN_GO(F16, 64) } else { SATTN_GO(F16, 128) }
  }
#undef SATTN_GO
}

void launch_merge(int dtype, int D, const float* pm, const float* pl, const float* pacc, int64_t rows, int nchunks,
                  uint16_t* o, float* lse, hipStream_t s) {
  if (dtype == 1) {
    if (D == 32) go_merge<Bf16, 32>(pm, pl, pacc, rows, nchunks, o, lse, s);
    else if (D == 64) go_merge<Bf16, 64>(pm, pl, pacc, rows, nchunks, o, lse, s);
    else go_merge<Bf16, 128>(pm, pl, pacc, rows, nchunks, o, lse, s);
  } else {
    if (D == 32) go_merge<F16, 32>(pm, pl, pacc, rows, nchunks, o, lse, s);
    else if (D == 64) go_merge<F16, 64>(pm, pl, pacc, rows, nchunks, o, lse, s);
    else go_merge<F16, 128>(pm, pl, pacc, rows, nchunks, o, lse, s);
  }
}

}  // namespace sattn

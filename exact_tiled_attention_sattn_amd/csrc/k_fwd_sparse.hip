// Sliding-window / global-token / block-mask forward (cache layout).
#include "launch.hpp"

namespace sattn {

namespace {
template <class E, int D, bool CAUSAL>
void go(const FwdParams& p, int64_t grid, hipStream_t s) {
  constexpr int NW = Tile<D, MODE_SPARSE>::NW;
  hipLaunchKernelGGL((fwd_kernel<E, D, 64, NW, CAUSAL, MODE_SPARSE>), dim3((unsigned)grid), dim3(NW * 64), 0, s, p);
}
}  // namespace

void launch_fwd_sparse(int dtype, int D, bool causal, const FwdParams& p, int64_t grid, hipStream_t s) {
#define SATTN_GO(E_, D_) \
  if (causal) go<E_, D_, true>(p, grid, s); else go<E_, D_, false>(p, grid, s);
  if (dtype == 1) {
    if (D == 32) { SATTN_GO(Bf16, 32) } else if (D == 64) { SATTN_GO(Bf16, 64) } else { SATTN_GO(Bf16, 128) }
  } else {
    if (D == 32) { SATTN_GO(F16, 32) } else if (D == 64) { SATTN_GO(F16, 64) } else { SATTN_GO(F16, 128) }
  }
#undef SATTN_GO
}

}  // namespace sattn

// Dense [B, H, N, D] forward: the streaming kernel in MODE_DENSE and the
// small-problem kernel (D <= 64, few query tiles).
#include "launch.hpp"
#include "fwd_small.hpp"

namespace sattn {

namespace {
template <class E, int D, bool CAUSAL>
void go(const FwdParams& p, int64_t grid, hipStream_t s) {
  constexpr int NW = Tile<D, MODE_DENSE>::NW;
  hipLaunchKernelGGL((fwd_kernel<E, D, kDenseBN, NW, CAUSAL, MODE_DENSE>), dim3((unsigned)grid), dim3(NW * 64), 0,
                     s, p);
}
template <class E, int D>
void go_small(bool causal, bool wide, const FwdParams& p, int64_t grid, hipStream_t s) {
  const dim3 g((unsigned)grid);
  if (wide) {
    if (causal) hipLaunchKernelGGL((fwd_small_kernel<E, D, 8, true>), g, dim3(512), 0, s, p);
    else hipLaunchKernelGGL((fwd_small_kernel<E, D, 8, false>), g, dim3(512), 0, s, p);
  } else {
    if (causal) hipLaunchKernelGGL((fwd_small_kernel<E, D, 4, true>), g, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((fwd_small_kernel<E, D, 4, false>), g, dim3(256), 0, s, p);
  }
}
}  // namespace

void launch_fwd_dense(int dtype, int D, bool causal, const FwdParams& p, int64_t grid, hipStream_t s) {
#define SATTN_GO(E_, D_) \
  if (causal) go<E_, D_, true>(p, grid, s); else go<E_, D_, false>(p, grid, s);
  if (dtype == 1) {
    if (D == 32) { SATTN_GO(Bf16, 32) } else if (D == 64) { SATTN_GO(Bf16, 64) } else { SATTN_GO(Bf16, 128) }
  } else {
    if (D == 32) { SATTN_GO(F16, 32) } else if (D == 64) { SATTN_GO(F16, 64) } else { SATTN_GO(F16, 128) }
  }
#undef SATTN_GO
}

void launch_fwd_small(int dtype, int D, bool causal, bool wide, const FwdParams& p, int64_t grid, hipStream_t s) {
  if (dtype == 1) {
    if (D == 32) go_small<Bf16, 32>(causal, wide, p, grid, s);
    else go_small<Bf16, 64>(causal, wide, p, grid, s);
  } else {
    if (D == 32) go_small<F16, 32>(causal, wide, p, grid, s);
    else go_small<F16, 64>(causal, wide, p, grid, s);
  }
}

}  // namespace sattn

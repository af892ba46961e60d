// Queries against a K/V cache (bottom-right causal alignment, grouped KV
// heads, element strides): 4-wave tiles, or 8-wave tiles for long chunks.
#include "launch.hpp"

namespace sattn {

namespace {
template <class E, int D, int NW, bool CAUSAL>
void go(const FwdParams& p, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((fwd_kernel<E, D, 64, NW, CAUSAL, MODE_CACHE>), dim3((unsigned)grid), dim3(NW * 64), 0, s, p);
}
}  // namespace

void launch_fwd_cache(int dtype, int D, bool causal, bool wide, const FwdParams& p, int64_t grid, hipStream_t s) {
#define SATTN_GO(E_, D_) \
  if (causal) go<E_, D_, Tile<D_, MODE_CACHE>::NW, true>(p, grid, s); \
  else go<E_, D_, Tile<D_, MODE_CACHE>::NW, false>(p, grid, s);
  if (wide && D == 128) {
    if (dtype == 1) {
      if (causal) go<Bf16, 128, 8, true>(p, grid, s); else go<Bf16, 128, 8, false>(p, grid, s);
    } else {
      if (causal) go<F16, 128, 8, true>(p, grid, s); else go<F16, 128, 8, false>(p, grid, s);
    }
    return;
  }
  if (dtype == 1) {
    if (D == 32) { SATTN_GO(Bf16, 32) } else if (D == 64) { SATTN_GO(Bf16, 64) } else { SATTN_GO(Bf16, 128) }
  } else {
    if (D == 32) { SATTN_GO(F16, 32) } else if (D == 64) { SATTN_GO(F16, 64) } else { SATTN_GO(F16, 128) }
  }
#undef SATTN_GO
}

}  // namespace sattn

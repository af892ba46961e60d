// Backward kernels (dQ with Delta, then dK/dV) in the BWD_VARLEN row layout.
#include "launch.hpp"

namespace sattn {

namespace {
template <class E, int D>
void go(bool causal, const BwdParams& p, int64_t grid_q, int64_t grid_kv, hipStream_t s) {
  if (causal) {
    constexpr int NWQ = bwd_dq_waves(D, true, BWD_VARLEN);
    hipLaunchKernelGGL((bwd_dq_kernel<E, D, true, BWD_VARLEN, NWQ>), dim3((unsigned)grid_q), dim3(NWQ * 64), 0, s, p);
    if (grid_kv > 0)
      launch_dkdv<E, D, true, BWD_VARLEN>(p, grid_kv, s);
  } else {
    constexpr int NWQ = bwd_dq_waves(D, false, BWD_VARLEN);
    hipLaunchKernelGGL((bwd_dq_kernel<E, D, false, BWD_VARLEN, NWQ>), dim3((unsigned)grid_q), dim3(NWQ * 64), 0, s, p);
    if (grid_kv > 0)
      launch_dkdv<E, D, false, BWD_VARLEN>(p, grid_kv, s);
  }
}
}  // namespace

// Explicit instantiations, so that every kernel of this layout has its
// device code and host stub in this object: dQ for every D; dK/dV in two
// roles where bwd_dkdv_roles says so, else one wave per key block.
#define SATTN_INST(E_, D_)                                                                      \
  template __global__ void bwd_dq_kernel<E_, D_, true, BWD_VARLEN, bwd_dq_waves(D_, true, BWD_VARLEN)>(const BwdParams);  \
  template __global__ void bwd_dq_kernel<E_, D_, false, BWD_VARLEN, bwd_dq_waves(D_, false, BWD_VARLEN)>(const BwdParams);
#define SATTN_INST_KV(E_, D_)                                                         \
  template __global__ void bwd_dkdv_kernel<E_, D_, true, BWD_VARLEN>(const BwdParams);  \
  template __global__ void bwd_dkdv_kernel<E_, D_, false, BWD_VARLEN>(const BwdParams);
#define SATTN_INST_KV2(E_, D_)                                                                 \
  template __global__ void bwd_dkdv_roles_kernel<E_, D_, true, BWD_VARLEN>(const BwdParams);  \
  template __global__ void bwd_dkdv_roles_kernel<E_, D_, false, BWD_VARLEN>(const BwdParams);
SATTN_INST(Bf16, 32) SATTN_INST(Bf16, 64) SATTN_INST(Bf16, 128)
SATTN_INST(F16, 32) SATTN_INST(F16, 64) SATTN_INST(F16, 128)
SATTN_INST_KV(Bf16, 32) SATTN_INST_KV(F16, 32) SATTN_INST_KV2(Bf16, 128) SATTN_INST_KV2(F16, 128)
template __global__ void bwd_dkdv_kernel<Bf16, 64, false, BWD_VARLEN>(const BwdParams);
template __global__ void bwd_dkdv_kernel<F16, 64, false, BWD_VARLEN>(const BwdParams);
template __global__ void bwd_dkdv_roles_kernel<Bf16, 64, true, BWD_VARLEN>(const BwdParams);
template __global__ void bwd_dkdv_roles_kernel<F16, 64, true, BWD_VARLEN>(const BwdParams);
#undef SATTN_INST
#undef SATTN_INST_KV
#undef SATTN_INST_KV2

void launch_bwd_varlen(int dtype, int D, bool causal, const BwdParams& p, int64_t grid_q, int64_t grid_kv,
                   hipStream_t s) {
  if (dtype == 1) {
    if (D == 32) go<Bf16, 32>(causal, p, grid_q, grid_kv, s);
    else if (D == 64) go<Bf16, 64>(causal, p, grid_q, grid_kv, s);
    else go<Bf16, 128>(causal, p, grid_q, grid_kv, s);
  } else {
    if (D == 32) go<F16, 32>(causal, p, grid_q, grid_kv, s);
    else if (D == 64) go<F16, 64>(causal, p, grid_q, grid_kv, s);
    else go<F16, 128>(causal, p, grid_q, grid_kv, s);
  }
}

}  // namespace sattn

// A plain streaming read of a device buffer (the bandwidth ceiling that the
// split-KV decode is compared against); see include/sattn_probe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sattn_probe.h"

namespace {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                   uint32_t* __restrict__ out) {
  constexpr int U = 8;   // 16-byte loads in flight per thread
  // each workgroup streams one contiguous slice of the buffer, U x 4 KiB at a time
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t begin = (int64_t)blockIdx.x * per;
  const int64_t end = begin + per < n16 ? begin + per : n16;
  int64_t i = begin + threadIdx.x;
  u32x4 x = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * 256 < end; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u];
  }
  for (; i < end; i += 256) x ^= __builtin_nontemporal_load(buf + i);
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}
}  // namespace

extern "C" int sattn_probe_read(const void* buf, int64_t bytes, uint32_t* out, int64_t out_count, int grid,
                                void* stream) {
  if (!buf || !out || bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0 || ((uintptr_t)out & 3) != 0 ||
      grid <= 0 || grid > 65536 || out_count < (int64_t)grid * 256)
    return -1;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(buf), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

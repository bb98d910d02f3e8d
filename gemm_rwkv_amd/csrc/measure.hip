// Measurement aid: a read-only stream over device memory, the ceiling that
// the weight-streaming products are compared with.  Every thread issues
// eight 16-byte non-temporal loads per step (grid-stride, 256 threads per
// workgroup) and folds them into one word, which is stored only if it equals
// a fixed value (so the loads cannot be dropped and nothing else is written).
#include "device_common.h"
#include "kernels.h"

namespace rq {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* sink) {
  constexpr int U = 8;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x;
  for (; i + (size_t)(U - 1) * 256 < n16; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + (size_t)u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  // the tail (fewer than 256 * U vectors past the last full step)
  for (; i < n16; i += 256) acc ^= __builtin_nontemporal_load(p + i)[0];
  if (acc == 0x9e3779b9u) *sink = acc;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  // at most 8192 workgroups (32 per compute unit), one step each where possible
  size_t blocks = (n16 + 256 * 8 - 1) / (256 * 8);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const u32x4*)buf, n16, sink);
  return hipGetLastError();
}

}  // namespace rq

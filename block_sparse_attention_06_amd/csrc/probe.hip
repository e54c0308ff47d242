// Measurement aid (not part of the QSA computation): the memory-system ceiling that
// the kept-token gather of the attention stage runs against. Each wave reads, per
// step, four 4 KiB blocks whose indices come from `block_ids` (random for a gather,
// consecutive for a stream) -- the access pattern of one 16-key step of the
// attention kernel -- and folds the data into a value that is never used, so the
// loads cannot be dropped.

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

__global__ __launch_bounds__(256) void probe_gather_kernel(const uint4* __restrict__ buf,
                                                           const int32_t* __restrict__ ids,
                                                           int steps, int64_t n_waves,
                                                           uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= n_waves) return;
  uint32_t acc = 0;
  const int32_t* my = ids + wave * (int64_t)steps * 4;
  for (int s = 0; s < steps; ++s) {
    uint4 v[16];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint4* p = buf + (int64_t)my[s * 4 + b] * 256;  // 4 KiB = 256 x 16 B
#pragma unroll
      for (int k = 0; k < 4; ++k) v[b * 4 + k] = p[lane + k * 64];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  if (acc == 0x9e3779b9u) sink[wave & 1023] = acc;  // practically never taken
}

hipError_t launch_probe_gather(const void* buf, const int32_t* ids, int steps, int64_t n_waves,
                               uint32_t* sink, hipStream_t stream) {
  if (n_waves <= 0 || steps <= 0) return hipSuccess;
  hipLaunchKernelGGL(probe_gather_kernel, dim3((unsigned)((n_waves + 3) / 4)), dim3(256), 0,
                     stream, static_cast<const uint4*>(buf), ids, steps, n_waves, sink);
  return hipGetLastError();
}

}  // namespace qsa

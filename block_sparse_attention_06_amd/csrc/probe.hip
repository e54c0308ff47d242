// Measurement aids, built as their own library (libqsa_probe.so), not part of the QSA
// computation or of libqsa.so.
// - Gather: the memory-system ceiling that the kept-token gather of the attention
//   stage runs against. Each wave reads, per step, four 4 KiB blocks whose indices
//   come from `block_ids` (random for a gather, consecutive for a stream) -- the access
//   pattern of one 16-key step of the attention kernel -- and folds the data into a
//   value that is never used, so the loads cannot be dropped.
// - Write stream: the ceiling of the score GEMM's output stream. Each lane writes
//   16-byte values, a wave 1 KiB of consecutive bytes per instruction, as the GEMM's
//   epilogue writes its rows of scores; optionally with the non-temporal hint.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "qsa_probe.h"

namespace {

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

typedef float probe_f4 __attribute__((ext_vector_type(4)));

template <bool NT>
__global__ __launch_bounds__(256) void probe_write_kernel(probe_f4* __restrict__ buf, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const float x = (float)(i & 0xffffff);
    const probe_f4 v = {x, x + 1.f, x + 2.f, x + 3.f};
    if (NT)
      __builtin_nontemporal_store(v, buf + i);
    else
      buf[i] = v;
  }
}

}  // namespace

extern "C" int qsa_probe_write(void* buf, size_t bytes, int nontemporal, void* stream) {
  if (!buf || (reinterpret_cast<uintptr_t>(buf) & 15) || (bytes & 15)) return 1;
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return 0;
  // Enough workgroups to fill the device several times over, each lane looping.
  const int64_t groups = (n16 + 255) / 256;
  const unsigned grid = (unsigned)(groups < 8192 ? groups : 8192);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(probe_write_kernel<true>, dim3(grid), dim3(256), 0, s,
                       static_cast<probe_f4*>(buf), n16);
  else
    hipLaunchKernelGGL(probe_write_kernel<false>, dim3(grid), dim3(256), 0, s,
                       static_cast<probe_f4*>(buf), n16);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int qsa_probe_gather(const void* buf, size_t buf_bytes, const int32_t* block_ids,
                                int64_t n_waves, int steps, uint32_t* sink, void* stream) {
  if (!buf || !block_ids || !sink) return 1;
  if ((reinterpret_cast<uintptr_t>(buf) & 15) || buf_bytes < 4096) return 1;
  if (n_waves < 0 || steps < 0 || n_waves / 4 >= ((int64_t)1 << 31)) return 1;
  if (n_waves == 0 || steps == 0) return 0;
  hipLaunchKernelGGL(probe_gather_kernel, dim3((unsigned)((n_waves + 3) / 4)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), block_ids,
                     steps, n_waves, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// Wave-level building blocks shared by the selection kernels: a wave-private LDS
// fence, wave-wide minima, the radix select of the need-th largest value and the
// ordered append of flagged entries.
#pragma once

#include "qsa_device.h"

namespace qsa {

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t y = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o, kWave) << 32) |
                       (uint32_t)__shfl_xor((int)(uint32_t)v, o, kWave);
    v = y < v ? y : v;
  }
  return v;
}

// The need-th largest of the BITS-wide values that each(f) presents (f(v) once per
// present value, on the lane holding it), found digit by digit from the top, starting
// below the bits that all values share. Returns the prefix fixed so far and its width
// in pbits: the values whose top pbits bits are at or above the prefix are the need
// largest (with ties, when every bit is fixed, the values equal to the need-th largest
// may add more). need is clamped to the number of present values.
template <int BITS, class Each>
__device__ __forceinline__ uint64_t wave_radix_select(uint32_t* hist, uint32_t need, Each each,
                                                      int& pbits) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t lo = ~0ull, nhi = ~0ull;  // min and (complemented) max
  uint32_t total = 0;
  each([&](uint64_t v) {
    lo = v < lo ? v : lo;
    nhi = ~v < nhi ? ~v : nhi;
    ++total;
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) total += (uint32_t)__shfl_xor((int)total, o, kWave);
  need = min(need, total);
  pbits = 0;
  if (need == 0) return 0;
  lo = wave_min_u64(lo);
  const uint64_t hi = ~wave_min_u64(nhi);
  if (lo == hi) {
    pbits = BITS;
    return hi;
  }
  const int diff = 64 - __clzll((long long)(lo ^ hi));  // width of the differing low part
  pbits = BITS - diff;
  uint64_t prefix = diff >= 64 ? 0ull : hi >> diff;
  while (pbits < BITS) {
    const int w = min(8, BITS - pbits);
    const int shift = BITS - pbits - w;
    *reinterpret_cast<uint4*>(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
    wave_lds_sync();
    each([&](uint64_t v) {
      if ((shift + w >= 64 ? 0ull : v >> (shift + w)) == prefix)
        atomicAdd(&hist[(uint32_t)(v >> shift) & ((1u << w) - 1u)], 1u);
    });
    wave_lds_sync();
    const uint4 h = *reinterpret_cast<const uint4*>(hist + 4 * lane);
    const uint32_t s = h.x + h.y + h.z + h.w;
    uint32_t suf = s;  // values in the bins of lanes >= this one
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t y = __shfl_down(suf, o, kWave);
      if (lane + o < kWave) suf += y;
    }
    // bin 4*lane + e holds h_e values, with a_e values in the bins above it
    const uint32_t a3 = suf - s, a2 = a3 + h.w, a1 = a2 + h.z, a0 = a1 + h.y;
    int e = -1;
    uint32_t above = 0, cnt = 0;
    if (a3 < need && need <= a3 + h.w) {
      e = 3; above = a3; cnt = h.w;
    } else if (a2 < need && need <= a2 + h.z) {
      e = 2; above = a2; cnt = h.z;
    } else if (a1 < need && need <= a1 + h.y) {
      e = 1; above = a1; cnt = h.y;
    } else if (a0 < need && need <= a0 + h.x) {
      e = 0; above = a0; cnt = h.x;
    }
    const uint64_t hit = __ballot(e >= 0);
    const int src = (int)__ffsll((unsigned long long)hit) - 1;  // exactly one bin holds it
    const int digit = __shfl(4 * lane + e, src, kWave);
    need -= (uint32_t)__shfl((int)above, src, kWave);
    const uint32_t in_bin = (uint32_t)__shfl((int)cnt, src, kWave);
    prefix = (prefix << w) | (uint32_t)digit;
    pbits += w;
    if (in_bin == need) break;  // the whole bin is kept
    wave_lds_sync();
  }
  return prefix;
}

// Appends the flagged entries of a lane's float4 (ids p0..p0+3) in id order, after
// `count` entries so far; returns this float4's entry total (wave-uniform).
template <class Put>
__device__ __forceinline__ uint32_t wave_append4(const bool (&f)[4], uint32_t count, Put put) {
  const int k = (int)f[0] + (int)f[1] + (int)f[2] + (int)f[3];
  const uint64_t b0 = __ballot(k & 1), b1 = __ballot(k & 2), b2 = __ballot(k & 4);
  uint32_t p = count + (uint32_t)(lane_prefix(b0) + 2 * lane_prefix(b1) + 4 * lane_prefix(b2));
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (f[e]) put(p++, e);
  return (uint32_t)(__popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2));
}

}  // namespace qsa

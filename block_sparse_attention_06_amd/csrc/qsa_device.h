// Device-side helpers shared by the QSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two fp32 values to a packed pair of bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16].
// Lane l holds A row (l % 16) and B column (l % 16), k = 8*(l/16) + [0..7];
// D column (l % 16), rows 4*(l/16) + [0..3].
__device__ __forceinline__ f32x4 mfma_16x16x32(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16: D[16x16] += A[16x16] * B[16x16].
// Lane l holds A row (l % 16) and B column (l % 16), k = 4*(l/16) + [0..3];
// D column (l % 16), rows 4*(l/16) + [0..3].
__device__ __forceinline__ f32x4 mfma_16x16x16(const uint2& a, const uint2& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// One block score from the 4 per-head dot products of a token (MFMA accumulator
// lanes): sum_h w_h * max(0, dot_h), always in this order, so that every kernel that
// scores blocks produces the same fp32 value.
__device__ __forceinline__ float score_of_heads(const float (&W)[4], const f32x4& acc) {
  // ReLU as an integer max on the bits: a finite float has its sign bit set exactly
  // when its bits, read as an int32, are negative (-0 included, which becomes +0), so
  // max(bits, 0) is max(x, 0) in one v_max_i32, where fmaxf costs a canonicalising max
  // before the max.
  auto relu = [](float x) { return __int_as_float(max(__float_as_int(x), 0)); };
  float s = W[0] * relu(acc[0]);
  s = fmaf(W[1], relu(acc[1]), s);
  s = fmaf(W[2], relu(acc[2]), s);
  return fmaf(W[3], relu(acc[3]), s);
}

// Order-preserving map of a finite fp32 to uint32 (larger float -> larger key),
// with -0.0 folded onto +0.0 so that the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key (-0.0 comes back as +0.0).
__device__ __forceinline__ float key_to_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Rank composite of a (score, id) pair: larger means ranked earlier (score
// descending, then id ascending). 0 is below every finite score's composite.
__device__ __forceinline__ uint64_t rank_key(float v, int32_t id) {
  return ((uint64_t)order_key(v) << 32) | (uint64_t)(0xffffffffu - (uint32_t)id);
}

__device__ __forceinline__ int32_t rank_key_id(uint64_t rk) {
  return (int32_t)(0xffffffffu - (uint32_t)rk);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Position of this lane among the set lanes of `mask` below it.
__device__ __forceinline__ int lane_prefix(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Wave-wide, by repeated maxima: extract the `keep` largest of the 64 x SLOTS rank
// keys held by the lanes (0 = empty slot), largest first; calls emit(k, rank_key) on
// the lane that held the k-th one. Returns the last extracted key (wave-uniform), 0 if
// keep == 0. Costs one wave-wide reduction per key.
template <int SLOTS, class Emit>
__device__ __forceinline__ uint64_t wave_extract_top_iter(uint64_t (&rk)[SLOTS], int keep,
                                                          Emit emit) {
  uint64_t last = 0;
  for (int k = 0; k < keep; ++k) {
    uint64_t best = 0;
    int slot = 0;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i)
      if (rk[i] > best) {
        best = rk[i];
        slot = i;
      }
    uint64_t wbest = best;
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)wbest, d, 64);
      const uint32_t hi = __shfl_xor((uint32_t)(wbest >> 32), d, 64);
      const uint64_t o = ((uint64_t)hi << 32) | lo;
      wbest = o > wbest ? o : wbest;
    }
    if (best == wbest && wbest != 0) {  // ids are unique: one lane holds the winner
#pragma unroll
      for (int i = 0; i < SLOTS; ++i)
        if (i == slot) rk[i] = 0ull;
      emit(k, wbest);
    }
    last = wbest;
  }
  return last;
}

// Same contract as wave_extract_top_iter for keep <= 16, in three wave-wide passes
// instead of one reduction per key:
//  1. the keep-th largest high word (the score's order key) of the 64 lane maxima,
//     found bit by bit with ballots, gives thr: every key whose high word reaches it
//     is a candidate, and there are at least keep of them (one per such lane);
//  2. the keys >= thr (at least keep of them) are packed into `scratch`, 64 wave-private
//     LDS slots (more than 64 of them, possible only when the largest keys crowd into
//     few lanes, falls back to the repeated maxima);
//  3. each packed key's rank is the number of packed keys above it.
// The nonzero keys must be distinct (rank keys carry the id).
template <int SLOTS, class Emit>
__device__ __forceinline__ uint64_t wave_extract_top(uint64_t (&rk)[SLOTS], int keep,
                                                     uint64_t* scratch, Emit emit) {
  if (keep <= 0) return 0;
  const int lane = threadIdx.x & 63;
  uint64_t mx = rk[0];
#pragma unroll
  for (int i = 1; i < SLOTS; ++i) mx = rk[i] > mx ? rk[i] : mx;
  const uint32_t mhi = (uint32_t)(mx >> 32);
  uint32_t pre = 0;  // the largest v with at least keep lanes' high words >= v
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = pre | (1u << b);
    if (__popcll(__ballot(mhi >= cand)) >= keep) pre = cand;
  }
  // Fewer than keep nonempty lanes leave pre = 0: every nonzero key is a candidate.
  const uint64_t thr = pre ? ((uint64_t)pre << 32) : 1ull;
  int total = 0;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const bool in = rk[i] >= thr;
    const uint64_t m = __ballot(in);
    const int pos = total + lane_prefix(m);
    if (in && pos < 64) scratch[pos] = rk[i];
    total += __popcll(m);
  }
  if (total > 64) return wave_extract_top_iter<SLOTS>(rk, keep, emit);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t v = lane < total ? scratch[lane] : 0ull;
  int r = 0;
  for (int j = 0; j < total; ++j) r += readlane_u64(v, j) > v ? 1 : 0;
  if (lane < total && r < keep) emit(r, v);
  const uint64_t at = __ballot(lane < total && r == keep - 1);
  return readlane_u64(v, __builtin_ctzll(at));
}

// Element offset of 16-byte chunk `ch` of row `row` in an LDS tile of pooled keys
// (DI bf16 a row, no padding). The score kernels read B operands with lane c16 taking
// row 4*c16 + j and one chunk per instruction, so with plain rows every fourth lane
// would hit the same banks; XOR-ing the chunk with the row's group of four, (row / 4)
// mod (chunks a row), gives the 16 lanes distinct chunk positions, while the 16-byte
// writes of one row still cover each position once.
template <int DI>
__device__ __forceinline__ int key_tile_off(int row, int ch) {
  constexpr int CPR = DI / 8;
  return row * DI + ((ch ^ ((row >> 2) & (CPR - 1))) << 3);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// The value of lane l and that of lane l ^ mask (mask 16 or 32, a constant), in some
// order, without a trip through LDS: gfx950's lane-swap instructions exchange odd
// 16-lane rows of one operand with even rows of the other (permlane16) or the upper
// half of one with the lower half of the other (permlane32), so with the same value
// as both operands the two results hold, lane by lane, the value and its partner's.
__device__ __forceinline__ u32x2 xor_pair(float x, int mask) {
  const uint32_t u = __float_as_uint(x);
  return mask == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                    : __builtin_amdgcn_permlane32_swap(u, u, false, false);
}

__device__ __forceinline__ float wave_xor_max(float x, int mask) {
  if (mask == 16 || mask == 32) {
    const u32x2 r = xor_pair(x, mask);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return fmaxf(x, __shfl_xor(x, mask, kWave));
}

// (Addition is commutative, so the order of the pair does not change the sum.)
__device__ __forceinline__ float wave_xor_sum(float x, int mask) {
  if (mask == 16 || mask == 32) {
    const u32x2 r = xor_pair(x, mask);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x + __shfl_xor(x, mask, kWave);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal (streamed data that will not be reused soon).
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

}  // namespace qsa

// Stage 3 of QSA: per query row, keep the best blocks under the token budget.
//
// Method ("Qwen3.8-Flash-Next" Miles recipe, section 1: each layer keeps
// indexer_budget key tokens per query; "On the Design of Qwen3.8-Next
// Architecture", item 2 QSA: token budget K = 2048 over micro-blocks of r = 4):
// keep the query's own block plus the m = min(K/r - 1, C) best of the C earlier
// blocks, ranked by score (descending) then block id (ascending); emit the kept ids
// in ascending order, padded with -1.
//
// One workgroup per row, exact radix select on order-preserving 32-bit keys:
//   1. up to three histogram passes over the row (12, 12, 8 key bits), each
//      restricted to the keys sharing the prefix found so far, until the bucket
//      that holds the m-th best key has at most kTieCap members;
//   2. a collection pass: keys above the bucket are kept outright, keys in the
//      bucket go to an LDS list that is sorted by (key desc, id asc) to take the
//      rest -- or, if even the full 32-bit key leaves more than kTieCap equal keys,
//      an in-order scan takes the lowest ids among them;
//   3. the kept ids are sorted ascending in LDS and written with the own block.
// No floating-point atomics; the result does not depend on scheduling.

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

constexpr int kTkThreads = 256;
constexpr int kTieCap = 4096;
constexpr int kMaxSel = 1024;
constexpr int kHistBins = 4096;

struct TopkShared {
  uint32_t hist[kHistBins];
  uint32_t tie_key[kTieCap];
  int32_t tie_idx[kTieCap];
  int32_t kept[kMaxSel];
  uint32_t scan[kTkThreads];
  int32_t misc[8];
};

// Block-wide: find digit D with above(D) < need <= above(D) + hist[D], where
// above(D) counts the keys in digits > D. Results in sm.misc[0..2].
__device__ void find_digit(TopkShared& sm, int nbins, uint32_t need) {
  const int tid = threadIdx.x;
  const int per = nbins / kTkThreads;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += sm.hist[tid * per + i];
  uint32_t v = local;
  sm.scan[tid] = v;
  __syncthreads();
  for (int off = 1; off < kTkThreads; off <<= 1) {
    const uint32_t add = (tid + off < kTkThreads) ? sm.scan[tid + off] : 0u;
    __syncthreads();
    v += add;
    sm.scan[tid] = v;
    __syncthreads();
  }
  const uint32_t above_me = v - local;  // keys in bins owned by higher threads
  if (above_me < need && need <= v) {
    uint32_t acc = above_me;
    for (int d = (tid + 1) * per - 1; d >= tid * per; --d) {
      const uint32_t h = sm.hist[d];
      if (acc + h >= need) {
        sm.misc[0] = d;
        sm.misc[1] = (int32_t)acc;
        sm.misc[2] = (int32_t)h;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTkThreads) void topk_rows_kernel(TopkArgs a) {
  __shared__ TopkShared sm;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int bi = blockIdx.y;
  const int64_t base = a.seq_lens ? (int64_t)a.seq_lens[bi] - a.lq : a.q_pos0;
  const int64_t t = base + row;
  int32_t* out = a.sel + ((int64_t)bi * a.lq + row) * a.n_sel;
  if (t < 0) {
    for (int k = tid; k < a.n_sel; k += kTkThreads) out[k] = -1;
    return;
  }
  const int64_t own = t / a.r;
  const int64_t C = min(own, a.nblk);
  const int m = (int)min((int64_t)(a.n_sel - 1), C);
  if (m == C) {  // every earlier block fits in the budget
    for (int k = tid; k < a.n_sel; k += kTkThreads)
      out[k] = k < C ? k : (k == C ? (int32_t)own : -1);
    return;
  }
  const float* srow = a.scores + (int64_t)bi * a.s_bs + row * a.ld;
  const int64_t n4 = (C + 3) / 4;  // float4 reads; ld % 4 == 0 keeps them inside the row

  // ---- 1. radix descent on the key prefix ----
  uint32_t prefix = 0;
  int pbits = 0;
  uint32_t need = (uint32_t)m;
  uint32_t bucket = 0;
  for (int level = 0; level < 3; ++level) {
    const int wbits = level < 2 ? 12 : 8;
    const int nbins = 1 << wbits;
    const int shift = 32 - pbits - wbits;
    for (int i = tid; i < nbins; i += kTkThreads) sm.hist[i] = 0;
    __syncthreads();
    for (int64_t i4 = tid; i4 < n4; i4 += kTkThreads) {
      const float4 x = *reinterpret_cast<const float4*>(srow + i4 * 4);
      const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (i4 * 4 + e < C) {
          const uint32_t key = order_key(xs[e]);
          if (pbits == 0 || (key >> (32 - pbits)) == prefix)
            atomicAdd(&sm.hist[(key >> shift) & (nbins - 1)], 1u);
        }
      }
    }
    __syncthreads();
    find_digit(sm, nbins, need);
    const uint32_t D = (uint32_t)sm.misc[0];
    need -= (uint32_t)sm.misc[1];
    bucket = (uint32_t)sm.misc[2];
    prefix = (prefix << wbits) | D;
    pbits += wbits;
    __syncthreads();
    if (bucket <= (uint32_t)kTieCap) break;
  }

  // ---- 2. collect ----
  const bool tie_fits = bucket <= (uint32_t)kTieCap;
  const int n_out = m - (int)need;  // keys strictly above the bucket
  if (tid == 0) {
    sm.misc[3] = 0;
    sm.misc[4] = 0;
  }
  __syncthreads();
  const int pshift = 32 - pbits;
  for (int64_t i4 = tid; i4 < n4; i4 += kTkThreads) {
    const float4 x = *reinterpret_cast<const float4*>(srow + i4 * 4);
    const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t idx = i4 * 4 + e;
      if (idx < C) {
        const uint32_t key = order_key(xs[e]);
        const uint32_t top = pshift == 32 ? 0u : (key >> pshift);
        if (top > prefix) {
          const int p = atomicAdd(&sm.misc[3], 1);
          sm.kept[p] = (int32_t)idx;
        } else if (top == prefix && tie_fits) {
          const int p = atomicAdd(&sm.misc[4], 1);
          sm.tie_key[p] = key;
          sm.tie_idx[p] = (int32_t)idx;
        }
      }
    }
  }
  __syncthreads();

  if (tie_fits) {
    const int n_tie = sm.misc[4];
    int P = 1;
    while (P < n_tie) P <<= 1;
    for (int i = n_tie + tid; i < P; i += kTkThreads) {
      sm.tie_key[i] = 0u;
      sm.tie_idx[i] = 0x7fffffff;
    }
    __syncthreads();
    // Bitonic sort into rank order: key descending, then id ascending.
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P; i += kTkThreads) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint32_t ka = sm.tie_key[i], kb = sm.tie_key[ixj];
            const int32_t ia = sm.tie_idx[i], ib = sm.tie_idx[ixj];
            const bool a_first = ka > kb || (ka == kb && ia < ib);
            const bool up = (i & k) == 0;
            if (up != a_first) {
              sm.tie_key[i] = kb;
              sm.tie_key[ixj] = ka;
              sm.tie_idx[i] = ib;
              sm.tie_idx[ixj] = ia;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int k = tid; k < (int)need; k += kTkThreads) sm.kept[n_out + k] = sm.tie_idx[k];
  } else {
    // The full key is known and more than kTieCap candidates share it: take the
    // `need` lowest ids among them, scanning the row in id order.
    const int lane = tid & 63, wave = tid >> 6;
    int taken = 0;
    for (int64_t b0 = 0; b0 < C && taken < (int)need; b0 += kTkThreads) {
      const int64_t idx = b0 + tid;
      const bool flag = idx < C && order_key(srow[idx]) == prefix;
      const uint64_t bal = __ballot(flag);
      const int wpre = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) sm.scan[wave] = (uint32_t)__popcll(bal);
      __syncthreads();
      int woff = 0, tot = 0;
      for (int w = 0; w < kTkThreads / 64; ++w) {
        if (w < wave) woff += (int)sm.scan[w];
        tot += (int)sm.scan[w];
      }
      const int pos = taken + woff + wpre;
      if (flag && pos < (int)need) sm.kept[n_out + pos] = (int32_t)idx;
      taken += tot;
      __syncthreads();
    }
  }
  __syncthreads();

  // ---- 3. ascending ids, own block last, -1 padding ----
  int P = 1;
  while (P < m) P <<= 1;
  for (int i = m + tid; i < P; i += kTkThreads) sm.kept[i] = 0x7fffffff;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += kTkThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const int32_t x = sm.kept[i], y = sm.kept[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            sm.kept[i] = y;
            sm.kept[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int k = tid; k < a.n_sel; k += kTkThreads)
    out[k] = k < m ? sm.kept[k] : (k == m ? (int32_t)own : -1);
}

hipError_t launch_topk_blocks(const TopkArgs& a, hipStream_t stream) {
  if (a.lq <= 0 || a.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)a.lq, (unsigned)a.batch), dim3(kTkThreads),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace qsa

// Stage 3 of QSA: per query row, keep the best blocks under the token budget.
//
// Method ("Qwen3.8-Flash-Next" Miles recipe, section 1: each layer keeps
// indexer_budget key tokens per query; "On the Design of Qwen3.8-Next
// Architecture", item 2 QSA: token budget K = 2048 over micro-blocks of r = 4):
// keep the query's own block plus the m = min(K/r - 1, C) best of the C earlier
// blocks, ranked by score (descending) then block id (ascending); emit the kept ids
// in ascending order, padded with -1.
//
// Rows of at most kSegMax candidates: one wave per row (topk_wave_rows_kernel below),
// reading the row about once -- a sample sets a key threshold, one streaming pass
// collects the scores at or above it into a wave-private list, and a radix select on
// (score, id) ranks finds the m best in it; a list that overflowed or came out short
// sends the wave through the whole row instead.
// Rows longer than kSegMax candidates, when there are many: one wave per kSegMax-score
// segment keeps the segment's m best with that same selection, and one wave per row
// selects the m best of what its segments kept (topk_long_segments_kernel,
// topk_long_merge_kernel). Few long rows (decode) use two launches with more, smaller
// pieces: one wave per segment of
// kWaveSeg scores keeps its kWaveKeep best (wave-wide passes, no barriers)
// and reports the worst of them; the merge (one workgroup per row) selects the m best
// of all kept candidates, which is the row's answer when every truncated segment's
// reported worst ranks at or after the m-th selected (nothing left behind could rank
// higher); otherwise the merge repeats the exact selection over the whole row. The
// merge's selection of the m best among n candidates:
//   0. for a long list, a sample (every k-th run of 32 consecutive scores) gives a
//      value bin above which roughly 2m candidates are expected, and one streaming
//      pass appends every candidate at or above it to an LDS list (an upper set of the
//      value order: if it holds at least m candidates it holds the m best);
//   a. min / max, then a histogram over kLinBins equal-width value bins; the map
//      x -> floor((x - min) * bins / (max - min)) is monotone and sends equal values
//      (and -0.0 / +0.0) to one bin, so every candidate in a bin above the bin B that
//      holds the m-th best ranks before every candidate in B;
//   b. only if B is large: radix descent on the order-preserving 32-bit key inside B;
//   c. candidates above the final bucket are kept; the bucket is sorted in LDS by
//      (key desc, id asc) -- or, when more than kTieCap candidates share one exact
//      key, a radix select on the id keeps the lowest ids.
// No floating-point atomics; results do not depend on scheduling.

#include "qsa_device.h"
#include "qsa_wave.h"
#include "qsa_internal.h"

namespace qsa {

constexpr int kTkThreads = 256;
constexpr int kWaves = kTkThreads / 64;
constexpr int kSegMax = 32768;  // candidates per workgroup (bitmap size of the output)
constexpr int kLinBins = 2048;
constexpr int kListCap = 2048;  // filtered candidates kept in LDS
constexpr int kTieCap = 512;
constexpr int kMaxSel = 1024;
constexpr int kSampleRun = 32;  // consecutive scores per sampled run
constexpr int kSampleMax = 4096;

constexpr int kWaveSeg = kTopkWaveSeg;    // scores per wave in the first pass
constexpr int kWaveKeep = kTopkWaveKeep;  // candidates kept per wave segment


template <int LIST, int BWORDS>
struct TkSharedT {
  static constexpr int kList = LIST;         // filtered candidates kept in LDS
  static constexpr int kBitmapWords = BWORDS;  // output bitmap (ids < 32 * BWORDS)
  uint32_t hist[kLinBins];
  float list_val[LIST];
  int32_t list_idx[LIST];
  uint32_t tie_key[kTieCap];
  int32_t tie_idx[kTieCap];
  uint32_t bitmap[BWORDS];
  int32_t kept[kMaxSel];
  uint32_t wsum[kWaves];
  float wred[2 * kWaves];
  int32_t misc[8];
};
using TkMergeShared = TkSharedT<2 * kListCap, 262144 / 32>;   // ~82 KB

// ---- block-level primitives ---------------------------------------------------------

template <class SM>
__device__ __forceinline__ uint32_t block_excl_scan(SM& sm, uint32_t v, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) sm.wsum[wave] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t s = sm.wsum[w];
    off += (w < wave) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return off + x - v;
}

template <class SM>
__device__ __forceinline__ void block_minmax(SM& sm, float& mn, float& mx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, d, 64));
    mx = fmaxf(mx, __shfl_xor(mx, d, 64));
  }
  if (lane == 0) {
    sm.wred[wave] = mn;
    sm.wred[kWaves + wave] = mx;
  }
  __syncthreads();
  mn = sm.wred[0];
  mx = sm.wred[kWaves];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    mn = fminf(mn, sm.wred[w]);
    mx = fmaxf(mx, sm.wred[kWaves + w]);
  }
  __syncthreads();
}

// Over hist[0..nbins), find D with above(D) < need <= above(D) + hist[D], above(D) being
// the count in digits > D (thread 0 owns the highest digits). Results in misc[0..2].
template <class SM>
__device__ __forceinline__ void find_digit(SM& sm, int nbins, uint32_t need) {
  const int tid = threadIdx.x;
  const int per = nbins / kTkThreads;
  const int hi = nbins - tid * per - 1;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += sm.hist[hi - i];
  uint32_t total;
  const uint32_t above_me = block_excl_scan(sm, local, total);
  if (above_me < need && need <= above_me + local) {
    uint32_t acc = above_me;
    for (int d = hi; d > hi - per; --d) {
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

template <class SM>
__device__ __forceinline__ void clear_hist(SM& sm, int nbins) {
  for (int i = threadIdx.x; i < nbins; i += kTkThreads) sm.hist[i] = 0u;
  __syncthreads();
}

// Equal-width value bins over [lo, lo + kLinBins / sc]; monotone, clamped.
struct LinBins {
  float lo, sc;
  __device__ __forceinline__ int operator()(float v) const {
    return max(0, min(kLinBins - 1, (int)((v - lo) * sc)));
  }
};

__device__ __forceinline__ LinBins make_bins(float mn, float mx) {
  float sc = (float)kLinBins / (mx - mn);
  if (!(mx > mn) || !(sc < 3.0e38f)) sc = 0.f;  // one value (or no usable range): one bin
  return LinBins{mn, sc};
}

// Block-wide minimum of a 64-bit value (the worst-ranked of the threads' values).
template <class SM>
__device__ __forceinline__ uint64_t block_min_u64(SM& sm, uint64_t v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, d, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o < v ? o : v;
  }
  if (lane == 0) {
    sm.wsum[wave] = (uint32_t)v;
    sm.wred[wave] = __uint_as_float((uint32_t)(v >> 32));
  }
  __syncthreads();
  uint64_t r = ~0ull;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint64_t o = ((uint64_t)__float_as_uint(sm.wred[w]) << 32) | sm.wsum[w];
    r = o < r ? o : r;
  }
  __syncthreads();
  return r;
}

// ---- element sources (NaN marks an absent element) ----------------------------------

struct RowSrc {  // values p[i] (NaN: absent), ids ids[i] when given, else lo + i
  const float* p;
  const int32_t* ids;
  int lo;
  __device__ __forceinline__ float val(int i) const { return p[i]; }
  __device__ __forceinline__ int id(int i) const { return ids ? ids[i] : lo + i; }
};

struct PairSrc {  // (value, id) pairs in global or shared memory; id < 0 is absent
  const float* v;
  const int32_t* ids;
  __device__ __forceinline__ float val(int i) const {
    return ids[i] >= 0 ? v[i] : __builtin_nanf("");
  }
  __device__ __forceinline__ int id(int i) const { return ids[i]; }
};

// ---- exact selection of the m best of n elements of a source ------------------------
// mark(i) is called exactly once for each selected element (by position i). With
// REGS (n <= kTkThreads * kRegSlots) each thread first loads its elements into
// registers with independent loads, and every pass runs on registers; otherwise each
// pass streams the source again.

constexpr int kRegSlots = 16;  // largest register-held share per thread

template <int SLOTS, class SM, class Src, class Mark>
__device__ void select_exact_impl(SM& sm, const Src& src, int n, int m, Mark mark) {
  constexpr bool REGS = SLOTS > 0;
  constexpr int kRegSlots = REGS ? SLOTS : 1;
  const int tid = threadIdx.x;
  float xr[kRegSlots];
  int32_t ir[kRegSlots];
  if constexpr (REGS) {
#pragma unroll
    for (int j = 0; j < kRegSlots; ++j) {
      const int i = tid + kTkThreads * j;
      xr[j] = i < n ? src.val(i) : __builtin_nanf("");
      ir[j] = i < n ? src.id(i) : -1;
    }
  }
  // each(f): f(position, value, id) over this thread's elements (NaN value: absent)
  auto each = [&](auto&& f) {
    if constexpr (REGS) {
#pragma unroll
      for (int j = 0; j < kRegSlots; ++j) f(tid + kTkThreads * j, xr[j], ir[j]);
    } else {
      for (int i = tid; i < n; i += kTkThreads) f(i, src.val(i), src.id(i));
    }
  };

  float mn = INFINITY, mx = -INFINITY;
  each([&](int, float v, int) {
    mn = fminf(mn, v);  // fminf / fmaxf ignore NaN
    mx = fmaxf(mx, v);
  });
  block_minmax(sm, mn, mx);
  const LinBins bins = make_bins(mn, mx);
  clear_hist(sm, kLinBins);
  each([&](int, float v, int) {
    if (v == v) atomicAdd(&sm.hist[bins(v)], 1u);
  });
  __syncthreads();
  find_digit(sm, kLinBins, (uint32_t)m);
  const int B = sm.misc[0];
  uint32_t need = (uint32_t)m - (uint32_t)sm.misc[1];
  uint32_t bucket = (uint32_t)sm.misc[2];
  __syncthreads();

  // Radix descent on the key inside bin B while the bucket is too large.
  uint32_t prefix = 0;
  int pbits = 0;
  for (int level = 0; level < 3 && bucket > (uint32_t)kTieCap; ++level) {
    const int wbits = level < 2 ? 11 : 10;
    const int nb = 1 << wbits;
    const int shift = 32 - pbits - wbits;
    clear_hist(sm, nb);
    each([&](int, float v, int) {
      if (v == v && bins(v) == B) {
        const uint32_t key = order_key(v);
        if (pbits == 0 || (key >> (32 - pbits)) == prefix)
          atomicAdd(&sm.hist[(key >> shift) & (nb - 1)], 1u);
      }
    });
    __syncthreads();
    find_digit(sm, nb, need);
    need -= (uint32_t)sm.misc[1];
    bucket = (uint32_t)sm.misc[2];
    prefix = (prefix << wbits) | (uint32_t)sm.misc[0];
    pbits += wbits;
    __syncthreads();
  }
  // rel: 1 above the bucket, 0 in it, -1 below (or absent)
  auto rel_of = [&](float v) -> int {
    if (!(v == v)) return -1;
    const int b = bins(v);
    if (b != B) return b > B ? 1 : -1;
    if (pbits == 0) return 0;
    const uint32_t top = order_key(v) >> (32 - pbits);
    return top > prefix ? 1 : (top == prefix ? 0 : -1);
  };

  const bool fits = bucket <= (uint32_t)kTieCap;
  if (tid == 0) sm.misc[4] = 0;
  __syncthreads();
  each([&](int i, float v, int id) {
    const int rel = rel_of(v);
    if (rel > 0) {
      mark(i);
    } else if (rel == 0 && fits) {
      const int p = atomicAdd(&sm.misc[4], 1);
      sm.tie_key[p] = order_key(v);
      sm.tie_idx[p] = id;
    }
  });
  __syncthreads();

  if (fits) {
    const int n_tie = sm.misc[4];
    int P = 1;
    while (P < n_tie) P <<= 1;
    for (int i = n_tie + tid; i < P; i += kTkThreads) {
      sm.tie_key[i] = 0u;
      sm.tie_idx[i] = 0x7fffffff;
    }
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P; i += kTkThreads) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint32_t ka = sm.tie_key[i], kb = sm.tie_key[ixj];
            const int32_t ia = sm.tie_idx[i], ib = sm.tie_idx[ixj];
            const bool a_first = ka > kb || (ka == kb && ia < ib);
            if (((i & k) == 0) != a_first) {
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
    if (need > 0) {
      // The first `need` of the sorted bucket are kept: everything ranking at or
      // before the need-th entry.
      const uint32_t lim_key = sm.tie_key[need - 1];
      const int32_t lim_idx = sm.tie_idx[need - 1];
      each([&](int i, float v, int id) {
        if (rel_of(v) == 0) {
          const uint32_t key = order_key(v);
          if (key > lim_key || (key == lim_key && id <= lim_idx)) mark(i);
        }
      });
    }
  } else {
    // pbits == 32: the bucket is one exact key; keep its `need` lowest ids. Radix
    // select on the 22-bit id, ascending (digits reversed for the generic search).
    uint32_t iprefix = 0;
    int ibits = 0;
    uint32_t ineed = need;
    for (int level = 0; level < 2; ++level) {
      const int nb = 1 << 11;
      const int shift = 22 - ibits - 11;
      clear_hist(sm, nb);
      each([&](int, float v, int id) {
        const uint32_t d = (uint32_t)id;
        if (rel_of(v) == 0 && (ibits == 0 || (d >> (22 - ibits)) == iprefix))
          atomicAdd(&sm.hist[nb - 1 - ((d >> shift) & (nb - 1))], 1u);
      });
      __syncthreads();
      find_digit(sm, nb, ineed);
      ineed -= (uint32_t)sm.misc[1];
      iprefix = (iprefix << 11) | (uint32_t)(nb - 1 - sm.misc[0]);
      ibits += 11;
      __syncthreads();
    }
    each([&](int i, float v, int id) {
      if (rel_of(v) == 0 && (uint32_t)id <= iprefix) mark(i);
    });
  }
  __syncthreads();
}

// SLOTS: register-held elements per thread for n <= kTkThreads * SLOTS (0: stream).
template <int SLOTS, class SM, class Src, class Mark>
__device__ __forceinline__ void select_exact(SM& sm, const Src& src, int n, int m, Mark mark) {
  if (SLOTS > 0 && n <= kTkThreads * SLOTS)
    select_exact_impl<SLOTS>(sm, src, n, m, mark);
  else
    select_exact_impl<0>(sm, src, n, m, mark);
}

// ---- filtered selection over a row segment ------------------------------------------
// Selects the m best of row[0..n) (16-byte aligned; NaN entries are absent; ids are
// ids[i] when given, else lo + i), calling mark(id, value) once per kept element.

constexpr int kChunkVec = 8;  // float4 loads in flight per thread in the streaming pass

__device__ __forceinline__ float4 load4_masked(const float* row, int i, int n) {
  const float qn = __builtin_nanf("");
  if (i + 3 < n) return *reinterpret_cast<const float4*>(row + i);
  float4 v = make_float4(qn, qn, qn, qn);
  if (i < n) v.x = row[i];
  if (i + 1 < n) v.y = row[i + 1];
  if (i + 2 < n) v.z = row[i + 2];
  return v;
}

template <class SM, class Mark>
__device__ void select_row(SM& sm, const float* row, const int32_t* ids, int lo, int n,
                           int m, Mark mark) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // 1. Sample every k-th run of kSampleRun scores (at most kSampleMax samples), held in
  //    registers: 4 float4 per thread.
  const int runs = (n + kSampleRun - 1) / kSampleRun;
  int k = 1;
  while ((runs + k - 1) / k * kSampleRun > kSampleMax) ++k;
  const int s_n4 = (runs + k - 1) / k * (kSampleRun / 4);
  constexpr int kS4 = kSampleMax / 4 / kTkThreads;
  float smp[kS4][4];
  float mn = INFINITY, mx = -INFINITY;
  int s_valid = 0;
#pragma unroll
  for (int q = 0; q < kS4; ++q) {
    const int s4 = tid + kTkThreads * q;
    const int i = (s4 / (kSampleRun / 4)) * k * kSampleRun + (s4 % (kSampleRun / 4)) * 4;
    const float qn = __builtin_nanf("");
    const float4 v = s4 < s_n4 ? load4_masked(row, i, n) : make_float4(qn, qn, qn, qn);
    smp[q][0] = v.x;
    smp[q][1] = v.y;
    smp[q][2] = v.z;
    smp[q][3] = v.w;
  }
#pragma unroll
  for (int q = 0; q < kS4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mn = fminf(mn, smp[q][e]);
      mx = fmaxf(mx, smp[q][e]);
      s_valid += smp[q][e] == smp[q][e];
    }
  block_minmax(sm, mn, mx);
  uint32_t s_total;
  block_excl_scan(sm, (uint32_t)s_valid, s_total);
  const LinBins sb = make_bins(mn, mx);
  // Sample rank aiming at ~2m candidates in the whole segment.
  const float frac = (float)s_total / (float)n;
  int rank = (int)ceilf(2.0f * (float)m * frac) + 8;
  rank = min(rank, (int)s_total);
  clear_hist(sm, kLinBins);
#pragma unroll
  for (int q = 0; q < kS4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (smp[q][e] == smp[q][e]) atomicAdd(&sm.hist[sb(smp[q][e])], 1u);
  __syncthreads();
  find_digit(sm, kLinBins, (uint32_t)rank);
  const int Bs = sm.misc[0];
  if (tid == 0) sm.misc[5] = 0;  // list length
  __syncthreads();

  // 2. One pass over the segment: append every element with sample bin >= Bs.
  constexpr int kChunk = kTkThreads * kChunkVec * 4;
  for (int c0 = 0; c0 < n; c0 += kChunk) {
    float4 v[kChunkVec];
#pragma unroll
    for (int q = 0; q < kChunkVec; ++q) v[q] = load4_masked(row, c0 + (q * kTkThreads + tid) * 4, n);
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < kChunkVec; ++q) {
      const float xs[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) cnt += (xs[e] == xs[e] && sb(xs[e]) >= Bs);
    }
    int x = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    int base = 0;
    if (lane == 63 && x > 0) base = atomicAdd(&sm.misc[5], x);
    base = __shfl(base, 63, 64);
    int p = base + x - cnt;
    if (cnt) {
#pragma unroll
      for (int q = 0; q < kChunkVec; ++q) {
        const float xs[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (xs[e] == xs[e] && sb(xs[e]) >= Bs) {
            if (p < SM::kList) {
              const int i = c0 + (q * kTkThreads + tid) * 4 + e;
              sm.list_val[p] = xs[e];
              sm.list_idx[p] = ids ? ids[i] : lo + i;
            }
            ++p;
          }
      }
    }
  }
  __syncthreads();
  const int n_list = sm.misc[5];
  __syncthreads();
  // 3. Exact selection on the list when it is a valid upper set, else on the segment.
  if (n_list >= m && n_list <= SM::kList) {
    select_exact<SM::kList / kTkThreads>(sm, PairSrc{sm.list_val, sm.list_idx}, n_list, m,
                                         [&](int i) { mark(sm.list_idx[i], sm.list_val[i]); });
  } else {
    select_exact<0>(sm, RowSrc{row, ids, lo}, n, m,
                    [&](int i) { mark(ids ? ids[i] : lo + i, row[i]); });
  }
}

// ---- kernels ------------------------------------------------------------------------

struct TopkLaunch {
  TopkArgs a;
  int seg;          // segment length
  int n_seg;        // segments per row
  float* cand_val;  // [rows][n_seg][kseg], NaN where absent
  int32_t* cand_idx;
  float* bnd_val;   // [rows][n_seg]: worst kept of a truncated segment (id -1: complete)
  int32_t* bnd_idx;
  int kseg;         // candidates kept per segment (multiple of 4)
};

// Position t, own block, candidate count C and kept count m of launch row `row` of
// sequence bi; returns the row's output (null when packed sequence bi has no such row).
__device__ __forceinline__ int32_t* row_geometry(const TopkArgs& a, int64_t row, int bi,
                                                 int64_t& t, int64_t& own, int64_t& C, int& m) {
  int64_t base = a.seq_lens ? (int64_t)a.seq_lens[bi] - a.lq : a.q_pos0;
  int32_t* out = a.sel + ((int64_t)bi * a.lq + row) * a.n_sel;
  if (a.vl.cu_q) {
    const SeqRows sr = varlen_rows(a.vl, bi, a.lq);
    if (row >= sr.n) return nullptr;
    base = sr.pos;
    out = a.sel + (sr.first + row) * a.n_sel;
  }
  t = base + row;
  own = t >= 0 ? t / a.r : -1;
  C = t >= 0 ? min(own, a.nblk) : 0;
  m = (int)min((int64_t)(a.n_sel - 1), C);
  return out;
}

// Writes the ids marked in sm.bitmap (ids < 32 * words) to out[0..) in ascending order.
template <class SM>
__device__ __forceinline__ void write_bitmap_ids(SM& sm, int words, int32_t* out) {
  const int tid = threadIdx.x;
  constexpr int wpt = SM::kBitmapWords / kTkThreads;
  uint32_t b[wpt];
  uint32_t cnt = 0;
#pragma unroll
  for (int w = 0; w < wpt; ++w) {
    const int wi = tid * wpt + w;
    b[w] = wi < words ? sm.bitmap[wi] : 0u;
    cnt += __popc(b[w]);
  }
  uint32_t total;
  uint32_t off = block_excl_scan(sm, cnt, total);
#pragma unroll
  for (int w = 0; w < wpt; ++w) {
    const int wi = tid * wpt + w;
    uint32_t bits = b[w];
    while (bits) {
      const int bpos = __ffs(bits) - 1;
      bits &= bits - 1;
      out[off++] = wi * 32 + bpos;
    }
  }
}

// Ascending sort of N ids in registers (bitonic network, N a power of 2).
template <int N>
__device__ __forceinline__ void sort_ids_asc(int32_t (&x)[N]) {
#pragma unroll
  for (int k = 2; k <= N; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int l = i ^ j;
        if (l > i) {
          const int32_t a = x[i], b = x[l];
          const bool up = (i & k) == 0;
          x[i] = up ? min(a, b) : max(a, b);
          x[l] = up ? max(a, b) : min(a, b);
        }
      }
}

// Merge of the segment winners when every segment fits a thread's share: thread t
// holds segments t + kTkThreads*j (j < kMergeSPT) with their kWaveKeep candidates
// each. merge_fetch issues their loads at kernel entry (they do not depend on the
// row's length) and clears the value histogram meanwhile; merge_segments_fast then
// finds the m-th best key T from one value histogram plus a rank count inside T's bin
// (at most 64 entries, else it returns 1 and the general merge runs). With fewer than
// m candidates, or a truncated segment whose reported worst ranks above T (it may
// hide a better candidate), it returns 2: the whole row must be selected. Otherwise
// each segment's kept ids are written, sorted, at the segment's offset (segments
// cover ascending id ranges, so the output is ascending) and it returns 0.
// segments per thread: enough for rows of 2^18 blocks (1M tokens at r = 4)
constexpr int kMergeSPT = (262144 / kWaveSeg + kTkThreads - 1) / kTkThreads;
constexpr int kMergeCand = kMergeSPT * kWaveKeep;  // candidates per thread
static_assert(kWaveKeep % 4 == 0 && (kWaveKeep & (kWaveKeep - 1)) == 0, "kept per segment");

struct MergeRegs {
  float v[kMergeCand];
  int32_t id[kMergeCand];
  uint64_t bkey[kMergeSPT];
};

template <class SM>
__device__ __forceinline__ void merge_fetch(SM& sm, const TopkLaunch& L, int64_t crow,
                                            MergeRegs& r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kMergeSPT; ++j) {
    const int seg = tid + kTkThreads * j;
    const bool have = seg < L.n_seg;
    const int64_t slot = crow * L.n_seg + (have ? seg : 0);
    const float4* cv4 = reinterpret_cast<const float4*>(L.cand_val + slot * kWaveKeep);
    const int4* ci4 = reinterpret_cast<const int4*>(L.cand_idx + slot * kWaveKeep);
#pragma unroll
    for (int q = 0; q < kWaveKeep / 4; ++q) {
      const float qn = __builtin_nanf("");
      const float4 a = have ? cv4[q] : make_float4(qn, qn, qn, qn);
      const int4 b = have ? ci4[q] : make_int4(-1, -1, -1, -1);
      float* v = r.v + j * kWaveKeep + 4 * q;
      int32_t* id = r.id + j * kWaveKeep + 4 * q;
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      id[0] = b.x; id[1] = b.y; id[2] = b.z; id[3] = b.w;
    }
    const int32_t bid = have ? L.bnd_idx[slot] : -1;
    const float bval = have ? L.bnd_val[slot] : 0.f;
    r.bkey[j] = bid >= 0 ? rank_key(bval, bid) : 0ull;
  }
  for (int i = tid; i < kLinBins; i += kTkThreads) sm.hist[i] = 0u;
  if (tid == 0) sm.misc[4] = 0;
}

template <class SM>
__device__ __forceinline__ int merge_segments_fast(SM& sm, MergeRegs& r, int m, int32_t* out) {
  constexpr int KC = kMergeCand;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* v = r.v;
  const int32_t* id = r.id;
  // One reduction for the value range and the number of candidates.
  float mn = INFINITY, mx = -INFINITY;
  uint32_t n_valid = 0;
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    if (id[j] < 0) v[j] = __builtin_nanf("");  // absent
    mn = fminf(mn, v[j]);  // fminf / fmaxf ignore NaN
    mx = fmaxf(mx, v[j]);
    n_valid += v[j] == v[j] ? 1u : 0u;
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, d, 64));
    mx = fmaxf(mx, __shfl_xor(mx, d, 64));
    n_valid += __shfl_xor(n_valid, d, 64);
  }
  if (lane == 0) {
    sm.wred[wave] = mn;
    sm.wred[kWaves + wave] = mx;
    sm.wsum[wave] = n_valid;
  }
  __syncthreads();  // also orders merge_fetch's histogram clear before the counts
  n_valid = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mn = fminf(mn, sm.wred[w]);
    mx = fmaxf(mx, sm.wred[kWaves + w]);
    n_valid += sm.wsum[w];
  }
  // Fewer candidates than places (short rows of a long launch): the whole row decides.
  if (n_valid < (uint32_t)m) return 2;
  const LinBins bins = make_bins(mn, mx);
#pragma unroll
  for (int j = 0; j < KC; ++j)
    if (v[j] == v[j]) atomicAdd(&sm.hist[bins(v[j])], 1u);
  __syncthreads();
  find_digit(sm, kLinBins, (uint32_t)m);
  const int B = sm.misc[0];
  const int need = m - sm.misc[1];
  const int bucket = sm.misc[2];
  if (bucket > 64) return 1;
#pragma unroll
  for (int j = 0; j < KC; ++j)
    if (v[j] == v[j] && bins(v[j]) == B) {
      const int p = atomicAdd(&sm.misc[4], 1);
      sm.tie_key[p] = order_key(v[j]);
      sm.tie_idx[p] = id[j];
    }
  __syncthreads();
  if (wave == 0) {
    const int nb = sm.misc[4];
    const uint64_t k =
        lane < nb ? rank_key(key_to_float(sm.tie_key[lane]), sm.tie_idx[lane]) : 0ull;
    int rk = 0;
    for (int j = 0; j < nb; ++j) rk += readlane_u64(k, j) > k ? 1 : 0;
    if (lane < nb && rk == need - 1) {
      sm.misc[5] = (int32_t)(uint32_t)(k >> 32);
      sm.misc[6] = (int32_t)(uint32_t)k;
    }
  }
  __syncthreads();
  const uint64_t T = ((uint64_t)(uint32_t)sm.misc[5] << 32) | (uint32_t)sm.misc[6];
  bool bad = false;
#pragma unroll
  for (int j = 0; j < kMergeSPT; ++j) bad |= r.bkey[j] > T;
  // Per-segment counts packed in 16-bit fields (a field's total stays below
  // kTkThreads * kWaveKeep <= 4096), one scan for all of this thread's segments. With
  // one field the scan also carries the truncation check: a flagged thread adds
  // 1 << 16, so the total shows whether any segment failed it.
  static_assert(kMergeSPT <= 2, "two 16-bit count fields");
  if (kMergeSPT > 1 && __syncthreads_or(bad)) return 2;
  uint32_t cnt[kMergeSPT], packed = (kMergeSPT == 1 && bad) ? (1u << 16) : 0u;
#pragma unroll
  for (int j = 0; j < kMergeSPT; ++j) {
    cnt[j] = 0;
#pragma unroll
    for (int e = 0; e < kWaveKeep; ++e) {
      const int c = j * kWaveKeep + e;
      cnt[j] += (v[c] == v[c] && rank_key(v[c], id[c]) >= T) ? 1u : 0u;
    }
    packed |= cnt[j] << (16 * j);
  }
  uint32_t total;
  const uint32_t off = block_excl_scan(sm, packed, total);
  if (kMergeSPT == 1 && total >= (1u << 16)) return 2;
  uint32_t base = 0;
#pragma unroll
  for (int j = 0; j < kMergeSPT; ++j) {
    const uint32_t o = base + ((off >> (16 * j)) & 0xffffu);
    base += (total >> (16 * j)) & 0xffffu;
    if (cnt[j]) {
      int32_t kept[kWaveKeep];
#pragma unroll
      for (int e = 0; e < kWaveKeep; ++e) {
        const int c = j * kWaveKeep + e;
        kept[e] = (v[c] == v[c] && rank_key(v[c], id[c]) >= T) ? id[c] : 0x7fffffff;
      }
      sort_ids_asc<kWaveKeep>(kept);
#pragma unroll
      for (int e = 0; e < kWaveKeep; ++e)
        if ((uint32_t)e < cnt[j]) out[o + e] = kept[e];
    }
  }
  return 0;
}

// Merge of the segment winners of long rows (one workgroup per row): check that no
// truncated segment could hide a better candidate (else redo the selection on the
// whole row), write the ids ascending.
__global__ __launch_bounds__(kTkThreads) void topk_merge_kernel(TopkLaunch L) {
  using SM = TkMergeShared;
  __shared__ SM sm;
  const TopkArgs& a = L.a;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int bi = blockIdx.z;
  const int64_t crow = (int64_t)bi * a.lq + row;
  MergeRegs mr;
  const bool fast_merge = L.n_seg <= kTkThreads * kMergeSPT;
  if (fast_merge) merge_fetch(sm, L, crow, mr);
  int64_t t, own, C;
  int m;
  int32_t* out = row_geometry(a, row, bi, t, own, C, m);
  if (!out) return;  // packed sequence shorter than this launch's rows
  const float* srow = a.scores + (int64_t)bi * a.s_bs + row * a.ld;

  if (t < 0 || m == C) {  // nothing to rank: every earlier block fits
    for (int k = tid; k < a.n_sel; k += kTkThreads)
      out[k] = t < 0 ? -1 : (k < C ? k : (k == C ? (int32_t)own : -1));
    return;
  }

  {
    int fast = 1;
    if (fast_merge) {
      fast = merge_segments_fast(sm, mr, m, out);
      if (fast == 0) {
        for (int k = m + tid; k < a.n_sel; k += kTkThreads) out[k] = k == m ? (int32_t)own : -1;
        return;
      }
    }
    const int n = L.n_seg * kWaveKeep;
    const float* cv = L.cand_val + crow * n;
    const int32_t* ci = L.cand_idx + crow * n;
    const bool use_bitmap = C <= (int64_t)SM::kBitmapWords * 32;
    const int words = use_bitmap ? (int)((C + 31) / 32) : 0;
    for (int i = tid; i < words; i += kTkThreads) sm.bitmap[i] = 0u;
    if (tid == 0) sm.misc[7] = 0;
    __syncthreads();
    uint64_t worst = ~0ull;
    auto keep_id = [&](int id, float v) {
      if (use_bitmap) {
        atomicOr(&sm.bitmap[id >> 5], 1u << (id & 31));
      } else {
        const int p = atomicAdd(&sm.misc[7], 1);
        sm.kept[p] = id;
      }
      const uint64_t rk = rank_key(v, id);
      worst = rk < worst ? rk : worst;
    };
    bool bad = fast == 2;  // the fast merge found the candidates insufficient
    if (!bad) {
      uint32_t my_valid = 0, total_valid;
      for (int i = tid; i < n; i += kTkThreads) my_valid += ci[i] >= 0 && cv[i] == cv[i];
      block_excl_scan(sm, my_valid, total_valid);
      bad = total_valid < (uint32_t)m;  // fewer candidates than places: whole row
    }
    if (!bad) {
      if (n <= kTkThreads * kRegSlots) {
        // Few candidates: each thread holds its share in registers.
        select_exact<kRegSlots>(sm, PairSrc{cv, ci}, n, m, [&](int i) { keep_id(ci[i], cv[i]); });
      } else {
        select_row(sm, cv, ci, 0, n, m, keep_id);
      }
      worst = block_min_u64(sm, worst);
      for (int sg = tid; sg < L.n_seg; sg += kTkThreads) {
        const int32_t bid = L.bnd_idx[crow * L.n_seg + sg];
        if (bid >= 0 && rank_key(L.bnd_val[crow * L.n_seg + sg], bid) > worst) bad = true;
      }
    }
    if (__syncthreads_or(bad)) {
      for (int i = tid; i < words; i += kTkThreads) sm.bitmap[i] = 0u;
      if (tid == 0) sm.misc[7] = 0;
      __syncthreads();
      select_row(sm, srow, nullptr, 0, (int)C, m, keep_id);
    }
    if (use_bitmap) {
      write_bitmap_ids(sm, words, out);
    } else {
      int P = 1;
      while (P < m) P <<= 1;
      for (int i = m + tid; i < P; i += kTkThreads) sm.kept[i] = 0x7fffffff;
      __syncthreads();
      for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
          for (int i = tid; i < P; i += kTkThreads) {
            const int ixj = i ^ j;
            if (ixj > i) {
              const int32_t u = sm.kept[i], v = sm.kept[ixj];
              if ((u > v) == ((i & k) == 0)) {
                sm.kept[i] = v;
                sm.kept[ixj] = u;
              }
            }
          }
          __syncthreads();
        }
      }
      for (int k = tid; k < m; k += kTkThreads) out[k] = sm.kept[k];
    }
    for (int k = m + tid; k < a.n_sel; k += kTkThreads) out[k] = k == m ? (int32_t)own : -1;
  }
}

// First pass over long rows: each wave takes kSegsPerWave consecutive segments (row,
// seg) of kWaveSeg scores, each lane holding kWaveSeg / 64 of them, and extracts each
// segment's kWaveKeep best (score, id) rank keys. The next segment's scores are loaded
// before the current one is ranked; the winners wait in LDS and leave in one burst of
// coalesced stores at the end (a store among the loads would drain every wait).
constexpr int kSegsPerWave = 4;

__global__ __launch_bounds__(256) void topk_wave_segments_kernel(TopkLaunch L) {
  constexpr int kQ = kWaveSeg / 256;  // float4 loads per lane
  constexpr int kOut = kSegsPerWave * kWaveKeep;
  static_assert(kOut == 64, "one candidate per lane in the final stores");
  __shared__ uint64_t scratch[4][64];
  __shared__ float out_v[4][kOut];
  __shared__ int32_t out_i[4][kOut];
  __shared__ float out_bv[4][kSegsPerWave];
  __shared__ int32_t out_bi[4][kSegsPerWave];
  const TopkArgs& a = L.a;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t n_items = (int64_t)a.batch * a.lq * L.n_seg;  // item = row * n_seg + seg
  const int64_t item0 = ((int64_t)blockIdx.x * 4 + wave) * kSegsPerWave;
  if (item0 >= n_items) return;

  struct Seg {
    const float* src;  // the segment's first score (a valid address when not live)
    int n, lo;         // scores in the segment, first block id
    bool live;         // the merge reads this segment's candidates
  };
  auto geom = [&](int64_t item) {
    Seg sg{a.scores, 0, 0, false};
    if (item >= n_items) return sg;
    const int64_t crow = item / L.n_seg;
    const int seg_id = (int)(item - crow * L.n_seg);
    const int bi = (int)(crow / a.lq);
    const int64_t row = crow - (int64_t)bi * a.lq;
    int64_t t, own, C;
    int m;
    if (!row_geometry(a, row, bi, t, own, C, m)) return sg;
    if (t < 0 || m == C) return sg;  // the merge writes such rows without candidates
    sg.live = true;
    sg.lo = seg_id * kWaveSeg;
    sg.n = (int)max((int64_t)0, min(C - sg.lo, (int64_t)kWaveSeg));
    sg.src = a.scores + (int64_t)bi * a.s_bs + row * a.ld + sg.lo;
    return sg;
  };
  // lane holds positions 4*(lane + 64*q) + e; loads past the segment's scores read its
  // last aligned float4 (inside the row: ld % 4 == 0), so every load is unconditional.
  auto load = [&](const Seg& sg, float4 (&v)[kQ]) {
    const int pmax = sg.n > 0 ? ((sg.n - 1) & ~3) : 0;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      v[q] = *reinterpret_cast<const float4*>(sg.src + min(4 * (lane + 64 * q), pmax));
  };
  auto rank = [&](const Seg& sg, const float4 (&v)[kQ], int k) {
    uint64_t rk[4 * kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int p = 4 * (lane + 64 * q);
      const float xs[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) rk[4 * q + e] = p + e < sg.n ? rank_key(xs[e], sg.lo + p + e) : 0ull;
    }
    const int keep = min(sg.n, kWaveKeep);
    // Empty slots first (the extraction fills 0..keep-1), then the winners; a -0 score
    // comes back as +0, which ranks the same.
    if (lane < kWaveKeep) {
      out_v[wave][k * kWaveKeep + lane] = __builtin_nanf("");
      out_i[wave][k * kWaveKeep + lane] = -1;
    }
    const uint64_t last = wave_extract_top<4 * kQ>(rk, keep, scratch[wave], [&](int r, uint64_t w) {
      out_v[wave][k * kWaveKeep + r] = key_to_float((uint32_t)(w >> 32));
      out_i[wave][k * kWaveKeep + r] = rank_key_id(w);
    });
    if (lane == 0) {
      const bool truncated = sg.n > keep;
      out_bv[wave][k] = truncated ? key_to_float((uint32_t)(last >> 32)) : 0.f;
      out_bi[wave][k] = truncated ? rank_key_id(last) : -1;
    }
    // The next extraction reuses the scratch slots.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  bool live[kSegsPerWave];
  Seg cur = geom(item0);
  float4 vc[kQ], vn[kQ];
  load(cur, vc);
#pragma unroll
  for (int k = 0; k < kSegsPerWave; ++k) {
    const Seg nxt = geom(item0 + k + 1);
    if (k + 1 < kSegsPerWave) load(nxt, vn);
    __builtin_amdgcn_sched_barrier(0);
    live[k] = cur.live;
    if (cur.live) rank(cur, vc, k);
    cur = nxt;
#pragma unroll
    for (int q = 0; q < kQ; ++q) vc[q] = vn[q];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // Consecutive items have consecutive candidate slots: lane L stores candidate L % 16
  // of segment L / 16.
  const int k = lane / kWaveKeep;
  bool mine = false;
#pragma unroll
  for (int j = 0; j < kSegsPerWave; ++j) mine = j == k ? live[j] : mine;
  if (mine) {
    L.cand_val[item0 * kWaveKeep + lane] = out_v[wave][lane];
    L.cand_idx[item0 * kWaveKeep + lane] = out_i[wave][lane];
  }
  if (lane < kSegsPerWave) {
    bool lv = false;
#pragma unroll
    for (int j = 0; j < kSegsPerWave; ++j) lv = j == lane ? live[j] : lv;
    if (lv) {
      L.bnd_val[item0 + lane] = out_bv[wave][lane];
      L.bnd_idx[item0 + lane] = out_bi[wave][lane];
    }
  }
}

// ---- one wave per row ----------------------------------------------------------------
// Rows of at most kSegMax candidates, one wave each and no workgroup barriers, so that
// many rows are in flight per CU:
//   1. a row longer than the list (cap entries) is sampled at 64 evenly spaced runs of
//      32 scores (one 128-byte line each); the k-th largest sample, k aiming at
//      sqrt(m * cap) list entries over the whole row, is the key threshold. Shorter
//      rows take every score;
//   2. one streaming pass appends each score at or above the threshold, as (order key,
//      position), to a wave-private LDS list in position order: a lane's 0..4 entries
//      of a float4 are placed by three ballots of its count's bits;
//   3. the list is held in registers as 48-bit ranks (key, then 0xffff - position:
//      larger ranks first, all distinct) and a radix select with 8-bit digits finds the
//      m-th rank; the entries at or above it are written in list order, which is
//      ascending id order.
// A list that overflowed or came out shorter than m runs step 3 over the whole row,
// streamed from memory once per digit. NaN scores are absent, as in the rest of this
// file. The result is the same as the workgroup kernel's for any row.
constexpr int kWrCap = 2048;              // list entries per wave, at most
constexpr int kWrCapSmall = 1664;         // for m <= 511: 4 workgroups per CU
constexpr int kWrSlots = kWrCap / kWave;  // list entries per lane, at most
constexpr int kWrSampleSlots = 32;        // sampled scores per lane (2048 a wave)
constexpr int kWrVec = 8;                 // float4 loads in flight per lane while streaming
constexpr int kWrRowsPerWg = 4;

// A wave's LDS: key[cap] then pos[cap]; the 256-bin histogram of the radix select
// reuses key[0..256), which holds nothing live while a histogram is in use (the list
// is read into registers before its selection).
struct WrLds {
  uint32_t* key;
  uint16_t* pos;
  uint32_t* hist;
  int cap;
};

__device__ __forceinline__ uint64_t wr_rank(uint32_t key, int pos) {
  return ((uint64_t)key << 16) | (uint64_t)(0xffffu - (uint32_t)pos);
}

// Float4 q of the streaming chunk at c0 (clamped into the row; positions >= n absent).
__device__ __forceinline__ float4 wr_load(const float* row, int c0, int q, int n) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i = min(c0 + (q * kWave + lane) * 4, (n - 1) & ~3);
  return *reinterpret_cast<const float4*>(row + i);
}

// This wave's part of the dynamic LDS of a launch with list size cap.
__device__ __forceinline__ WrLds wr_lds(uint32_t* smem, int cap) {
  const int wave = threadIdx.x >> 6;
  return WrLds{smem + wave * cap,
               reinterpret_cast<uint16_t*>(smem + kWrRowsPerWg * cap) + wave * cap,
               smem + wave * cap, cap};
}

// Selects the m best of row[0..n) (positions as ids; NaN absent) and calls emit(k, pos,
// value) for the k-th kept in ascending position order (k < m), then pad(k) for the
// places a row with fewer than m present scores leaves empty.
template <class Emit, class Pad>
__device__ void wave_select_row(const WrLds L, const float* row, int n, int m, Emit emit,
                                Pad pad) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int kChunk = kWave * 4 * kWrVec;
  // 1. Threshold key (0 admits every score).
  uint32_t tau = 0;
  const int cap = L.cap;
  if (n > cap) {
    // 64 runs of 32 consecutive scores (8 float4, 128 bytes), evenly spaced: a
    // lane reads float4 (lane & 7) of run s * 8 + (lane >> 3).
    const int n_runs = (n >> 2) >> 3;  // complete runs, >= 64 here
    uint32_t sk[kWrSampleSlots];
#pragma unroll
    for (int s = 0; s < kWrSampleSlots / 4; ++s) {
      const int run = (int)((int64_t)(s * 8 + (lane >> 3)) * n_runs / 64);
      const int i = (run * 8 + (lane & 7)) * 4;
      const float4 v = *reinterpret_cast<const float4*>(row + i);
      const float xs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) sk[4 * s + e] = xs[e] == xs[e] ? order_key(xs[e]) : 0u;
    }
    uint32_t nv = 0;
#pragma unroll
    for (int j = 0; j < kWrSampleSlots; ++j) nv += sk[j] != 0u;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) nv += __shfl_xor(nv, o, kWave);
    if (nv > 0) {
      // aim at the geometric mean of m and cap: the count's error is a factor
      const int64_t tgt = (int64_t)sqrtf((float)m * (float)cap);
      const uint32_t k = (uint32_t)max<int64_t>(1, (tgt * nv + n - 1) / n);
      int pb;
      const uint64_t pre = wave_radix_select<32>(
          L.hist, k,
          [&](auto&& f) {
#pragma unroll
            for (int j = 0; j < kWrSampleSlots; ++j)
              if (sk[j]) f((uint64_t)sk[j]);
          },
          pb);
      tau = (uint32_t)(pre << (32 - pb));
      // A threshold on a value the row's scores tie at in numbers (exact zeros after
      // the ReLU) admits every tie: when the sample says that overflows the list while
      // the scores above it still fill m, admit only those above.
      uint32_t above = 0, atleast = 0;
#pragma unroll
      for (int j = 0; j < kWrSampleSlots; ++j) {
        above += sk[j] > tau;
        atleast += sk[j] >= tau;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        above += __shfl_xor(above, o, kWave);
        atleast += __shfl_xor(atleast, o, kWave);
      }
      if ((int64_t)atleast * n > (int64_t)cap * nv && (int64_t)above * n >= (int64_t)m * nv &&
          tau < 0xffffffffu)
        ++tau;
    }
    wave_lds_sync();
  }
  // 2. Stream the row into the list, the next chunk's loads in flight meanwhile. The
  // key threshold is compared as the least float whose key reaches it.
  const float tf = tau <= 0x007fffffu ? -INFINITY : key_to_float(tau);
  uint32_t count = 0;
  auto take = [&](const float4 (&v)[kWrVec], int c0) {
#pragma unroll
    for (int q = 0; q < kWrVec; ++q) {
      const int i = c0 + (q * kWave + lane) * 4;
      const float xs[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
      bool f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = xs[e] >= tf && i + e < n;  // NaN: false
      if (__ballot(f[0] || f[1] || f[2] || f[3]) == 0ull) continue;
      count += wave_append4(f, count, [&](uint32_t p, int e) {
        if (p < (uint32_t)cap) {
          L.key[p] = order_key(xs[e]);
          L.pos[p] = (uint16_t)(i + e);
        }
      });
    }
  };
  // Loads are issued unconditionally (clamped into the row), so that waiting for one
  // buffer never waits for the other.
  float4 va[kWrVec], vb[kWrVec];
#pragma unroll
  for (int q = 0; q < kWrVec; ++q) va[q] = wr_load(row, 0, q, n);
  for (int c0 = 0; c0 < n; c0 += 2 * kChunk) {
#pragma unroll
    for (int q = 0; q < kWrVec; ++q) vb[q] = wr_load(row, c0 + kChunk, q, n);
    take(va, c0);
#pragma unroll
    for (int q = 0; q < kWrVec; ++q) va[q] = wr_load(row, c0 + 2 * kChunk, q, n);
    if (c0 + kChunk < n) take(vb, c0 + kChunk);
  }
  wave_lds_sync();
  uint32_t written = 0;
  if (count >= (uint32_t)m && count <= (uint32_t)cap) {
    // 3. Select on the list, in registers.
    uint64_t rk[kWrSlots];
#pragma unroll
    for (int j = 0; j < kWrSlots; ++j) {
      const uint32_t p = (uint32_t)(j * kWave + lane);
      rk[j] = p < count ? wr_rank(L.key[p], L.pos[p]) : 0ull;
    }
    int pb;
    const uint64_t pre = wave_radix_select<48>(
        L.hist, (uint32_t)m,
        [&](auto&& f) {
#pragma unroll
          for (int j = 0; j < kWrSlots; ++j)
            if (rk[j]) f(rk[j]);
        },
        pb);
#pragma unroll
    for (int j = 0; j < kWrSlots; ++j) {
      const bool kp = rk[j] != 0ull && (rk[j] >> (48 - pb)) >= pre;
      const uint64_t b = __ballot(kp);
      const uint32_t p = written + (uint32_t)lane_prefix(b);
      if (kp && p < (uint32_t)m)
        emit(p, (int)(0xffffu - (uint32_t)(rk[j] & 0xffffu)), key_to_float((uint32_t)(rk[j] >> 16)));
      written += (uint32_t)__popcll(b);
    }
    written = min(written, (uint32_t)m);
  } else {
    // The whole row, one streaming pass per digit, then one to write the kept ids.
    auto each_row = [&](auto&& f) {
      for (int c0 = 0; c0 < n; c0 += kChunk) {
        float4 v[kWrVec];
#pragma unroll
        for (int q = 0; q < kWrVec; ++q) v[q] = wr_load(row, c0, q, n);
#pragma unroll
        for (int q = 0; q < kWrVec; ++q) {
          const int i = c0 + (q * kWave + lane) * 4;
          const float xs[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (i + e < n && xs[e] == xs[e]) f(wr_rank(order_key(xs[e]), i + e));
        }
      }
    };
    int pb;
    const uint64_t pre = wave_radix_select<48>(L.hist, (uint32_t)m, each_row, pb);
    for (int c0 = 0; c0 < n; c0 += kChunk) {
      float4 v[kWrVec];
#pragma unroll
      for (int q = 0; q < kWrVec; ++q) v[q] = wr_load(row, c0, q, n);
#pragma unroll
      for (int q = 0; q < kWrVec; ++q) {
        const int i = c0 + (q * kWave + lane) * 4;
        const float xs[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
        bool f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          f[e] = i + e < n && xs[e] == xs[e] &&
                 (wr_rank(order_key(xs[e]), i + e) >> (48 - pb)) >= pre;
        written += wave_append4(f, written, [&](uint32_t p, int e) {
          if (p < (uint32_t)m) emit(p, i + e, xs[e]);
        });
      }
    }
    written = min(written, (uint32_t)m);
  }
  for (int k = (int)written + lane; k < m; k += kWave) pad(k);  // only with NaN scores
}

__global__ __launch_bounds__(kWrRowsPerWg * kWave) void topk_wave_rows_kernel(TopkArgs a,
                                                                              int cap) {
  extern __shared__ uint32_t wr_smem[];  // kWrRowsPerWg * cap * 6 bytes
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kWrRowsPerWg + wave;
  const int bi = blockIdx.z;
  if (row >= a.lq) return;
  int64_t t, own, C;
  int m;
  int32_t* out = row_geometry(a, row, bi, t, own, C, m);
  if (!out) return;
  if (t < 0 || m == C) {
    for (int k = lane; k < a.n_sel; k += kWave)
      out[k] = t < 0 ? -1 : (k < C ? k : (k == C ? (int32_t)own : -1));
    return;
  }
  if (m > 0)
    wave_select_row(wr_lds(wr_smem, cap), a.scores + (int64_t)bi * a.s_bs + row * a.ld, (int)C,
                    m, [&](uint32_t k, int pos, float) { out[k] = pos; },
                    [&](int k) { out[k] = -1; });
  for (int k = m + lane; k < a.n_sel; k += kWave) out[k] = k == m ? (int32_t)own : -1;
}

// ---- long rows by waves ----------------------------------------------------------------
// Rows of more than kSegMax candidates, when there are enough (row, segment) items to
// fill the GPU: pass 1 selects the m best of each kSegMax-score segment of a row with
// the one-wave selection and stores them in ascending id order as (score, id) in the
// segment's ks slots (NaN / -1 after them); pass 2 runs the same selection over the
// row's stored slots, whose order is id order, so ties still go to the lower id. A
// segment keeps its m best and the row keeps m, so nothing a segment dropped can be
// among the row's m best: the result is exact.
struct TopkLong {
  TopkArgs a;
  int n_wseg;  // segments of kSegMax scores per row
  int ks;      // candidate slots per segment (n_sel rounded up to 4)
  float* cand_val;  // [batch * lq][n_wseg][ks]
  int32_t* cand_idx;
  int cap;
};

__global__ __launch_bounds__(kWrRowsPerWg * kWave) void topk_long_segments_kernel(TopkLong T) {
  extern __shared__ uint32_t wr_smem[];  // kWrRowsPerWg * cap * 6 bytes
  const TopkArgs& a = T.a;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * kWrRowsPerWg + wave;
  if (item >= a.lq * T.n_wseg) return;
  const int64_t row = item / T.n_wseg;
  const int seg = (int)(item - row * T.n_wseg);
  const int bi = blockIdx.z;
  int64_t t, own, C;
  int m;
  if (!row_geometry(a, row, bi, t, own, C, m) || t < 0 || m == C) return;  // no candidates
  const int64_t slot0 = (((int64_t)bi * a.lq + row) * T.n_wseg + seg) * T.ks;
  float* cv = T.cand_val + slot0;
  int32_t* ci = T.cand_idx + slot0;
  const int64_t lo = (int64_t)seg * kSegMax;
  const int ns = (int)max<int64_t>(0, min<int64_t>(kSegMax, C - lo));
  const float* srow = a.scores + (int64_t)bi * a.s_bs + row * a.ld + lo;
  int kept;
  if (ns > m) {
    if (m > 0)
      wave_select_row(wr_lds(wr_smem, T.cap), srow, ns, m,
                      [&](uint32_t k, int pos, float v) {
                        cv[k] = v;
                        ci[k] = (int32_t)(lo + pos);
                      },
                      [&](int k) {
                        cv[k] = __builtin_nanf("");
                        ci[k] = -1;
                      });
    kept = m;
  } else {
    for (int k = lane; k < ns; k += kWave) {
      cv[k] = srow[k];
      ci[k] = (int32_t)(lo + k);
    }
    kept = ns;
  }
  for (int k = kept + lane; k < T.ks; k += kWave) {
    cv[k] = __builtin_nanf("");
    ci[k] = -1;
  }
}

__global__ __launch_bounds__(kWrRowsPerWg * kWave) void topk_long_merge_kernel(TopkLong T) {
  extern __shared__ uint32_t wr_smem[];
  const TopkArgs& a = T.a;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kWrRowsPerWg + wave;
  const int bi = blockIdx.z;
  if (row >= a.lq) return;
  int64_t t, own, C;
  int m;
  int32_t* out = row_geometry(a, row, bi, t, own, C, m);
  if (!out) return;
  if (t < 0 || m == C) {
    for (int k = lane; k < a.n_sel; k += kWave)
      out[k] = t < 0 ? -1 : (k < C ? k : (k == C ? (int32_t)own : -1));
    return;
  }
  if (m > 0) {
    const int64_t slot0 = ((int64_t)bi * a.lq + row) * T.n_wseg * T.ks;
    const int32_t* ci = T.cand_idx + slot0;
    const int n2 = (int)((C + kSegMax - 1) / kSegMax) * T.ks;  // this row's segments
    wave_select_row(wr_lds(wr_smem, T.cap), T.cand_val + slot0, n2, m,
                    [&](uint32_t k, int pos, float) { out[k] = ci[pos]; },
                    [&](int k) { out[k] = -1; });
  }
  for (int k = m + lane; k < a.n_sel; k += kWave) out[k] = k == m ? (int32_t)own : -1;
}

// ---- host side ----------------------------------------------------------------------

static int64_t max_candidates(const TopkArgs& a) {
  // Upper bound of C over the launch's rows (positions may come from the device).
  if (a.seq_lens || a.vl.cu_q) return a.nblk;
  const int64_t t_last = a.q_pos0 + a.lq - 1;
  return t_last < 0 ? 0 : min(t_last / a.r, a.nblk);
}

static int n_wave_segs(const TopkArgs& a) {
  return (int)((max_candidates(a) + kWaveSeg - 1) / kWaveSeg);
}

static size_t align_up(size_t n) { return (n + 255) & ~size_t(255); }

static int n_long_segs(const TopkArgs& a) {
  return (int)((max_candidates(a) + kSegMax - 1) / kSegMax);
}

static int long_slots(const TopkArgs& a) { return (a.n_sel + 3) & ~3; }

// Long rows by waves when there are at least 2048 (row, segment) items and a row's
// stored candidates fit one wave selection; else segments of kWaveSeg and the merge.
static bool long_by_waves(const TopkArgs& a) {
  if (max_candidates(a) <= kSegMax) return false;
  const int64_t items = (int64_t)a.batch * a.lq * n_long_segs(a);
  return items >= 2048 && (int64_t)n_long_segs(a) * long_slots(a) <= kSegMax;
}

// Either layout fits (the launch may pick the other one when its rows turn out shorter
// than the sizing assumed).
size_t topk_workspace_bytes(const TopkArgs& a) {
  if (max_candidates(a) <= kSegMax) return 0;
  const size_t rows = (size_t)a.batch * a.lq;
  const size_t segs = rows * n_wave_segs(a);
  const size_t seg_layout = 2 * align_up(segs * kWaveKeep * 4) + 2 * align_up(segs * 4);
  const size_t slots = rows * n_long_segs(a) * long_slots(a);
  const size_t wave_layout = 2 * align_up(slots * 4);
  return seg_layout > wave_layout ? seg_layout : wave_layout;
}

bool topk_supported(const TopkArgs& a) {
  return max_candidates(a) <= kSegMax ||
         (int64_t)n_wave_segs(a) * kWaveKeep < ((int64_t)1 << 30);
}

TopkCandidates topk_candidates(const TopkArgs& a, void* ws) {
  const int n_seg = n_wave_segs(a);
  const size_t segs = (size_t)a.batch * a.lq * n_seg;
  char* p = static_cast<char*>(ws);
  TopkCandidates c;
  c.n_seg = n_seg;
  c.cand_val = reinterpret_cast<float*>(p);
  p += align_up(segs * kWaveKeep * 4);
  c.cand_idx = reinterpret_cast<int32_t*>(p);
  p += align_up(segs * kWaveKeep * 4);
  c.bnd_val = reinterpret_cast<float*>(p);
  p += align_up(segs * 4);
  c.bnd_idx = reinterpret_cast<int32_t*>(p);
  return c;
}

static TopkLaunch merge_launch(const TopkArgs& a, void* ws) {
  const TopkCandidates c = topk_candidates(a, ws);
  return TopkLaunch{a, kWaveSeg, c.n_seg, c.cand_val, c.cand_idx, c.bnd_val, c.bnd_idx, kWaveKeep};
}

hipError_t launch_topk_merge(const TopkArgs& a, void* ws, hipStream_t stream) {
  if (a.lq <= 0 || a.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)a.lq, 1, (unsigned)a.batch),
                     dim3(kTkThreads), 0, stream, merge_launch(a, ws));
  return hipGetLastError();
}

hipError_t launch_topk_blocks(const TopkArgs& a, void* ws, hipStream_t stream) {
  if (a.lq <= 0 || a.batch <= 0) return hipSuccess;
  if (max_candidates(a) <= kSegMax) {
    const int cap = a.n_sel <= 512 ? kWrCapSmall : kWrCap;
    hipLaunchKernelGGL(topk_wave_rows_kernel,
                       dim3((unsigned)((a.lq + kWrRowsPerWg - 1) / kWrRowsPerWg), 1,
                            (unsigned)a.batch),
                       dim3(kWrRowsPerWg * kWave), (size_t)kWrRowsPerWg * cap * 6, stream, a,
                       cap);
    return hipGetLastError();
  }
  if (long_by_waves(a)) {
    const int n_wseg = n_long_segs(a), ks = long_slots(a);
    const size_t slots = (size_t)a.batch * a.lq * n_wseg * ks;
    float* cv = static_cast<float*>(ws);
    int32_t* ci = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + align_up(slots * 4));
    const int cap = a.n_sel <= 512 ? kWrCapSmall : kWrCap;
    const TopkLong T{a, n_wseg, ks, cv, ci, cap};
    const size_t lds = (size_t)kWrRowsPerWg * cap * 6;
    const int64_t items = a.lq * n_wseg;
    hipLaunchKernelGGL(topk_long_segments_kernel,
                       dim3((unsigned)((items + kWrRowsPerWg - 1) / kWrRowsPerWg), 1,
                            (unsigned)a.batch),
                       dim3(kWrRowsPerWg * kWave), lds, stream, T);
    hipLaunchKernelGGL(topk_long_merge_kernel,
                       dim3((unsigned)((a.lq + kWrRowsPerWg - 1) / kWrRowsPerWg), 1,
                            (unsigned)a.batch),
                       dim3(kWrRowsPerWg * kWave), lds, stream, T);
    return hipGetLastError();
  }
  const TopkLaunch L = merge_launch(a, ws);
  const size_t segs = (size_t)a.batch * a.lq * L.n_seg;
  const size_t per_wg = 4 * kSegsPerWave;
  hipLaunchKernelGGL(topk_wave_segments_kernel, dim3((unsigned)((segs + per_wg - 1) / per_wg)),
                     dim3(256), 0, stream, L);
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)a.lq, 1, (unsigned)a.batch),
                     dim3(kTkThreads), 0, stream, L);
  return hipGetLastError();
}

}  // namespace qsa

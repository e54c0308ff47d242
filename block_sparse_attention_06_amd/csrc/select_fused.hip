// Stages 2 and 3 of QSA fused for prefill rows: the block scores of a row never go to
// memory whole; only the scores that can still be among the row's best do.
//
// Method ("On the Design of Qwen3.8-Next Architecture", item 2 QSA: the light indexer
// scores micro-blocks of r = 4 tokens and the query keeps the best ones up to its token
// budget; "Qwen3.8-Flash-Next开源", section GDN+QSA: finding the important context is
// a cost of its own). The selection is the same as the two-kernel path's (the m best
// earlier blocks by score, then block id; own block kept), on the very same fp32 scores
// (score_of_heads), so the kept ids are identical.
//
// Per chunk of rows, five launches:
//  1. score_list_kernel<SAMPLE>: a workgroup takes 64 rows and one piece of their block
//     range, and scores its share of an evenly strided sample of the rows' blocks (one
//     in about lim * sample_k / target), keeping each lane's 8 best sampled keys per row.
//  2. score_list_kernel: the same workgroups merge the pieces' sampled keys and set each
//     row's threshold at about the sample_k-th best sampled score, which about `target`
//     of the row's scores reach. They then score their piece on MFMA as the plain GEMM
//     does, and each of the 16 lanes that hold a row's scores appends its own scores at
//     or above the threshold, with their block ids, to a list of its own: no cross-lane
//     bookkeeping, no atomics (placing entries by ballot prefix counts cost as much as
//     the products).
//  3. list_select_kernel: one wave per row. A row whose candidates all fit keeps them;
//     otherwise, if its lane lists hold at least m and at most the capacity in all,
//     they hold the row's m best (every score that is not in them is below the
//     threshold, below each of at least m listed ones). A radix select on the listed
//     ranks finds the m-th; the kept ids go out ascending through an LDS bitmap over
//     the row's blocks. Other rows are flagged.
//  4. The plain score GEMM, only on 64-row tiles that hold a flagged row.
//  5. fallback_select_kernel: one wave per flagged row, an exact radix select streamed
//     over its materialised scores.

#include <type_traits>

#include "qsa_device.h"
#include "qsa_internal.h"
#include "qsa_wave.h"

namespace qsa {

namespace {

constexpr int kFsRows = 64;    // query rows per workgroup (4 waves x 16)
constexpr int kFsTileN = 64;   // pooled keys per LDS tile
constexpr int kFsTopR = 8;     // sampled keys a lane keeps per row (two uint4)
constexpr int kFsIdBits = 24;  // block ids in a rank (ids < 2^24)
constexpr int kFsRankBits = 32 + kFsIdBits;
constexpr uint32_t kFsIdMask = (1u << kFsIdBits) - 1u;
constexpr int kLsSlots = kFusedListCap / kWave;
constexpr int kFsLanes = 16;  // lanes holding one row's scores: one list each
constexpr int kLsMapWords = 2048;  // bitmap words of a list-select wave (65536 blocks)

// Rank of a (score, id) pair: larger ranks earlier (score descending, then id
// ascending); 0 is no entry.
__device__ __forceinline__ uint64_t fs_rank(float v, int id) {
  return ((uint64_t)order_key(v) << kFsIdBits) | (uint64_t)(kFsIdMask - (uint32_t)id);
}

__device__ __forceinline__ int fs_rank_id(uint64_t rk) {
  return (int)(kFsIdMask - (uint32_t)(rk & kFsIdMask));
}

// Sum over the 16 lanes of this lane's quad group (lanes 16q .. 16q + 15).
__device__ __forceinline__ int group16_sum(int x) {
  x += __shfl_xor(x, 1, kWave);
  x += __shfl_xor(x, 2, kWave);
  x += __shfl_xor(x, 4, kWave);
  x += __shfl_xor(x, 8, kWave);
  return x;
}

// SAMPLE: score this piece's share of the rows' strided sample and store, per row and
// lane, its kFsTopR best sampled keys and its sample count (no lists). Otherwise: take
// the row thresholds from all pieces' sample shares, then score the piece and append.
template <int DI, bool SAMPLE>
__global__ __launch_bounds__(256, 2) void score_list_kernel(FusedSelArgs f) {
  constexpr int NC = DI / 32;
  constexpr int VPR = DI / 8;
  constexpr int LPT = kFsTileN * VPR / 256;
  __shared__ __attribute__((aligned(16))) uint16_t tile[2][kFsTileN * DI];  // key_tile_off layout

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int64_t n_tiles = (f.lq + kFsRows - 1) / kFsRows;
  const int64_t i0 = (n_tiles - 1 - (int64_t)blockIdx.x) * kFsRows;  // longest rows first
  const int split = blockIdx.y;
  const int64_t t_last = f.q_pos0 + min(i0 + kFsRows - 1, f.lq - 1);
  const int64_t nb_need = min(t_last / f.r, f.nblk);

  // Per accumulator row of this lane: token (mt*4 + quad) of the wave's 16.
  float W[4][4];
  int lim[4];   // candidates of the token (blocks < 2^24)
  int tokv[4];  // the token's row in the chunk, -1 past its end
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t tok = i0 + wave * 16 + mt * 4 + quad;
    const bool valid = tok < f.lq;
    tokv[mt] = valid ? (int)tok : -1;
    lim[mt] = valid ? (int)min((f.q_pos0 + tok) / f.r, f.nblk) : 0;
#pragma unroll
    for (int h = 0; h < 4; ++h) W[mt][h] = (valid && h < f.h_idx) ? f.w[tok * f.h_idx + h] : 0.f;
  }
  int cnt[4] = {0, 0, 0, 0};  // entries in this lane's list of each of its rows
  if (nb_need > 0) {
    const int64_t n_begin = (nb_need * split / f.n_split) / kFsTileN * kFsTileN;
    const int64_t n_end = split + 1 == f.n_split
                              ? nb_need
                              : (nb_need * (split + 1) / f.n_split) / kFsTileN * kFsTileN;
    // A operands: this wave's 16 tokens as 4 M-tiles of (4 tokens x 4 heads).
    uint4 A[4][NC];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int64_t tok = i0 + wave * 16 + mt * 4 + (c16 >> 2);
      const int h = c16 & 3;
      const bool ok = tok < f.lq && h < f.h_idx;
      const uint16_t* p = f.q_idx + (tok * f.h_idx + h) * DI + quad * 8;
#pragma unroll
      for (int c = 0; c < NC; ++c) A[mt][c] = ok ? ld16(p + c * 32) : make_uint4(0, 0, 0, 0);
    }
    uint4 stage[LPT];
    // Tile rows from a map row -> block (< 0: zero row).
    auto load_rows = [&](auto&& blk_of) {
#pragma unroll
      for (int u = 0; u < LPT; ++u) {
        const int v = threadIdx.x + 256 * u;
        const int row = v / VPR, cv = v - row * VPR;
        const int64_t blk = blk_of(row);
        stage[u] = (blk >= 0 && blk < f.nblk) ? ld16(f.kp + blk * DI + cv * 8)
                                              : make_uint4(0, 0, 0, 0);
      }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
      for (int u = 0; u < LPT; ++u) {
        const int v = threadIdx.x + 256 * u;
        const int row = v / VPR, cv = v - row * VPR;
        *reinterpret_cast<uint4*>(&tile[buf][key_tile_off<DI>(row, cv)]) = stage[u];
      }
    };
    // acc[mt][j]: token (mt, quad), tile row 4*c16 + j.
    auto multiply = [&](const uint16_t* tb, f32x4 (&acc)[4][4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 B[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c)
          B[c] = *reinterpret_cast<const uint4*>(&tb[key_tile_off<DI>(4 * c16 + j, 4 * c + quad)]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NC; ++c) acc[mt][j] = mfma_16x16x32(A[mt][c], B[c], acc[mt][j]);
        }
      }
    };

    // 1. Thresholds from a strided sample (rows whose candidates all fit admit all).
    // The sample is scored once per row tile: each piece scores its share of it.
    float thr[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (nb_need > f.cap) {
      const int64_t want = ((int64_t)f.sample_k * nb_need + f.target - 1) / f.target;
      const int S = (int)min(nb_need, (want + kFsTileN - 1) / kFsTileN * kFsTileN);
      const int n_st = (S + kFsTileN - 1) / kFsTileN;
      if constexpr (SAMPLE) {
        // sample i is block i * stride: evenly spaced over the first S * stride blocks,
        // in 32-bit arithmetic (blocks < 2^24; a 64-bit division per sample cost as much
        // as the whole scoring pass)
        const int stride = (int)(nb_need / S);
        auto sample_blk = [&](int i) -> int64_t { return i < S ? (int64_t)(i * stride) : -1; };
        const int st0 = n_st * split / f.n_split, st1 = n_st * (split + 1) / f.n_split;
        uint32_t top[4][kFsTopR];
        int nv[4] = {0, 0, 0, 0};
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int q = 0; q < kFsTopR; ++q) top[mt][q] = 0u;
        if (st0 < st1) {
          load_rows([&](int row) { return sample_blk(st0 * kFsTileN + row); });
          store_tile(0);
          __syncthreads();
        }
        for (int st = st0; st < st1; ++st) {
          const bool more = st + 1 < st1;
          if (more) load_rows([&](int row) { return sample_blk((st + 1) * kFsTileN + row); });
          f32x4 acc[4][4];
          multiply(tile[(st - st0) & 1], acc);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int64_t b = sample_blk(st * kFsTileN + 4 * c16 + j);
              if (b >= 0 && b < lim[mt]) {
                uint32_t x = order_key(score_of_heads(W[mt], acc[mt][j]));
                ++nv[mt];
#pragma unroll
                for (int q = 0; q < kFsTopR; ++q) {  // keep the kFsTopR largest, sorted
                  const uint32_t hi = max(top[mt][q], x);
                  x = min(top[mt][q], x);
                  top[mt][q] = hi;
                }
              }
            }
          if (more) store_tile((st + 1 - st0) & 1);
          __syncthreads();
        }
        static_assert(kFsTopR == 8, "two uint4 of sampled keys per lane and row");
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          if (tokv[mt] >= 0) {
            const int64_t at = ((int64_t)tokv[mt] * f.n_split + split) * kFsLanes + c16;
            f.s_top[2 * at] = make_uint4(top[mt][0], top[mt][1], top[mt][2], top[mt][3]);
            f.s_top[2 * at + 1] = make_uint4(top[mt][4], top[mt][5], top[mt][6], top[mt][7]);
            f.s_nv[at] = nv[mt];
          }
      } else {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          // This lane's kFsTopR best sampled keys over every piece's share (0: none):
          // the same keys as one pass over the whole sample would keep. Keeping only a
          // lane's best few lowers the threshold a little where a lane holds more of
          // the row's best samples; the target is set with that margin, which keeps
          // rows with fewer than m entries (each an exact fallback) rare.
          uint32_t top[kFsTopR] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
          int nv = 0;
#pragma unroll
          for (int sp = 0; sp < 4; ++sp) {
            if (sp < f.n_split && tokv[mt] >= 0) {
              const int64_t at = ((int64_t)tokv[mt] * f.n_split + sp) * kFsLanes + c16;
              const uint4 t0 = f.s_top[2 * at], t1 = f.s_top[2 * at + 1];
              nv += f.s_nv[at];
              const uint32_t ks[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                uint32_t x = ks[e];
#pragma unroll
                for (int q = 0; q < kFsTopR; ++q) {  // insert into the sorted kFsTopR best
                  const uint32_t hi = max(top[q], x);
                  x = min(top[q], x);
                  top[q] = hi;
                }
              }
            }
          }
          const int nvg = group16_sum(nv);
          int kept = 0;
#pragma unroll
          for (int q = 0; q < kFsTopR; ++q) kept += top[q] != 0u;
          kept = group16_sum(kept);
          if (lim[mt] > f.cap && kept > 0) {
            // about `target` of the lim scores reach the k-th best of the nvg sampled
            int64_t k = ((int64_t)nvg * f.target + lim[mt] - 1) / lim[mt];
            k = k < 1 ? 1 : (k > kept ? kept : k);  // fewer kept: a lower threshold
            uint32_t pre = 0u;
            for (int b = 31; b >= 0; --b) {
              const uint32_t cand = pre | (1u << b);
              int c = 0;
#pragma unroll
              for (int q = 0; q < kFsTopR; ++q) c += top[q] >= cand;
              if (group16_sum(c) >= k) pre = cand;
            }
            thr[mt] = key_to_float(pre);  // the key of a sampled score
          }
        }
      }
    }
    if constexpr (SAMPLE) return;

    // 2. The piece's scores; those at or above the threshold go to the lists. Per row:
    // the end of its candidates in this piece and its lane list (block ids < 2^24).
    int lim_p[4];
    uint2* lbase[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      lim_p[mt] = (int)min((int64_t)lim[mt], n_end);
      lbase[mt] = f.lists + ((int64_t)max(tokv[mt], 0) * f.n_split + split) * kFsLanes * f.lane_cap +
                  (int64_t)c16 * f.lane_cap;
    }
    // The smallest end over the wave's 16 rows (0 if one is past the chunk): a tile
    // below it needs no per-score range test.
    int lim_lo = min(min(lim_p[0], lim_p[1]), min(lim_p[2], lim_p[3]));
    lim_lo = min(lim_lo, __shfl_xor(lim_lo, 16, kWave));
    lim_lo = min(lim_lo, __shfl_xor(lim_lo, 32, kWave));
    lim_lo = __builtin_amdgcn_readfirstlane(lim_lo);
    const unsigned slot_max = (unsigned)f.lane_cap - 1u;
    const int n_main = (int)((n_end - n_begin + kFsTileN - 1) / kFsTileN);
    if (n_main > 0) {
      load_rows([&](int row) { return n_begin + row < n_end ? n_begin + row : (int64_t)-1; });
      store_tile(0);
      __syncthreads();
      for (int it = 0; it < n_main; ++it) {
        const int64_t n0 = n_begin + (int64_t)it * kFsTileN;
        // The next tile's loads and LDS writes run on every pass (the last one's are
        // zero rows into a buffer nothing reads): with both under one condition the
        // compiler could not tell that the writes had waited for the loads.
        load_rows([&](int row) {
          const int64_t b = n0 + kFsTileN + row;
          return b < n_end ? b : (int64_t)-1;
        });
        f32x4 acc[4][4];
        multiply(tile[it & 1], acc);
        const int blk0 = (int)n0 + 4 * c16;
        float sv[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) sv[mt][j] = score_of_heads(W[mt], acc[mt][j]);
        // The next tile goes to LDS (the other buffer, read by no wave until the
        // barrier) before the appends: loads and stores share one counter, so a wait
        // for the tile's loads placed after the appends would wait for them too.
        store_tile((it + 1) & 1);
        // An entry is the score's bits and its block id; the rank is formed when the
        // list is read, which keeps the appends (executed for nearly every slot, with
        // a few lanes active) short.
        auto append = [&](auto ranged) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            bool fl[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              fl[j] = sv[mt][j] >= thr[mt] && (!decltype(ranged)::value || blk0 + j < lim_p[mt]);
            if (fl[0] | fl[1] | fl[2] | fl[3]) {  // this lane's own list, ascending ids
              unsigned p = (unsigned)cnt[mt];
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (fl[j]) {
                  // past the capacity the count still grows (the row then takes the
                  // exact fallback) while the entry lands on the last slot
                  lbase[mt][min(p, slot_max)] =
                      make_uint2(__float_as_uint(sv[mt][j]), (unsigned)(blk0 + j));
                  ++p;
                }
              cnt[mt] = (int)p;
            }
          }
        };
        if (n0 + kFsTileN <= lim_lo)
          append(std::false_type{});
        else
          append(std::true_type{});
        __syncthreads();
      }
    }
  }
  if constexpr (!SAMPLE) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      if (tokv[mt] >= 0) f.counts[((int64_t)tokv[mt] * f.n_split + split) * kFsLanes + c16] = cnt[mt];
  }
}

__global__ __launch_bounds__(256) void list_select_kernel(FusedSelArgs f) {
  // A wave's LDS area: the radix histogram, then a bitmap of the kept ids.
  __shared__ __attribute__((aligned(16))) uint32_t area[4][kLsMapWords];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= f.lq) return;
  const int64_t own = (f.q_pos0 + row) / f.r;
  const int lim = (int)min(own, f.nblk);  // blocks < 2^24
  int32_t* srow = f.sel + row * f.n_sel;
  const int m = f.n_sel - 1;
  if (lim <= m) {  // every candidate is kept
    for (int k = lane; k < f.n_sel; k += kWave) srow[k] = k < lim ? k : (k == lim ? (int)own : -1);
    if (lane == 0) f.flags[row] = 0;
    return;
  }
  // Lane l holds the count of list l (lists: pieces x 16 lanes, <= 64).
  const int n_lists = f.n_split * kFsLanes;
  const int c = lane < n_lists ? f.counts[row * n_lists + lane] : 0;
  int incl = c;  // inclusive prefix over the lanes
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  const int total = __shfl(incl, kWave - 1, kWave);
  const bool bad = __ballot(c > f.lane_cap) != 0ull;
  if (bad || total < m || total > f.cap) {
    if (lane == 0) f.flags[row] = 1;
    return;
  }
  // Entry p of the row (slot p / 64 of lane p % 64) is entry p - start(l) of list l.
  // Each lane writes the places of its own list's entries into an LDS map (the wave's
  // area, free until the radix select), so a slot finds its entry with one LDS read;
  // every slot's load is then issued before any is used, all in flight at once.
  // Slots past the last entry hold nothing in every lane: the wave skips them.
  uint16_t* place = reinterpret_cast<uint16_t*>(area[wave]);  // < 64 * 128 places
  int cmax = c;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cmax = max(cmax, __shfl_xor(cmax, o, kWave));
  for (int i = 0; i < cmax; ++i)
    if (i < c) place[incl - c + i] = (uint16_t)(lane * f.lane_cap + i);
  wave_lds_sync();
  const uint2* lrow = f.lists + row * n_lists * (int64_t)f.lane_cap;
  const int n_slots = (total + kWave - 1) / kWave;
  uint2 ent[kLsSlots];
#pragma unroll
  for (int j = 0; j < kLsSlots; ++j) {
    ent[j] = make_uint2(0u, 0u);
    const int p = j * kWave + lane;
    if (j < n_slots && p < total) ent[j] = lrow[place[p]];
  }
  wave_lds_sync();  // the map is read before the histogram reuses the area
  uint64_t rk[kLsSlots];
#pragma unroll
  for (int j = 0; j < kLsSlots; ++j)
    rk[j] = j * kWave + lane < total ? fs_rank(__uint_as_float(ent[j].x), (int)ent[j].y) : 0ull;
  uint32_t* hist = area[wave];
  int pb;
  const uint64_t pre = wave_radix_select<kFsRankBits>(
      hist, (uint32_t)m,
      [&](auto&& fn) {
#pragma unroll
        for (int j = 0; j < kLsSlots; ++j)
          if (j < n_slots && rk[j]) fn(rk[j]);
      },
      pb);
  uint32_t kept_mask = 0u;  // bit j: slot j holds one of the m kept
#pragma unroll
  for (int j = 0; j < kLsSlots; ++j)
    if (j < n_slots && rk[j] != 0ull && (rk[j] >> (kFsRankBits - pb)) >= pre) kept_mask |= 1u << j;
  // Ascending order: the kept ids set bits of a bitmap over the row's blocks, one
  // window of kLsMapWords * 32 blocks at a time; each lane owns a run of words,
  // counts their bits, and writes its ids after those of the lanes before it.
  uint32_t* bm = area[wave];
  const int n_words = (lim + 31) >> 5;
  int written = 0;
  for (int w0 = 0; w0 < n_words; w0 += kLsMapWords) {
    const int nw = min(n_words - w0, kLsMapWords);
    const int wpl = (nw + kWave - 1) / kWave;  // words per lane
    wave_lds_sync();  // the histogram, or the last window, is no longer read
    for (int i = lane; i < nw; i += kWave) bm[i] = 0u;
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < kLsSlots; ++j)
      if (j < n_slots && (kept_mask & (1u << j))) {
        const int rel = fs_rank_id(rk[j]) - (w0 << 5);
        if (rel >= 0 && rel < (nw << 5)) atomicOr(&bm[rel >> 5], 1u << (rel & 31));
      }
    wave_lds_sync();
    const int q0 = lane * wpl, q1 = min(q0 + wpl, nw);
    int cl = 0;
    for (int q = q0; q < q1; ++q) cl += __popc(bm[q]);
    int ci = cl;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(ci, o, kWave);
      if (lane >= o) ci += y;
    }
    int pos = written + ci - cl;
    for (int q = q0; q < q1; ++q) {
      uint32_t x = bm[q];
      while (x) {
        const int b = __ffs(x) - 1;
        if (pos < m) srow[pos] = ((w0 + q) << 5) + b;
        ++pos;
        x &= x - 1u;
      }
    }
    written += __shfl(ci, kWave - 1, kWave);
  }
  for (int k = m + lane; k < f.n_sel; k += kWave) srow[k] = k == m ? (int)own : -1;
  if (lane == 0) f.flags[row] = 0;
}

__global__ __launch_bounds__(256) void fallback_select_kernel(FusedSelArgs f) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= f.lq || f.flags[row] == 0) return;
  const int64_t own = (f.q_pos0 + row) / f.r;
  const int n = (int)min(own, f.nblk);  // > m here
  const int m = f.n_sel - 1;
  const float* srow_s = f.scores + row * f.ld;
  int32_t* srow = f.sel + row * f.n_sel;
  // The row streams in chunks of 8 float4 per lane (2048 scores), every load issued
  // before any is used; loads are clamped into the row (ids >= n are absent).
  constexpr int kVec = 8;
  constexpr int kChunk = 4 * kWave * kVec;
  auto load_chunk = [&](int c0, float4 (&v)[kVec]) {
#pragma unroll
    for (int q = 0; q < kVec; ++q) {
      const int i = min(c0 + (q * kWave + lane) * 4, (n - 1) & ~3);
      v[q] = *reinterpret_cast<const float4*>(srow_s + i);
    }
  };
  int pb;
  const uint64_t pre = wave_radix_select<kFsRankBits>(
      hist[wave], (uint32_t)m,
      [&](auto&& fn) {
        for (int c0 = 0; c0 < n; c0 += kChunk) {
          float4 v[kVec];
          load_chunk(c0, v);
#pragma unroll
          for (int q = 0; q < kVec; ++q) {
            const int i = c0 + (q * kWave + lane) * 4;
            const float xs[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (i + e < n) fn(fs_rank(xs[e], i + e));
          }
        }
      },
      pb);
  uint32_t written = 0;
  for (int c0 = 0; c0 < n; c0 += kChunk) {
    float4 v[kVec];
    load_chunk(c0, v);
#pragma unroll
    for (int q = 0; q < kVec; ++q) {
      const int i = c0 + (q * kWave + lane) * 4;
      const float xs[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
      bool fl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        fl[e] = i + e < n && (fs_rank(xs[e], i + e) >> (kFsRankBits - pb)) >= pre;
      written += wave_append4(fl, written, [&](uint32_t p, int e) {
        if (p < (uint32_t)m) srow[p] = i + e;
      });
    }
  }
  for (int k = m + lane; k < f.n_sel; k += kWave) srow[k] = k == m ? (int)own : -1;
}

}  // namespace

int fused_n_split(int64_t lq) {
  const int64_t tiles = (lq + kFsRows - 1) / kFsRows;
  const int64_t ns = 512 / (tiles > 0 ? tiles : 1);
  return (int)(ns < 1 ? 1 : (ns > 4 ? 4 : ns));
}

hipError_t launch_select_fused(const FusedSelArgs& f, hipStream_t stream) {
  if (f.lq <= 0) return hipSuccess;
  if (f.n_split < 1 || f.n_split > 4 || f.cap > kFusedListCap || f.nblk >= (1 << kFsIdBits) ||
      f.target < 1 || f.sample_k < 1 || f.lane_cap < 1 ||
      (int64_t)f.n_split * kFsLanes * f.lane_cap > 65536)  // list places in 16 bits
    return hipErrorInvalidValue;
  const int64_t tiles = (f.lq + kFsRows - 1) / kFsRows;
  const dim3 g1((unsigned)tiles, (unsigned)f.n_split);
  if (f.d_idx == 128) {
    hipLaunchKernelGGL((score_list_kernel<128, true>), g1, dim3(256), 0, stream, f);
    hipLaunchKernelGGL((score_list_kernel<128, false>), g1, dim3(256), 0, stream, f);
  } else {
    hipLaunchKernelGGL((score_list_kernel<64, true>), g1, dim3(256), 0, stream, f);
    hipLaunchKernelGGL((score_list_kernel<64, false>), g1, dim3(256), 0, stream, f);
  }
  const dim3 gr((unsigned)((f.lq + 3) / 4));
  hipLaunchKernelGGL(list_select_kernel, gr, dim3(256), 0, stream, f);
  ScoreArgs sa{};
  sa.q_idx = f.q_idx;
  sa.w = f.w;
  sa.kp = f.kp;
  sa.nblk = f.nblk;
  sa.lq = f.lq;
  sa.h_idx = f.h_idx;
  sa.d_idx = f.d_idx;
  sa.r = f.r;
  sa.q_pos0 = f.q_pos0;
  sa.scores = f.scores;
  sa.ld = f.ld;
  sa.batch = 1;
  sa.row_flags = f.flags;
  const hipError_t e = launch_index_scores(sa, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fallback_select_kernel, gr, dim3(256), 0, stream, f);
  return hipGetLastError();
}

}  // namespace qsa

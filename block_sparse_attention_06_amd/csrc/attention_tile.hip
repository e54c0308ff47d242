// Stage 4 of QSA as a multi-row tile: four neighbouring query rows of one KV group
// share a workgroup, which stages the union of their kept blocks in LDS once; each
// row's wave attends over it with the blocks its row did not keep masked.
//
// Method ("Qwen3.8-Flash-Next" Miles recipe, section 1 "Model Introduction"):
// attention reads only the key tokens the indexer kept for each query. Neighbouring
// queries, and an MTP layer that reuses the main layer's selections ("On the Design of
// Qwen3.8-Next Architecture", item 2 QSA; "Qwen3.8-Flash-Next开源", section on the
// multi-token prediction module), keep many of the same blocks: a block kept by
// several rows of a tile is read from memory once for all of them.
//
// The result is that of the per-row kernel up to the order of the online softmax: a
// row still visits its kept blocks in ascending order, with the other rows' blocks in
// between as masked columns (an all-masked step changes nothing; a partly masked one
// can move the running maximum at a different step).
//
// Per workgroup (4 waves = rows i0 .. i0+3 of one KV group):
//  1. each wave copies its row's kept list into LDS (-1 padding as INT_MAX, so the
//     list stays sorted) and counts its entries;
//  2. unless the rows share too little -- 64 evenly spaced blocks of row 0 looked up in
//     row 1's list, fewer than min_shared found -- the tile builds the sorted union:
//     wave w marks the entries of its list that no lower row holds (first
//     occurrences) and prefix-counts them; a first occurrence x goes to union place
//     sum over rows of (their first occurrences below x), with the mask of the rows
//     that keep it;
//  3. the union goes through LDS 16 keys (4 blocks) at a time, double-buffered (one
//     step loading into registers, one in LDS), K and V in 16-byte chunks XOR-swizzled
//     by key; each wave reads its MFMA operands from there and runs the per-row step
//     with the blocks of other rows given id -1, which the step masks.
//  Otherwise each wave walks its own row like the per-row kernel.

#include <climits>

#include "attn_step.h"
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kTileRows = 4;
constexpr int kTileUnionMax = kTileRows * kTileMaxSel;

// First index of sorted l[0..n) whose value is not below x.
__device__ __forceinline__ int lower_bound_lds(const int32_t* l, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (l[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

template <int D>
__global__ __launch_bounds__(256, 2) void sparse_attn_tile_kernel(AttnArgs a, int min_shared) {
  constexpr int NH = D / 128;          // 128-dim halves
  constexpr int NT = D / 16;           // output dim tiles
  constexpr int NC = D / 32;           // k-chunks of Q.K^T
  constexpr int CH = D / 8;            // 16-byte chunks of a key row
  constexpr int PER = 16 * CH / 256;   // chunks of a 16-key step per thread (K and V each)
  static_assert(PER >= 1 && 16 * CH % 256 == 0, "a step's chunks spread over the threads");
  __shared__ __attribute__((aligned(16))) uint4 stage[2][2][16 * CH];  // [buffer][K, V]
  __shared__ int32_t uni[kTileUnionMax];
  __shared__ uint8_t umask[kTileUnionMax];
  __shared__ int32_t lists[kTileRows][kTileMaxSel];
  __shared__ uint16_t pref[kTileRows][kTileMaxSel + 1];
  __shared__ int cnt[kTileRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, quad = lane >> 4;
  const int G = a.hq / a.hkv;
  const int g = a.kv_group;
  const int64_t lrow = (int64_t)blockIdx.x * kTileRows + wave;
  const bool valid = lrow < a.lq;
  const int64_t row = a.row_begin + (valid ? lrow : 0);
  const int64_t t = a.q_pos0 + row;
  const int64_t kstride = (int64_t)a.hkv * D;
  const int32_t* srow = a.sel + row * a.n_sel;

  // 1. The row's kept list and its entry count (ids ascending, then -1).
  int nv = 0;
  for (int i = lane; i < kTileMaxSel; i += kWave) {
    const int x = i < a.n_sel ? srow[i] : -1;
    lists[wave][i] = x < 0 ? INT_MAX : x;
    nv += __popcll(__ballot(x >= 0));
  }
  if (lane == 0) cnt[wave] = valid ? nv : -1;
  __syncthreads();
  const bool all_valid = cnt[0] >= 0 && cnt[1] >= 0 && cnt[2] >= 0 && cnt[3] >= 0;
  bool use_union = false;
  if (all_valid) {
    if (min_shared <= 0) {
      use_union = true;
    } else {
      const int n0 = cnt[0], n1 = cnt[1];
      const int x = n0 > 0 ? lists[0][(int)((int64_t)lane * n0 / kWave)] : INT_MAX;
      const int p = lower_bound_lds(lists[1], n1, x);
      use_union = __popcll(__ballot(x != INT_MAX && p < n1 && lists[1][p] == x)) >= min_shared;
    }
  }

  uint4 Qc[NC];
  attn_load_q<D>(Qc, a.q + row * (int64_t)a.hq * D, g, G, c16, quad);
  f32x4 O[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) O[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  if (!use_union) {
    // Each wave walks its own row (no workgroup barrier from here on).
    if (!valid) return;
    const int n_steps = (a.n_sel + 3) / 4;
    for (int s = 0; s < n_steps; ++s) {
      int b4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) b4[j] = (4 * s + j < a.n_sel) ? srow[4 * s + j] : -1;
      if (b4[0] < 0) break;
      AttnStep<D> st;
      attn_load_step<D>(st, b4, b4, false, a.k, a.v, kstride, g, t, c16, quad);
      attn_compute_step<D>(st, b4, Qc, O, m_run, l_run, a.scale_log2, t, quad);
    }
  } else {
    // 2a. First occurrences of list `wave` (no lower row holds the block) and their
    // exclusive prefix counts; pref[w][i] for i >= cnt[w] is list w's total.
    const int nw = cnt[wave];
    uint32_t run = 0;
    for (int k = 0; k < kTileMaxSel / kWave; ++k) {
      const int i = k * kWave + lane;
      bool first = false;
      if (i < nw) {
        const int x = lists[wave][i];
        first = true;
        for (int r = 0; r < wave; ++r) {
          const int p = lower_bound_lds(lists[r], cnt[r], x);
          if (p < cnt[r] && lists[r][p] == x) first = false;
        }
      }
      const uint64_t b = __ballot(first);
      pref[wave][i] = (uint16_t)(run + (uint32_t)lane_prefix(b));
      run += (uint32_t)__popcll(b);
    }
    if (lane == 0) pref[wave][kTileMaxSel] = (uint16_t)run;
    __syncthreads();
    // 2b. Each first occurrence at its place in the sorted union, with its rows' mask.
    for (int k = 0; k < kTileMaxSel / kWave; ++k) {
      const int i = k * kWave + lane;
      if (i < nw && pref[wave][i + 1] != pref[wave][i]) {
        const int x = lists[wave][i];
        int pos = pref[wave][i];
        uint32_t mask = 1u << wave;
        for (int r = 0; r < kTileRows; ++r) {
          if (r == wave) continue;
          const int p = lower_bound_lds(lists[r], cnt[r], x);
          pos += pref[r][p];
          if (p < cnt[r] && lists[r][p] == x) mask |= 1u << r;
        }
        uni[pos] = x;
        umask[pos] = (uint8_t)mask;
      }
    }
    __syncthreads();
    const int total = pref[0][kTileMaxSel] + pref[1][kTileMaxSel] + pref[2][kTileMaxSel] +
                      pref[3][kTileMaxSel];
    const int n_steps = (total + 3) / 4;
    // every row of the tile is valid here: the last one has the largest position
    const int64_t t_max = a.q_pos0 + a.row_begin + (int64_t)blockIdx.x * kTileRows + kTileRows - 1;
    // Thread tid stages chunks tid + 256u (u < PER) of the step's 16 keys, K and V.
    uint4 rk[PER], rv[PER];
    auto load = [&](int s) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int e = tid + 256 * u;
        const int key = e / CH, ch = e - key * CH;
        const int slot = 4 * s + (key >> 2);
        const int id = slot < total ? uni[slot] : -1;
        const int64_t tok = id < 0 ? 0 : min((int64_t)id * 4 + (key & 3), t_max);
        const int64_t off = tok * kstride + (int64_t)g * D + ch * 8;
        rk[u] = ld16(a.k + off);
        rv[u] = ld16(a.v + off);
      }
    };
    auto store = [&](int buf) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int e = tid + 256 * u;
        const int key = e / CH, ch = e - key * CH;
        stage[buf][0][key * CH + (ch ^ key)] = rk[u];
        stage[buf][1][key * CH + (ch ^ key)] = rv[u];
      }
    };
    if (n_steps > 0) {
      load(0);
      store(0);
      if (n_steps > 1) load(1);
    }
    __syncthreads();
    for (int s = 0; s < n_steps; ++s) {
      const int buf = s & 1;
      int b4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int slot = 4 * s + q;
        b4[q] = (slot < total && ((umask[slot] >> wave) & 1)) ? uni[slot] : -1;
      }
      if (b4[0] >= 0 || b4[1] >= 0 || b4[2] >= 0 || b4[3] >= 0) {  // the row keeps one
        // The step's operands in the per-row kernel's layouts: K row c16 (key c16),
        // chunk 4c + quad; V rows of keys 4*quad + kk, chunk c16 + 16*hf.
        AttnStep<D> st;
#pragma unroll
        for (int c = 0; c < NC; ++c) st.Kc[c] = stage[buf][0][c16 * CH + ((4 * c + quad) ^ c16)];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int key = 4 * quad + kk;
#pragma unroll
          for (int hf = 0; hf < NH; ++hf)
            st.Vr[kk][hf] = stage[buf][1][key * CH + ((c16 + 16 * hf) ^ key)];
        }
        attn_compute_step<D>(st, b4, Qc, O, m_run, l_run, a.scale_log2, t, quad);
      }
      if (s + 1 < n_steps) {
        store(buf ^ 1);  // the step loaded one iteration ago, into the buffer read last
        if (s + 2 < n_steps) load(s + 2);
      }
      __syncthreads();
    }
  }

  float l_tot = wave_xor_sum(l_run, 16);
  l_tot = wave_xor_sum(l_tot, 32);
  float lh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lh[i] = __shfl(l_tot, 4 * quad + i, kWave);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hl = 4 * quad + i;
    if (hl < G) {
      const float inv = lh[i] > 0.f ? 1.f / lh[i] : 0.f;
      uint16_t* op = a.out + (row * a.hq + g * G + hl) * (int64_t)D + c16 * 8;
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        uint4 v;
        v.x = pack_bf16x2(O[hf * 8 + 0][i] * inv, O[hf * 8 + 1][i] * inv);
        v.y = pack_bf16x2(O[hf * 8 + 2][i] * inv, O[hf * 8 + 3][i] * inv);
        v.z = pack_bf16x2(O[hf * 8 + 4][i] * inv, O[hf * 8 + 5][i] * inv);
        v.w = pack_bf16x2(O[hf * 8 + 6][i] * inv, O[hf * 8 + 7][i] * inv);
        *reinterpret_cast<uint4*>(op + hf * 128) = v;
      }
    }
  }
  if (a.lse && quad == 0 && c16 < G)
    a.lse[row * a.hq + g * G + c16] = l_tot > 0.f ? m_run * kLn2 + logf(l_tot) : -INFINITY;
}

const void* sparse_attn_tile_fn(int d) {
  return d == 256 ? reinterpret_cast<const void*>(&sparse_attn_tile_kernel<256>)
                  : reinterpret_cast<const void*>(&sparse_attn_tile_kernel<128>);
}

}  // namespace

// One resident generation of tiles (4 rows each); -1 when the occupancy is unknown.
int64_t sparse_attn_tiled_rows_per_launch(int d) {
  const int64_t gen = resident_workgroups(sparse_attn_tile_fn(d), 256);
  return gen <= 0 ? -1 : gen * kTileRows;
}

// Like the per-row kernel, the tiles go to the GPU one resident generation and one KV
// group at a time (a tile holds rows of one group).
hipError_t launch_sparse_attn_fwd_tiled(const AttnArgs& a, int min_shared, hipStream_t stream) {
  if (a.lq <= 0) return hipSuccess;
  if (a.n_sel > kTileMaxSel || a.hq / a.hkv > 16 || a.cu_q || (a.d != 128 && a.d != 256))
    return hipErrorInvalidValue;
  const int64_t gen = sparse_attn_tiled_rows_per_launch(a.d);
  const int64_t rows = gen <= 0 ? a.lq : gen;
  for (int gp = 0; gp < a.hkv; ++gp) {
    for (int64_t c0 = 0; c0 < a.lq; c0 += rows) {
      AttnArgs c = a;
      c.lq = a.lq - c0 < rows ? a.lq - c0 : rows;
      c.row_begin = a.row_begin + c0;
      c.kv_group = gp;
      const dim3 grid((unsigned)((c.lq + kTileRows - 1) / kTileRows));
      if (a.d == 256)
        hipLaunchKernelGGL(sparse_attn_tile_kernel<256>, grid, dim3(256), 0, stream, c, min_shared);
      else
        hipLaunchKernelGGL(sparse_attn_tile_kernel<128>, grid, dim3(256), 0, stream, c, min_shared);
    }
  }
  return hipGetLastError();
}

}  // namespace qsa

// Stage 4 of QSA: exact softmax attention restricted to the kept tokens.
//
// Method ("Qwen3.8-Flash-Next" Miles recipe, section 1 "Model Introduction"):
// attention reads only the key tokens the indexer kept for each query; the
// selection rows are built before the kernel, which needs no causal or segment
// logic of its own beyond masking keys after the query inside its own block. GQA:
// 24 query heads in 2 KV groups, head dim 256 (same section); THD tensors
// (section 5.3).
//
// Work decomposition: one wave per (query token, KV group). The wave keeps the
// group's <= 16 query heads in registers and walks the row's kept blocks 4 at a
// time (16 keys); the kept blocks of neighbouring queries differ, so each wave
// gathers its own K/V (K through a wave-private LDS tile, see attn_load_k_staged) with
// no cross-wave synchronisation. Blocks that many rows keep are shared
// through L2 instead: the launcher starts the rows one resident generation at a
// time, so that rows in flight walk their ascending block lists in step, and one KV
// group at a time, so that the group's K/V stays in the last-level cache.
//
//   S^T[16 keys x 16 heads] = K[16 x d] . Q^T        8 x v_mfma_f32_16x16x32_bf16
//     lane l: key row (l%16) -> 16 B of that key; output: head (l%16), keys 4*(l/16)+i
//   O[16 heads x d] += P[16 x 16 keys] . V[16 keys x d]   d/16 x v_mfma_f32_16x16x16_bf16
//     the S^T output layout is exactly the A-operand layout of P, so P never moves;
//     the B operand needs 4 keys of one dim per lane, which a row-major V does not
//     give. Instead the output columns are permuted: in dim-tile n, column c stands
//     for dim (n/8)*128 + 8c + n%8, so each lane loads 16 contiguous bytes (8 dims)
//     of each of its 4 keys and repacks them in registers (v_perm), and at the end
//     each lane again owns 8 contiguous dims per head: 16-byte output stores.
// Softmax: fp32, base-2 with the scale folded in, running max per head shared by
// the 4 lanes that hold the head's keys, per-lane partial sums reduced at the end.
// Decode splits each sequence's kept blocks over waves, merges the four waves of a
// workgroup in LDS and writes (m, l, o) partials that a second kernel combines.

#include <mutex>
#include <tuple>
#include <vector>

#include "attn_step.h"
#include "qsa_device.h"
#include "qsa_internal.h"
#include "qsa_wave.h"

namespace qsa {

// Prefill: one wave per (query row, KV group) walks the row's kept blocks.
// K rows of one step through a wave-private LDS tile. Loaded straight into the MFMA
// A-operand layout, each K load instruction touches 16 key rows for 64 B apiece (half
// a cache line each); loaded here two whole rows (four lines) an instruction, K costs
// the L1 half the line accesses, and the operands are read back from LDS (chunks
// XOR-swizzled by row, conflict-free both ways). Where the K/V fit the last-level
// cache the L1's line accesses, not the misses, bound the call: on MI355X at 128K
// 38.8 -> 38.3 ms on random selections and 37.4 -> 29.6 ms on token-correlated ones,
// 32K 9.0 -> 7.8 ms, 16 packed prompts 36.4 -> 29.4 ms. Beyond it (8192 rows over 1M
// keys) the misses go to HBM and the LDS hop only adds latency (4.33 -> 4.54 ms): such
// sequences load K straight into the operands.
template <int D>
__device__ __forceinline__ void attn_load_k_staged(AttnStep<D>& st, const int (&b4)[4],
                                                   const uint16_t* kb, int64_t kstride, int g,
                                                   int64_t t, int lane) {
  constexpr int CH = D / 8;     // 16-byte chunks of a key row
  constexpr int RPI = 64 / CH;  // rows per load instruction
  constexpr int KI = 16 / RPI;  // load instructions for the step's 16 keys
  static_assert(KI <= D / 32, "the loaded chunks land in the operand registers");
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int row = i * RPI + lane / CH, ch = lane % CH;  // key row = 4 * slot + token
    const int b = pick4(b4[0], b4[1], b4[2], b4[3], row >> 2);
    const int64_t tk = attn_row(b, b, row & 3, t, false);
    st.Kc[i] = ld16(kb + tk * kstride + g * D + ch * 8);
  }
}

template <int D>
__device__ __forceinline__ void attn_k_from_lds(AttnStep<D>& st, uint4* kst, int lane, int c16,
                                                int quad) {
  constexpr int CH = D / 8, RPI = 64 / CH, KI = 16 / RPI;
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int row = i * RPI + lane / CH, ch = lane % CH;
    kst[row * CH + (ch ^ row)] = st.Kc[i];
  }
  wave_lds_sync();
  // A operand of k-chunk c: key row c16, dims 32c + 8 quad .. + 7. All chunks are read
  // before the first product uses one (the barrier keeps the compiler from
  // interleaving each read with its product, which serialised eight LDS round trips).
#pragma unroll
  for (int c = 0; c < D / 32; ++c) st.Kc[c] = kst[c16 * CH + ((4 * c + quad) ^ c16)];
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, bool KLDS>
__global__ __launch_bounds__(256) void sparse_attn_kernel(AttnArgs a) {
  constexpr int NH = D / 128;  // 128-dim halves
  constexpr int NT = D / 16;   // output dim tiles
  __shared__ __attribute__((aligned(16))) uint4 kst_all[4][KLDS ? 16 * (D / 8) : 1];  // K tiles
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int G = a.hq / a.hkv;

  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  const int64_t lrow = a.kv_group >= 0 ? item : item / a.hkv;
  const int g = a.kv_group >= 0 ? a.kv_group : (int)(item - lrow * a.hkv);
  if (lrow >= a.lq) return;
  const int64_t row = a.row_begin + lrow;      // row of q, sel, out and lse
  const int64_t kstride = (int64_t)a.hkv * D;  // elements between consecutive tokens
  const uint16_t* kb = a.k;
  const uint16_t* vb = a.v;
  int64_t t = a.q_pos0 + row;
  if (a.cu_q) {
    // Packed sequences: the row's sequence is the last one starting at or before it.
    int lo = 0, hi = a.batch_vl;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_q[mid] <= row) lo = mid; else hi = mid;
    }
    const int64_t q0 = a.cu_q[lo], q1 = a.cu_q[lo + 1];
    const int64_t k0 = a.cu_k[lo], k1 = a.cu_k[lo + 1];
    t = (k1 - k0) - (q1 - q0) + (row - q0);
    kb += k0 * kstride;
    vb += k0 * kstride;
  }
  const int n_steps = (a.n_sel + 3) / 4;
  const int32_t* srow = a.sel + row * a.n_sel;

  uint4 Qc[D / 32];
  attn_load_q<D>(Qc, a.q + row * (int64_t)a.hq * D, g, G, c16, quad);

  f32x4 O[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) O[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max (log2 domain) of head c16
  float l_run = 0.f;        // this lane's partial sum for head c16

  // A step's four block ids are read one step ahead (uniform: scalar loads), 16 bytes
  // at once when the rows are 16-byte aligned, so no id load waits at the top of a
  // step. With the K operands read from LDS in one batch (attn_k_from_lds), at 128K on
  // MI355X: 38.4 -> 37.8 ms on random selections, 29.6 -> 27.2 ms on token-correlated
  // ones, 32K 7.5 -> 7.2 ms, 8192 rows over 1M keys 4.24 -> 4.18 ms. Outputs are
  // bit-identical.
  const bool ids4 = (a.n_sel & 3) == 0 && (reinterpret_cast<uintptr_t>(a.sel) & 15) == 0;
  auto read_ids = [&](int s, int (&b)[4]) {
    if (ids4 && s < n_steps) {
      const int4 v = *reinterpret_cast<const int4*>(srow + 4 * s);
      b[0] = v.x; b[1] = v.y; b[2] = v.z; b[3] = v.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = (4 * s + j < a.n_sel) ? srow[4 * s + j] : -1;
    }
  };
  int nb4[4];
  read_ids(0, nb4);
  for (int s = 0; s < n_steps; ++s) {
    int b4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b4[j] = nb4[j];
    if (b4[0] < 0) break;  // -1 padding reached
    read_ids(s + 1, nb4);
    AttnStep<D> st;
    if constexpr (KLDS) {
      attn_load_k_staged<D>(st, b4, kb, kstride, g, t, lane);
      attn_load_v<D>(st, b4, b4, false, vb, kstride, g, t, c16, quad);
      attn_k_from_lds<D>(st, kst_all[wave], lane, c16, quad);
    } else {
      attn_load_step<D>(st, b4, b4, false, kb, vb, kstride, g, t, c16, quad);
    }
    attn_compute_step<D>(st, b4, Qc, O, m_run, l_run, a.scale_log2, t, quad);
    if constexpr (KLDS) wave_lds_sync();  // the tile is read before the next step's K
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

// Decode: a workgroup per (sequence, KV group, range of 4*SPS steps); each wave takes
// SPS consecutive steps. The wave reads all its block ids first (they are uniform:
// scalar loads) and keeps two steps' loads in flight. The four waves then merge
// their (m, l, O) in LDS, so one partial per workgroup and head goes to memory for
// the combine kernel.
template <int D, int SPS>
__global__ __launch_bounds__(256) void sparse_attn_decode_kernel(AttnArgs a) {
  constexpr int NH = D / 128;
  constexpr int NT = D / 16;
  constexpr int kMaxG = 16;
  __shared__ float red_o[4][kMaxG][D];
  __shared__ float red_ml[4][kMaxG][2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int G = a.hq / a.hkv;

  const int64_t wg = blockIdx.x;  // (row, g, wg_split)
  const int64_t per_seq = (int64_t)a.hkv * a.n_split;
  const int64_t row = wg / per_seq;
  if (row >= a.lq) return;
  const int rem = (int)(wg - row * per_seq);
  const int g = rem / a.n_split;
  const int wg_split = rem - g * a.n_split;
  const int64_t t = (int64_t)a.seq_lens[row] - 1;
  const bool paged = a.block_table != nullptr;
  const uint16_t* kb = paged ? a.k : a.k + row * a.cache_bs;
  const uint16_t* vb = paged ? a.v : a.v + row * a.cache_bs;
  const int32_t* srow = a.sel + row * a.n_sel;
  const int64_t kstride = (int64_t)a.hkv * D;
  const int s_begin = (wg_split * 4 + wave) * SPS;

  // ids: the kept blocks; pids: where their rows sit (paged: page from the block table,
  // clamped to the table and the pool, times blocks per page, plus the block's offset).
  int ids[SPS][4], pids[SPS][4];
#pragma unroll
  for (int si = 0; si < SPS; ++si)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = 4 * (s_begin + si) + j;
      ids[si][j] = (t >= 0 && k < a.n_sel) ? srow[k] : -1;
      pids[si][j] = ids[si][j];
    }
  if (paged) {
    const int32_t* trow = a.block_table + row * a.table_stride;
    const int pb = a.page_blocks;
#pragma unroll
    for (int si = 0; si < SPS; ++si)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = ids[si][j];
        if (b >= 0) {
          const int pi = b / pb;
          int pg = trow[pi < a.table_stride ? pi : a.table_stride - 1];
          pg = pg < 0 ? 0 : (pg < a.num_pages ? pg : a.num_pages - 1);
          pids[si][j] = pg * pb + (b - pi * pb);
        }
      }
  }

  uint4 Qc[D / 32];
  attn_load_q<D>(Qc, a.q + row * (int64_t)a.hq * D, g, G, c16, quad);
  f32x4 O[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) O[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Loads are issued for every step (padding reads an in-bounds row); a step whose
  // first block is padding is skipped (the padding is at the end of the row).
  AttnStep<D> A, B;
  attn_load_step<D>(A, ids[0], pids[0], paged, kb, vb, kstride, g, t, c16, quad);
#pragma unroll
  for (int si = 0; si < SPS; si += 2) {
    if (si + 1 < SPS)
      attn_load_step<D>(B, ids[si + 1], pids[si + 1], paged, kb, vb, kstride, g, t, c16,
                        quad);
    if (ids[si][0] >= 0)
      attn_compute_step<D>(A, ids[si], Qc, O, m_run, l_run, a.scale_log2, t, quad);
    if (si + 2 < SPS)
      attn_load_step<D>(A, ids[si + 2], pids[si + 2], paged, kb, vb, kstride, g, t, c16,
                        quad);
    if (si + 1 < SPS && ids[si + 1][0] >= 0)
      attn_compute_step<D>(B, ids[si + 1], Qc, O, m_run, l_run, a.scale_log2, t, quad);
  }

  float l_tot = wave_xor_sum(l_run, 16);
  l_tot = wave_xor_sum(l_tot, 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hl = 4 * quad + i;
    if (hl < G) {
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        float* dst = &red_o[wave][hl][hf * 128 + c16 * 8];
        *reinterpret_cast<float4*>(dst) =
            make_float4(O[hf * 8 + 0][i], O[hf * 8 + 1][i], O[hf * 8 + 2][i], O[hf * 8 + 3][i]);
        *reinterpret_cast<float4*>(dst + 4) =
            make_float4(O[hf * 8 + 4][i], O[hf * 8 + 5][i], O[hf * 8 + 6][i], O[hf * 8 + 7][i]);
      }
    }
  }
  if (quad == 0 && c16 < G) {
    red_ml[wave][c16][0] = m_run;
    red_ml[wave][c16][1] = l_tot;
  }
  __syncthreads();
  // Merge the four waves' partials: rescale to the common max (a wave without keys
  // has m = -inf and contributes nothing).
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, dim = idx - h * D;
    float M = red_ml[0][h][0];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, red_ml[w][h][0]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = red_ml[w][h][0];
      const float f = mw > -INFINITY ? exp2f(mw - M) : 0.f;
      o += f * red_o[w][h][dim];
      L += f * red_ml[w][h][1];
    }
    const int64_t slot = (row * a.hq + g * G + h) * (int64_t)a.n_split + wg_split;
    a.part_o[slot * D + dim] = o;
    if (dim == 0) {
      a.part_ml[slot * 2 + 0] = M;
      a.part_ml[slot * 2 + 1] = L;
    }
  }
}

// Combine the decode partials of one (sequence, head): rescale each split's
// (m, l, o) to the common max and normalise. The loads of the first 16 partial
// outputs of column `dim` are issued together with the (m, l) loads (thread s holds
// split s's; n_split <= D), so the common case takes one round trip to memory.
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(AttnArgs a) {
  constexpr int NW = D / 64;
  constexpr int kEarly = 16;
  __shared__ float wgt[D];
  __shared__ float red[2][NW];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = a.n_split;
  const float* po = a.part_o + bh * ns * D + tid;
  float x[kEarly];
#pragma unroll
  for (int u = 0; u < kEarly; ++u) x[u] = u < ns ? po[(int64_t)u * D] : 0.f;
  const float* ml = a.part_ml + bh * ns * 2;
  float ms = -INFINITY, ls = 0.f;
  if (tid < ns) {
    ms = ml[2 * tid];
    ls = ml[2 * tid + 1];
  }
  float M = ms;
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) M = fmaxf(M, __shfl_xor(M, d, 64));
  if (lane == 0) red[0][wave] = M;
  __syncthreads();
  M = red[0][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, red[0][w]);
  const float ws = ms > -INFINITY ? exp2f(ms - M) : 0.f;
  wgt[tid] = ws;
  float L = ws * ls;
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) L += __shfl_xor(L, d, 64);
  if (lane == 0) red[1][wave] = L;
  __syncthreads();
  L = red[1][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) L += red[1][w];
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < kEarly; ++u)
    if (u < ns) acc += wgt[u] * x[u];
  for (int s = kEarly; s < ns; ++s) acc += wgt[s] * po[(int64_t)s * D];
  const float o = L > 0.f ? acc / L : 0.f;
  a.out[bh * D + tid] = (uint16_t)(pack_bf16x2(o, 0.f) & 0xffffu);
  if (a.lse && tid == 0) a.lse[bh] = L > 0.f ? M * kLn2 + logf(L) : -INFINITY;
}

// Workgroups of `kernel` (block_threads threads, no dynamic LDS) that the current
// device holds at once: compute units x workgroups per unit, cached per kernel and
// device; 0 when the runtime cannot say.
int resident_workgroups(const void* kernel, int block_threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::mutex mu;
  static std::vector<std::tuple<const void*, int, int>> cache;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& e : cache)
    if (std::get<0>(e) == kernel && std::get<1>(e) == dev) return std::get<2>(e);
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, 0) !=
          hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  cache.emplace_back(kernel, dev, cus * per_cu);
  return cus * per_cu;
}

namespace {

// Both variants hold the same workgroups at once (registers bound them; the K tiles
// take 32 KB of LDS a workgroup at d = 256); the staged one is asked.
const void* sparse_attn_fn(int d) {
  return d == 256 ? reinterpret_cast<const void*>(&sparse_attn_kernel<256, true>)
                  : reinterpret_cast<const void*>(&sparse_attn_kernel<128, true>);
}

}  // namespace

// One resident generation of 256-thread workgroups of 4 waves, each wave one row of
// the launch's KV group; -1 when the occupancy is unknown.
int64_t sparse_attn_fwd_rows_per_launch(int hkv, int d) {
  (void)hkv;
  const int64_t gen = resident_workgroups(sparse_attn_fn(d), 256);
  if (gen <= 0) return -1;
  return gen * 4;
}

// K/V bytes of a sequence above which the rows are launched one KV group at a time.
constexpr int64_t kGroupOrderBytes = (int64_t)128 << 20;

// The rows are launched one generation at a time (as many workgroups as the device
// holds at once) and, when a sequence's K/V outgrow half the 256 MB last-level cache
// (MALL), one KV group at a time.
// - Generations: rows that start together walk their ascending kept-block lists at
//   the same pace, so a block that several of them kept is read by all of them within
//   a short time and comes from L2 after the first read. In one grid over all rows
//   the resident workgroups drift apart as they finish at different times, and such
//   blocks come from beyond L2 again. At 128K tokens (24/2 heads, d=256, K=2048) on
//   MI355X: one grid 66.8 ms, L2 hit rate 10 %; generations of 512 workgroups
//   44.1 ms, L2 hit rate 53 %, half the bytes fetched.
// - One group at a time: a group's K and V of a 128K context take 128 MB, which the
//   MALL keeps across the generations, while both groups' 256 MB do not, and a
//   generation then holds twice the rows of one group: 44.0 ms with the two groups of
//   a row in one generation, 39.2 ms group by group (L2 hit rate 71 %). Packed short
//   sequences (whose K/V fit the cache either way) keep the two groups together:
//   36.9 against 37.9 ms for 16 prompts of 2K-24K tokens. For packed sequences the
//   size is that of the longest sequence when the caller knows it (a chunk of new
//   rows after a long cached prefix then runs group by group), else it is estimated
//   from the average sequence (rows / sequences).
// Each row's sums run in the same order either way, so the outputs are identical.
namespace {

bool fwd_by_group(int64_t keys, int hkv, int d) {
  return keys * hkv * d * 4 > kGroupOrderBytes;  // K and V, bf16
}

// K through LDS while a sequence's K and V fit the 256 MB last-level cache.
constexpr int64_t kStagedKBytes = (int64_t)256 << 20;
bool fwd_k_staged(int64_t keys, int hkv, int d) { return keys * hkv * d * 4 <= kStagedKBytes; }

// Rows per launch: a generation of (row, group) waves, one group or all of a row's.
int64_t fwd_launch_rows(int64_t lq, bool by_group, int hkv, int d) {
  const int64_t gen_rows = sparse_attn_fwd_rows_per_launch(hkv, d);
  return gen_rows <= 0 ? lq : (by_group ? gen_rows : (gen_rows + hkv - 1) / hkv);
}

}  // namespace

int64_t sparse_attn_fwd_launches(int64_t lq, int64_t keys, int hkv, int d) {
  if (lq <= 0) return 0;
  const bool by_group = fwd_by_group(keys, hkv, d);
  const int64_t rows = fwd_launch_rows(lq, by_group, hkv, d);
  return (by_group ? hkv : 1) * ((lq + rows - 1) / rows);
}

hipError_t launch_sparse_attn_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.lq <= 0) return hipSuccess;
  const int64_t keys =
      a.keys_hint > 0 ? a.keys_hint
                      : (a.cu_q ? a.lq / (a.batch_vl > 0 ? a.batch_vl : 1) : a.lk);
  const bool by_group = fwd_by_group(keys, a.hkv, a.d);
  const bool staged = fwd_k_staged(keys, a.hkv, a.d);
  const int64_t rows = fwd_launch_rows(a.lq, by_group, a.hkv, a.d);
  for (int gp = 0; gp < (by_group ? a.hkv : 1); ++gp) {
    for (int64_t c0 = 0; c0 < a.lq; c0 += rows) {
      AttnArgs c = a;
      c.lq = a.lq - c0 < rows ? a.lq - c0 : rows;
      c.row_begin = a.row_begin + c0;
      c.kv_group = by_group ? gp : -1;
      const dim3 grid((unsigned)((c.lq * (by_group ? 1 : a.hkv) + 3) / 4));
      if (a.d == 256) {
        if (staged) hipLaunchKernelGGL((sparse_attn_kernel<256, true>), grid, dim3(256), 0, stream, c);
        else hipLaunchKernelGGL((sparse_attn_kernel<256, false>), grid, dim3(256), 0, stream, c);
      } else {
        if (staged) hipLaunchKernelGGL((sparse_attn_kernel<128, true>), grid, dim3(256), 0, stream, c);
        else hipLaunchKernelGGL((sparse_attn_kernel<128, false>), grid, dim3(256), 0, stream, c);
      }
    }
  }
  return hipGetLastError();
}

// Decode splits: a wave takes SPS steps of 4 blocks (SPS = 1, 2 or 4, so that about
// 64 waves share a (sequence, KV group)), a workgroup 4 waves; n_split counts the
// workgroups (= partials) per (sequence, head).
int decode_steps_per_split(int n_sel) {
  const int steps = (n_sel + 3) / 4;
  return steps <= 64 ? 1 : (steps <= 128 ? 2 : 4);
}

int decode_num_splits(int n_sel) {
  const int steps = (n_sel + 3) / 4;
  const int sps = decode_steps_per_split(n_sel);
  const int waves = (steps + sps - 1) / sps;
  return (waves + 3) / 4;
}

hipError_t launch_sparse_attn_decode(const AttnArgs& a, hipStream_t stream) {
  if (a.lq <= 0) return hipSuccess;
  // combine: a partial per thread; merge in LDS: at most 16 heads per group
  if (a.n_split < 1 || a.n_split > a.d || a.hq / a.hkv > 16) return hipErrorInvalidValue;
  const int sps = a.steps_per_split;
  if ((int64_t)a.n_split * 4 * sps * 4 < a.n_sel) return hipErrorInvalidValue;  // ranges cover n_sel
  const dim3 grid((unsigned)(a.lq * a.hkv * a.n_split));
  const dim3 cgrid((unsigned)(a.lq * a.hq));
#define QSA_DECODE_LAUNCH(DD, S) \
  hipLaunchKernelGGL((sparse_attn_decode_kernel<DD, S>), grid, dim3(256), 0, stream, a)
  if (a.d == 256) {
    if (sps == 1) QSA_DECODE_LAUNCH(256, 1);
    else if (sps == 2) QSA_DECODE_LAUNCH(256, 2);
    else if (sps == 4) QSA_DECODE_LAUNCH(256, 4);
    else return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_combine_kernel<256>), cgrid, dim3(256), 0, stream, a);
  } else {
    if (sps == 1) QSA_DECODE_LAUNCH(128, 1);
    else if (sps == 2) QSA_DECODE_LAUNCH(128, 2);
    else if (sps == 4) QSA_DECODE_LAUNCH(128, 4);
    else return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_combine_kernel<128>), cgrid, dim3(128), 0, stream, a);
  }
#undef QSA_DECODE_LAUNCH
  return hipGetLastError();
}

}  // namespace qsa

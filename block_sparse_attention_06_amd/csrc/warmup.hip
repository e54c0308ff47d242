// Indexer warm-up: KL distillation of the full attention onto the block scores.
//
// Method ("On the Design of Qwen3.8-Next Architecture", four architecture
// components, item 2 QSA): before sparse training the indexer is warmed up by
// distilling the full attention distribution, max-pooled to the block level, into it
// with a KL loss. Readings: the heads' probabilities are summed, the target lives on
// the blocks the indexer scores (complete blocks before the own block) and is
// normalised there, the indexer's distribution is the softmax of its scores over the
// same blocks, the loss is KL(target || indexer) per query row, and the target is a
// constant.
//
// Kernels:
//  * kl_split_kernel / kl_dense_kernel <TARGET = false>: dense causal lse of every
//    (query row, head); <TARGET = true>: per scored block, the max over its 4 keys of
//    the head-summed probabilities exp(S - lse) (unnormalised). Both walk the keys in
//    steps shared by a workgroup's rows through LDS (S = Q.K^T on
//    v_mfma_f32_16x16x32_bf16); the split kernel (up to 2 KV groups) gives each group
//    its own waves, the dense one (3 or 4 groups) keeps a row's groups in one wave.
//  * kl_loss_kernel: one workgroup per row: normalises the target, the scores'
//    log-softmax, the KL value and dL/ds = softmax(s) - target, sums in fp64.
//  * index_scores_bwd_dq_kernel / _dk_kernel: the gradients of the scores with
//    respect to q_idx and w (row-major: z^T = kbar.q^T puts dz in the A layout of
//    dq = dz.kbar) and to the pooled keys (block-major: z = q.kbar^T puts dz in the A
//    layout of dkbar = dz^T.q), each recomputing z, no atomics; the pooling's
//    gradient spreads dkbar / r over each block's tokens.

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr float kLog2eW = 1.4426950408889634f;
constexpr float kLn2W = 0.6931471805599453f;

__device__ __forceinline__ uint32_t w_half(uint32_t w, int hi) {
  return hi ? (w >> 16) : (w & 0xffffu);
}
__device__ __forceinline__ uint32_t w_word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
// B operand of a 16x16x16 MFMA from 4 rows (k) of 8 consecutive bf16: column e packs
// element e of the 4 rows.
__device__ __forceinline__ uint2 w_repack(const uint4 (&r)[4], int e) {
  const int wi = e >> 1, hi = e & 1;
  const uint32_t lo = w_half(w_word(r[0], wi), hi) | (w_half(w_word(r[1], wi), hi) << 16);
  const uint32_t up = w_half(w_word(r[2], wi), hi) | (w_half(w_word(r[3], wi), hi) << 16);
  return make_uint2(lo, up);
}

}  // namespace

// ---- dense passes over shared key tiles --------------------------------------------------
//
// Both passes read every key before the query. A workgroup of 8 waves takes 8 * RPW
// consecutive query rows (RPW per wave, all KV groups of a row in one wave, so the
// target's head sum stays in the wave) and walks the keys its rows need in steps of KS:
// the step's keys (every group) are loaded once, cooperatively, into a double-buffered
// LDS tile, two steps ahead in registers, and every wave reads them from there as the
// B operand of S = Q.K^T for each of its rows. The lse pass keeps the online max and
// sum of every (row, head); the target pass sums exp(S - lse) over the heads and takes
// the max over each block's 4 keys.

constexpr int kKlWaves = 8;
// Start of the running max: finite, so that x - m is never inf - inf, and far below any
// score, so that 2^(m - x) is 0 for the first real one.
constexpr float kKlNoMax = -1e30f;

template <int D, bool TARGET, int KS, int NG, int RPW>
__global__ __launch_bounds__(512) void kl_dense_kernel(KlArgs a) {
  constexpr int NC = D / 32;
  constexpr int VPR = D / 8;     // 16-byte vectors of one key row of one group
  constexpr int KROW = VPR + 1;  // padded LDS row
  constexpr int TILE_ROWS = kKlWaves * RPW;
  constexpr int LPT = (KS * NG * VPR + 511) / 512;  // 16-byte loads per thread per step
  __shared__ uint4 kt[2][NG][KS][KROW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int H = a.hkv;
  const int G = a.hq / H;
  const bool hv = c16 < G;  // the Q operand's row c16 is a head of the group
  const int64_t row0 = (int64_t)blockIdx.x * TILE_ROWS;
  const int64_t t_last = a.q_pos0 + min(row0 + TILE_ROWS, a.lq) - 1;
  // Keys the workgroup needs: 0..t_last (lse), or the last row's scored blocks (target).
  const int64_t kend = TARGET ? min(t_last / a.r, a.nblk) * a.r : t_last + 1;
  if (kend <= 0) return;
  const int nsteps = (int)((kend + KS - 1) / KS);
  const int64_t kstride = (int64_t)H * D;

  int64_t row[RPW], lim[RPW];  // lim: the row's keys are 0 .. lim-1
  bool rv[RPW];
  uint4 Qc[RPW][NG][NC];
  float L2v[RPW][NG][4], m_run[RPW][NG][4], l_run[RPW][NG][4];  // heads 4*quad + i
#pragma unroll
  for (int p = 0; p < RPW; ++p) {
    row[p] = row0 + wave * RPW + p;
    rv[p] = row[p] < a.lq;
    const int64_t t = a.q_pos0 + (rv[p] ? row[p] : 0);
    lim[p] = !rv[p] ? 0 : (TARGET ? min(t / a.r, a.nblk) * a.r : t + 1);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const bool ok = rv[p] && hv && g < H;
      const uint16_t* qp =
          a.q + ((rv[p] ? row[p] : 0) * a.hq + (g < H ? g : 0) * G + (hv ? c16 : 0)) * (int64_t)D +
          quad * 8;
#pragma unroll
      for (int c = 0; c < NC; ++c) Qc[p][g][c] = ok ? ld16(qp + c * 32) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * quad + i;
        L2v[p][g][i] = !TARGET ? 0.f
                       : (rv[p] && g < H && h < G) ? a.lse[row[p] * a.hq + g * G + h] * kLog2eW
                                                   : INFINITY;
        m_run[p][g][i] = kKlNoMax;
        l_run[p][g][i] = 0.f;
      }
    }
  }

  // Step loads: vector e = (key, group, v) of the 16 keys, every group.
  auto issue = [&](uint4 (&R)[LPT], int s) {
#pragma unroll
    for (int l = 0; l < LPT; ++l) {
      const int e = tid + 512 * l;
      const int key = e / (NG * VPR), g = (e / VPR) % NG, v = e % VPR;
      const int64_t j = min((int64_t)s * KS + key, kend - 1);
      // Unconditional (a group past the last reads the last one, never used), so that
      // the waits count loads exactly.
      R[l] = ld16(a.k + j * kstride + min(g, H - 1) * D + v * 8);
    }
  };
  auto store = [&](const uint4 (&R)[LPT], int slot) {
#pragma unroll
    for (int l = 0; l < LPT; ++l) {
      const int e = tid + 512 * l;
      const int key = e / (NG * VPR), g = (e / VPR) % NG, v = e % VPR;
      if (e < KS * NG * VPR) kt[slot][g][key][v] = R[l];
    }
  };
  // S = Q.K^T on the same operands (heads as MFMA rows, keys as columns): lane c16
  // holds key j0 + c16, rows 4*quad + i are the heads. The lse pass keeps running
  // (max, sum) per lane and head over the lane's keys (no cross-lane work per step);
  // the target pass sums a lane's heads in registers, then across the quads, and takes
  // each block's max over 4 neighbouring lanes.
  auto compute = [&](int s, int slot) {
#pragma unroll
    for (int u = 0; u < KS / 16; ++u) {
      const int64_t j0 = (int64_t)s * KS + u * 16;
      const int64_t key = j0 + c16;
      float acc[RPW];
#pragma unroll
      for (int p = 0; p < RPW; ++p) acc[p] = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g >= H) break;
        uint4 Kc[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) Kc[c] = kt[slot][g][u * 16 + c16][quad + 4 * c];
#pragma unroll
        for (int p = 0; p < RPW; ++p) {
          if (j0 >= lim[p]) continue;
          f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NC; ++c) S = mfma_16x16x32(Qc[p][g][c], Kc[c], S);
          if constexpr (TARGET) {
            // Padding heads carry L2 = +inf, so they add exp2(-inf) = 0.
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[p] += __builtin_amdgcn_exp2f(S[i] * a.scale_log2 - L2v[p][g][i]);
          } else {
            // Online (max, sum) with one exponential per score: e = 2^-|x - m| is the
            // factor for the old sum when x is the new max, else the new term.
            const bool kok = key < lim[p];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x = kok ? S[i] * a.scale_log2 : -INFINITY;
              const float dlt = x - m_run[p][g][i];
              const float e = __builtin_amdgcn_exp2f(-fabsf(dlt));
              const bool up = dlt > 0.f;
              l_run[p][g][i] = up ? fmaf(l_run[p][g][i], e, 1.f) : l_run[p][g][i] + e;
              m_run[p][g][i] = up ? x : m_run[p][g][i];
            }
          }
        }
      }
      if constexpr (TARGET) {
#pragma unroll
        for (int p = 0; p < RPW; ++p) {
          if (j0 >= lim[p]) continue;
          float v = key < lim[p] ? acc[p] : 0.f;
          v += __shfl_xor(v, 16, 64);
          v += __shfl_xor(v, 32, 64);  // key j0 + c16, summed over every head
          v = fmaxf(v, __shfl_xor(v, 1, 64));
          v = fmaxf(v, __shfl_xor(v, 2, 64));  // max over the block's 4 keys
          const int64_t b = key / 4;
          if (quad == 0 && (c16 & 3) == 0 && b * a.r < lim[p]) a.target[row[p] * a.ld + b] = v;
        }
      }
    }
  };

  // Two steps of loads in flight: unconditional (past the end they repeat the last
  // step), so that every wait is for exactly one step's loads.
  uint4 R0[LPT], R1[LPT];
  issue(R0, 0);
  issue(R1, min(1, nsteps - 1));
  store(R0, 0);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    issue(R0, min(s + 2, nsteps - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(s, 0);
    if (s + 1 < nsteps) store(R1, 1);
    __syncthreads();
    if (s + 1 >= nsteps) break;
    issue(R1, min(s + 3, nsteps - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(s + 1, 1);
    if (s + 2 < nsteps) store(R0, 0);
    __syncthreads();
  }

  if constexpr (!TARGET) {
    // Combine the 16 key lanes' (max, sum) of each head.
#pragma unroll
    for (int p = 0; p < RPW; ++p)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g >= H) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float m = m_run[p][g][i], l = l_run[p][g][i];
#pragma unroll
          for (int dd = 1; dd < 16; dd <<= 1) {
            const float mo = __shfl_xor(m, dd, 64), lo = __shfl_xor(l, dd, 64);
            const float mn = fmaxf(m, mo);
            l = l * exp2f(m - mn) + lo * exp2f(mo - mn);
            m = mn;
          }
          const int h = 4 * quad + i;
          if (rv[p] && c16 == 0 && h < G) a.lse[row[p] * a.hq + g * G + h] = m * kLn2W + logf(l);
        }
      }
  }
}

// ---- KL loss and score gradient -------------------------------------------------------

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, 64);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ double block_max_f64(double v, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) v = fmax(v, __shfl_xor(v, d, 64));
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
}

__global__ __launch_bounds__(256) void kl_loss_kernel(KlLossArgs a) {
  __shared__ double red[4];
  const int64_t row = blockIdx.x;
  const int64_t t = a.q_pos0 + row;
  const int64_t n = min(t / a.r, a.nblk);
  const float* s = a.scores + row * a.ld;
  const float* p = a.target + row * a.ld;
  float* ds = a.dscores + row * a.ld;
  if (n <= 0) {
    if (threadIdx.x == 0) a.loss[row] = 0.f;
    return;
  }
  double smax = -INFINITY, psum = 0.0;
  for (int64_t b = threadIdx.x; b < n; b += 256) {
    smax = fmax(smax, (double)s[b]);
    psum += (double)p[b];
  }
  smax = block_max_f64(smax, red);
  psum = block_sum_f64(psum, red);
  double esum = 0.0, plogp = 0.0, ps = 0.0;
  for (int64_t b = threadIdx.x; b < n; b += 256) {
    const double sb = s[b], pb = p[b];
    esum += exp(sb - smax);
    if (pb > 0.0) plogp += pb * log(pb);
    ps += pb * sb;
  }
  esum = block_sum_f64(esum, red);
  plogp = block_sum_f64(plogp, red);
  ps = block_sum_f64(ps, red);
  const double lse = smax + log(esum);
  // sum_b (p_b / P) (log(p_b / P) - (s_b - lse)), P = sum_b p_b
  if (threadIdx.x == 0) a.loss[row] = (float)(plogp / psum - log(psum) - ps / psum + lse);
  for (int64_t b = threadIdx.x; b < n; b += 256)
    ds[b] = (float)(exp((double)s[b] - lse) - (double)p[b] / psum);
}

// ---- indexer backward -----------------------------------------------------------------

// Rows (token, head): 4 tokens x 4 heads per wave (heads >= H_I are zero). Over the
// row's scored blocks in tiles of 16: z^T = kbar.q^T (A = pooled keys, B = q), so a
// lane holds (token, head) c16 and blocks 4*quad + i; dz = ds w [z > 0] is then the
// A operand of dq = dz.kbar (16x16x16, k = blocks), B = 4 pooled keys x 8 dims.
template <int DI>
__global__ __launch_bounds__(256) void index_scores_bwd_dq_kernel(IdxBwdArgs a) {
  constexpr int NC = DI / 32;
  constexpr int NT = 8;  // output tiles: dims 8*c16 + e (c16 < DI / 8)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int64_t tok0 = ((int64_t)blockIdx.x * 4 + wave) * 4;
  if (tok0 >= a.lq) return;
  // This lane's B column / A... (token, head) = c16.
  const int64_t tok = tok0 + (c16 >> 2);
  const int h = c16 & 3;
  const bool rv = tok < a.lq && h < a.h_idx;
  uint4 Qc[NC];
  {
    const uint16_t* qp = a.q_idx + ((rv ? tok : 0) * a.h_idx + (rv ? h : 0)) * DI + quad * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) Qc[c] = rv ? ld16(qp + c * 32) : make_uint4(0, 0, 0, 0);
  }
  const float wv = rv ? a.w[tok * a.h_idx + h] : 0.f;
  const int64_t own = rv ? min((a.q_pos0 + tok) / a.r, a.nblk) : 0;
  // The wave walks blocks up to the largest own block of its 4 tokens.
  const int64_t tl = min(tok0 + 3, a.lq - 1);
  const int64_t own_max = min((a.q_pos0 + tl) / a.r, a.nblk);
  const int n_tiles = (int)((own_max + 15) / 16);
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dw = 0.f;
  const float* dsrow = a.dscores + (rv ? tok : 0) * a.ld;
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int64_t b0 = (int64_t)tile * 16;
    // A: pooled key b0 + c16; B: (token, head) c16.
    const int64_t bk = min(b0 + c16, a.nblk - 1);
    const uint16_t* kp = a.kp + bk * DI + quad * 8;
    f32x4 Z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) Z = mfma_16x16x32(ld16(kp + c * 32), Qc[c], Z);
    // ds of blocks b0 + 4*quad + i for this lane's token (in-bounds: ld >= nblk and
    // ld % 4 == 0, blocks past the row's own are masked).
    const int64_t bq = b0 + 4 * quad;
    float4 g4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (rv && bq < own) g4 = *reinterpret_cast<const float4*>(dsrow + bq);
    const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
    float dz[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = rv && bq + i < own;
      const float gi = ok ? gs[i] : 0.f;
      dw += gi * fmaxf(Z[i], 0.f);
      dz[i] = Z[i] > 0.f ? gi * wv : 0.f;
    }
    const uint2 A = make_uint2(pack_bf16x2(dz[0], dz[1]), pack_bf16x2(dz[2], dz[3]));
    // B: pooled keys b0 + 4*quad + kk, dims 8*c16 .. 8*c16 + 7.
    uint4 Kr[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int64_t b = min(bq + kk, a.nblk - 1);
      Kr[kk] = c16 < DI / 8 ? ld16(a.kp + b * DI + c16 * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < NT; ++e) acc[e] = mfma_16x16x16(A, w_repack(Kr, e), acc[e]);
  }
  dw = wave_xor_sum(dw, 16);
  dw = wave_xor_sum(dw, 32);
  if (quad == 0 && rv) a.dw[tok * a.h_idx + h] = dw;
  // acc[e][i]: row (token, head) 4*quad + i, dim 8*c16 + e.
  if (c16 < DI / 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * quad + i;
      const int64_t tk = tok0 + (rr >> 2);
      const int hh = rr & 3;
      if (tk < a.lq && hh < a.h_idx) {
        float* op = a.dq_idx + (tk * a.h_idx + hh) * DI + c16 * 8;
        *reinterpret_cast<float4*>(op) = make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
        *reinterpret_cast<float4*>(op + 4) =
            make_float4(acc[4][i], acc[5][i], acc[6][i], acc[7][i]);
      }
    }
  }
}

// Block-major: a workgroup owns 16 pooled keys; its 4 waves split the query rows that
// score any of them, 4 tokens (16 (token, head) rows) per step, wave v taking steps v,
// v + 4, ... : z = q.kbar^T (A = q, B = pooled keys), so a lane holds block c16 and rows
// 4*quad + i (token quad's heads); dz is the A operand of dkbar = dz^T.q (k = rows), B =
// the token's 4 heads x 8 dims. Every load is unconditional (clamped rows, heads and
// dims meet dz = 0 or are never stored) and a wave's next step is loaded before the
// current one is multiplied. The 4 partial sums are added in LDS in a fixed order.
template <int DI>
__global__ __launch_bounds__(256) void index_scores_bwd_dk_kernel(IdxBwdArgs a) {
  constexpr int NC = DI / 32;
  constexpr int NT = 8;
  __shared__ float part[3][NT * 4][64];  // waves 1..3: acc[e][i] of each lane
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int64_t b0 = (int64_t)blockIdx.x * 16;
  if (b0 >= a.nblk) return;  // uniform over the workgroup
  const int64_t blk = b0 + c16;
  const bool bv = blk < a.nblk;
  const int64_t blk_c = bv ? blk : a.nblk - 1;
  uint4 Kc[NC];
  {
    const uint16_t* kp = a.kp + blk_c * DI + quad * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) Kc[c] = ld16(kp + c * 32);
  }
  // Rows that score block b0: t / r > b0, i.e. t >= r * (b0 + 1).
  const int64_t t_first = (int64_t)a.r * (b0 + 1);
  const int64_t tok_base = max((int64_t)0, t_first - a.q_pos0) / 4 * 4;
  const int64_t n_steps = a.lq > tok_base ? (a.lq - tok_base + 3) / 4 : 0;
  const int hmax = a.h_idx - 1;
  const int dmax = DI / 8 - 1;

  struct In {
    uint4 Aq[NC];  // q of (token tok0 + (c16 >> 2), head c16 & 3), dims quad*8 + 32c
    uint4 Qr[4];   // q of (token tok0 + quad, head kk), dims 8*c16 ..
    float g, w[4];
  };
  auto fetch = [&](In& in, int64_t s) {
    const int64_t tok0 = tok_base + 4 * s;
    const int64_t tka = min(tok0 + (c16 >> 2), a.lq - 1);
    const uint16_t* qp = a.q_idx + (tka * a.h_idx + min(c16 & 3, hmax)) * DI + quad * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) in.Aq[c] = ld16(qp + c * 32);
    const int64_t tk = min(tok0 + quad, a.lq - 1);
    in.g = a.dscores[tk * a.ld + blk_c];
#pragma unroll
    for (int i = 0; i < 4; ++i) in.w[i] = a.w[tk * a.h_idx + min(i, hmax)];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      in.Qr[kk] = ld16(a.q_idx + (tk * a.h_idx + min(kk, hmax)) * DI + min(c16, dmax) * 8);
  };
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](const In& in, int64_t s) {
    f32x4 Z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) Z = mfma_16x16x32(in.Aq[c], Kc[c], Z);
    // Output rows 4*quad + i: token tok0 + quad, head i; column c16: block blk.
    const int64_t tk = tok_base + 4 * s + quad;
    const bool tv = tk < a.lq;
    const int64_t own = tv ? min((a.q_pos0 + tk) / a.r, a.nblk) : 0;
    const float g = (tv && bv && blk < own) ? in.g : 0.f;
    float dz[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) dz[i] = (Z[i] > 0.f && i < a.h_idx) ? g * in.w[i] : 0.f;
    const uint2 A = make_uint2(pack_bf16x2(dz[0], dz[1]), pack_bf16x2(dz[2], dz[3]));
#pragma unroll
    for (int e = 0; e < NT; ++e) acc[e] = mfma_16x16x16(A, w_repack(in.Qr, e), acc[e]);
  };
  In i0, i1;
  fetch(i0, wave);
  fetch(i1, wave + 4);
  for (int64_t s = wave; s < n_steps; s += 8) {
    step(i0, s);
    fetch(i0, s + 8);
    __builtin_amdgcn_sched_barrier(0);
    if (s + 4 < n_steps) step(i1, s + 4);
    fetch(i1, s + 12);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < NT; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wave - 1][e * 4 + i][lane] = acc[e][i];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int e = 0; e < NT; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[e][i] += part[w][e * 4 + i][lane];
  // acc[e][i]: block b0 + 4*quad + i, dim 8*c16 + e.
  if (c16 < DI / 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t b = b0 + 4 * quad + i;
      if (b < a.nblk) {
        float* op = a.dk_pooled + b * DI + c16 * 8;
        *reinterpret_cast<float4*>(op) = make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
        *reinterpret_cast<float4*>(op + 4) =
            make_float4(acc[4][i], acc[5][i], acc[6][i], acc[7][i]);
      }
    }
  }
}

// The same passes with the KV groups split over the waves (up to 2 groups): 8 / H waves
// per group, 4 rows each, so a workgroup takes 4 * 8 / H rows and a wave reads only its
// own group's keys from the shared tile, each key fragment serving 4 rows (the kernel
// above reads both groups' keys for 2 rows). The target pass adds the groups' head
// sums through LDS: every wave parks its per-(row, key) sums, and after the step's
// barrier the waves of group 0 add them up and take each block's max.
template <int D, bool TARGET, int KS, int H>
__global__ __launch_bounds__(512) void kl_split_kernel(KlArgs a) {
  constexpr int NC = D / 32;
  constexpr int VPR = D / 8;
  constexpr int KROW = VPR + 1;
  constexpr int RPW = 4;
  constexpr int WPG = kKlWaves / H;     // waves per group
  constexpr int TILE_ROWS = WPG * RPW;  // rows per workgroup
  constexpr int LPT = (KS * H * VPR + 511) / 512;
  __shared__ uint4 kt[2][H][KS][KROW];
  __shared__ float xch[2][H][TARGET ? TILE_ROWS : 1][TARGET ? KS : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int grp = wave / WPG, wr = wave % WPG;
  const int G = a.hq / H;
  const bool hv = c16 < G;  // the Q operand's row c16 is a head of the group
  const int64_t row0 = (int64_t)blockIdx.x * TILE_ROWS;
  const int64_t t_last = a.q_pos0 + min(row0 + TILE_ROWS, a.lq) - 1;
  const int64_t kend = TARGET ? min(t_last / a.r, a.nblk) * a.r : t_last + 1;
  if (kend <= 0) return;
  const int nsteps = (int)((kend + KS - 1) / KS);
  const int64_t kstride = (int64_t)H * D;

  int64_t row[RPW], lim[RPW];
  bool rv[RPW];
  uint4 Qc[RPW][NC];
  float L2v[RPW][4], m_run[RPW][4], l_run[RPW][4];  // heads 4*quad + i
#pragma unroll
  for (int p = 0; p < RPW; ++p) {
    row[p] = row0 + wr * RPW + p;
    rv[p] = row[p] < a.lq;
    const int64_t t = a.q_pos0 + (rv[p] ? row[p] : 0);
    lim[p] = !rv[p] ? 0 : (TARGET ? min(t / a.r, a.nblk) * a.r : t + 1);
    const bool ok = rv[p] && hv;
    const uint16_t* qp =
        a.q + ((rv[p] ? row[p] : 0) * a.hq + grp * G + (hv ? c16 : 0)) * (int64_t)D + quad * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) Qc[p][c] = ok ? ld16(qp + c * 32) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * quad + i;
      L2v[p][i] = !TARGET ? 0.f
                  : (rv[p] && h < G) ? a.lse[row[p] * a.hq + grp * G + h] * kLog2eW : INFINITY;
      m_run[p][i] = kKlNoMax;
      l_run[p][i] = 0.f;
    }
  }

  auto issue = [&](uint4 (&R)[LPT], int s) {
#pragma unroll
    for (int l = 0; l < LPT; ++l) {
      const int e = tid + 512 * l;
      const int key = e / (H * VPR), g = (e / VPR) % H, v = e % VPR;
      const int64_t j = min((int64_t)s * KS + min(key, KS - 1), kend - 1);
      R[l] = ld16(a.k + j * kstride + g * D + v * 8);
    }
  };
  auto store = [&](const uint4 (&R)[LPT], int slot) {
#pragma unroll
    for (int l = 0; l < LPT; ++l) {
      const int e = tid + 512 * l;
      const int key = e / (H * VPR), g = (e / VPR) % H, v = e % VPR;
      if (e < KS * H * VPR) kt[slot][g][key][v] = R[l];
    }
  };
  auto compute = [&](int s, int slot) {
#pragma unroll
    for (int u = 0; u < KS / 16; ++u) {
      const int64_t j0 = (int64_t)s * KS + u * 16;
      const int64_t key = j0 + c16;
      uint4 Kc[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) Kc[c] = kt[slot][grp][u * 16 + c16][quad + 4 * c];
#pragma unroll
      for (int p = 0; p < RPW; ++p) {
        float acc = 0.f;
        if (j0 < lim[p]) {
          f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NC; ++c) S = mfma_16x16x32(Qc[p][c], Kc[c], S);
          if constexpr (TARGET) {
            // Padding heads carry L2 = +inf, so they add exp2(-inf) = 0.
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc += __builtin_amdgcn_exp2f(S[i] * a.scale_log2 - L2v[p][i]);
          } else {
            // One exponential per score: e = 2^-|x - m| is the old sum's factor when x
            // is the new max, else the new term.
            const bool kok = key < lim[p];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x = kok ? S[i] * a.scale_log2 : -INFINITY;
              const float dlt = x - m_run[p][i];
              const float e = __builtin_amdgcn_exp2f(-fabsf(dlt));
              const bool up = dlt > 0.f;
              l_run[p][i] = up ? fmaf(l_run[p][i], e, 1.f) : l_run[p][i] + e;
              m_run[p][i] = up ? x : m_run[p][i];
            }
          }
        }
        if constexpr (TARGET) {
          float v = key < lim[p] ? acc : 0.f;
          v += __shfl_xor(v, 16, 64);
          v += __shfl_xor(v, 32, 64);  // key j0 + c16, summed over the group's heads
          if (quad == 0) xch[slot][grp][wr * RPW + p][u * 16 + c16] = v;
        }
      }
    }
  };
  // After the step's barrier: the group-0 waves add the groups' sums of their rows (row
  // wr * 4 + quad) and write each scored block's max over its 4 keys.
  auto finalize = [&](int s, int slot) {
    if constexpr (TARGET) {
      if (grp != 0) return;
      const int lr = wr * RPW + quad;
      const int64_t rq = row0 + lr;
      const int64_t lq_ = quad == 0 ? lim[0] : (quad == 1 ? lim[1] : (quad == 2 ? lim[2] : lim[3]));
#pragma unroll
      for (int u = 0; u < KS / 16; ++u) {
        const int64_t key = (int64_t)s * KS + u * 16 + c16;
        float v = xch[slot][0][lr][u * 16 + c16];
        if (H == 2) v += xch[slot][H - 1][lr][u * 16 + c16];
        v = fmaxf(v, __shfl_xor(v, 1, 64));
        v = fmaxf(v, __shfl_xor(v, 2, 64));  // max over the block's 4 keys
        const int64_t b = key / 4;
        if ((c16 & 3) == 0 && rq < a.lq && b * a.r < lq_) a.target[rq * a.ld + b] = v;
      }
    }
  };

  uint4 R0[LPT], R1[LPT];
  issue(R0, 0);
  issue(R1, min(1, nsteps - 1));
  store(R0, 0);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    issue(R0, min(s + 2, nsteps - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(s, 0);
    if (s + 1 < nsteps) store(R1, 1);
    __syncthreads();
    finalize(s, 0);
    if (s + 1 >= nsteps) break;
    issue(R1, min(s + 3, nsteps - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(s + 1, 1);
    if (s + 2 < nsteps) store(R0, 0);
    __syncthreads();
    finalize(s + 1, 1);
  }

  if constexpr (!TARGET) {
#pragma unroll
    for (int p = 0; p < RPW; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = m_run[p][i], l = l_run[p][i];
#pragma unroll
        for (int dd = 1; dd < 16; dd <<= 1) {
          const float mo = __shfl_xor(m, dd, 64), lo = __shfl_xor(l, dd, 64);
          const float mn = fmaxf(m, mo);
          l = l * exp2f(m - mn) + lo * exp2f(mo - mn);
          m = mn;
        }
        const int h = 4 * quad + i;
        if (rv[p] && c16 == 0 && h < G) a.lse[row[p] * a.hq + grp * G + h] = m * kLn2W + logf(l);
      }
  }
}

// dk_idx[j] = dk_pooled[j / r] / r for tokens of complete blocks, 0 for the rest.
__global__ __launch_bounds__(256) void pool_keys_bwd_kernel(IdxBwdArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = a.n_tokens * a.d_idx;
  if (i >= n) return;
  const int64_t tokn = i / a.d_idx, c = i - tokn * a.d_idx;
  const int64_t b = tokn / a.r;
  a.dk_idx[i] = b < a.nblk ? a.dk_pooled[b * a.d_idx + c] / (float)a.r : 0.f;
}

// ---- host side ------------------------------------------------------------------------

namespace {

// Both passes of one shape: rows per workgroup = 8 waves * RPW.
template <int D, int KS, int NG, int RPW>
void launch_kl_pair(const KlArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.lq + kKlWaves * RPW - 1) / (kKlWaves * RPW)));
  hipLaunchKernelGGL((kl_dense_kernel<D, false, KS, NG, RPW>), grid, dim3(512), 0, stream, a);
  hipLaunchKernelGGL((kl_dense_kernel<D, true, KS, NG, RPW>), grid, dim3(512), 0, stream, a);
}

// Both passes with the groups split over the waves: rows per workgroup = 4 * 8 / H.
template <int D, int KS, int H>
void launch_kl_split(const KlArgs& a, hipStream_t stream) {
  constexpr int rows = 4 * kKlWaves / H;
  const dim3 grid((unsigned)((a.lq + rows - 1) / rows));
  hipLaunchKernelGGL((kl_split_kernel<D, false, KS, H>), grid, dim3(512), 0, stream, a);
  hipLaunchKernelGGL((kl_split_kernel<D, true, KS, H>), grid, dim3(512), 0, stream, a);
}

}  // namespace

hipError_t launch_kl_target(const KlArgs& a, hipStream_t stream) {
  if (a.lq <= 0) return hipSuccess;
  if (a.hkv > kKlMaxGroups) return hipErrorInvalidValue;
  // Up to 2 groups: 2 rows per wave, 32 keys per step; 3 or 4 groups: 1 row per wave
  // (the same Q registers), 16 keys per step (the same LDS).
  if (a.hkv <= 2) {
    if (a.hkv == 2) {
      if (a.d == 256) launch_kl_split<256, 32, 2>(a, stream);
      else launch_kl_split<128, 32, 2>(a, stream);
    } else {
      if (a.d == 256) launch_kl_split<256, 32, 1>(a, stream);
      else launch_kl_split<128, 32, 1>(a, stream);
    }
  } else {
    if (a.d == 256) launch_kl_pair<256, 16, 4, 1>(a, stream);
    else launch_kl_pair<128, 16, 4, 1>(a, stream);
  }
  return hipGetLastError();
}

hipError_t launch_kl_loss(const KlLossArgs& a, hipStream_t stream) {
  if (a.lq <= 0) return hipSuccess;
  hipLaunchKernelGGL(kl_loss_kernel, dim3((unsigned)a.lq), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_index_scores_bwd(const IdxBwdArgs& a, hipStream_t stream) {
  if (a.lq > 0) {
    const dim3 gq((unsigned)((a.lq + 15) / 16));
    if (a.d_idx == 128)
      hipLaunchKernelGGL(index_scores_bwd_dq_kernel<128>, gq, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(index_scores_bwd_dq_kernel<64>, gq, dim3(256), 0, stream, a);
  }
  if (a.nblk > 0) {
    const dim3 gk((unsigned)((a.nblk + 15) / 16));
    if (a.d_idx == 128)
      hipLaunchKernelGGL(index_scores_bwd_dk_kernel<128>, gk, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(index_scores_bwd_dk_kernel<64>, gk, dim3(256), 0, stream, a);
  }
  if (a.dk_idx && a.n_tokens > 0) {
    const int64_t n = a.n_tokens * a.d_idx;
    hipLaunchKernelGGL(pool_keys_bwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, a);
  }
  return hipGetLastError();
}

}  // namespace qsa

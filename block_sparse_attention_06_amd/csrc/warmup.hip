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
//  * kl_lse_kernel: dense causal lse of every (query row, head), one wave per (row,
//    KV group) over keys 0..t in tiles of 16 (S^T = K.Q^T on v_mfma_f32_16x16x32_bf16,
//    online max and sum as in the sparse forward), two tiles in flight.
//  * kl_target_kernel: one wave per row over the keys of its scored blocks: both
//    groups' probabilities, summed over the heads (a reduction across the 16 lanes of
//    a quad group), then the max over each block's 4 keys; writes the unnormalised
//    pooled values.
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

// ---- dense lse ------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void kl_lse_kernel(KlArgs a) {
  constexpr int NC = D / 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int G = a.hq / a.hkv;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  const int64_t row = item / a.hkv;
  const int g = (int)(item - row * a.hkv);
  if (row >= a.lq) return;
  const int64_t t = a.q_pos0 + row;
  const int64_t kstride = (int64_t)a.hkv * D;
  const bool hv = c16 < G;
  uint4 Qc[NC];
  {
    const uint16_t* qp = a.q + (row * a.hq + g * G + (hv ? c16 : 0)) * (int64_t)D + quad * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) Qc[c] = hv ? ld16(qp + c * 32) : make_uint4(0, 0, 0, 0);
  }
  const int n_tiles = (int)(t / 16) + 1;  // keys 0..t
  auto load = [&](uint4 (&K)[NC], int tile) {
    const int64_t j = min((int64_t)tile * 16 + c16, t);  // past t: an in-bounds row, masked
    const uint16_t* kp = a.k + j * kstride + g * D + quad * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) K[c] = ld16(kp + c * 32);
  };
  float m_run = -INFINITY, l_run = 0.f;
  auto step = [&](const uint4 (&K)[NC], int tile) {
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) S = mfma_16x16x32(K[c], Qc[c], S);
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = ((int64_t)tile * 16 + 4 * quad + i <= t) ? S[i] * a.scale_log2 : -INFINITY;
    float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mt = wave_xor_max(mt, 16);
    mt = wave_xor_max(mt, 32);
    const float m_new = fmaxf(m_run, mt);  // finite: key tile*16 <= t is never masked
    l_run = l_run * exp2f(m_run - m_new) + (exp2f(x[0] - m_new) + exp2f(x[1] - m_new)) +
            (exp2f(x[2] - m_new) + exp2f(x[3] - m_new));
    m_run = m_new;
  };
  uint4 K0[NC], K1[NC];
  load(K0, 0);
  for (int tile = 0; tile < n_tiles; tile += 2) {
    load(K1, min(tile + 1, n_tiles - 1));
    __builtin_amdgcn_sched_barrier(0);
    step(K0, tile);
    load(K0, min(tile + 2, n_tiles - 1));
    __builtin_amdgcn_sched_barrier(0);
    if (tile + 1 < n_tiles) step(K1, tile + 1);
  }
  float l_tot = wave_xor_sum(l_run, 16);
  l_tot = wave_xor_sum(l_tot, 32);
  if (quad == 0 && hv) a.lse[row * a.hq + g * G + c16] = m_run * kLn2W + logf(l_tot);
}

// ---- pooled target --------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void kl_target_kernel(KlArgs a) {
  constexpr int NC = D / 32;
  constexpr int kMaxGroups = 2;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int G = a.hq / a.hkv;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= a.lq) return;
  const int64_t t = a.q_pos0 + row;
  const int64_t own = min(t / a.r, a.nblk);  // scored blocks 0 .. own-1
  if (own <= 0) return;
  const int64_t kstride = (int64_t)a.hkv * D;
  const bool hv = c16 < G;
  float* trow = a.target + row * a.ld;
  const int n_tiles = (int)((own + 3) / 4);  // 16 keys = 4 blocks per tile
  for (int g0 = 0; g0 < a.hkv; g0 += kMaxGroups) {
    const int ng = min(kMaxGroups, a.hkv - g0);
    uint4 Qc[kMaxGroups][NC];
    float L2[kMaxGroups];
#pragma unroll
    for (int gi = 0; gi < kMaxGroups; ++gi) {
      const int g = g0 + (gi < ng ? gi : 0);
      const bool ok = hv && gi < ng;
      const uint16_t* qp = a.q + (row * a.hq + g * G + (hv ? c16 : 0)) * (int64_t)D + quad * 8;
#pragma unroll
      for (int c = 0; c < NC; ++c) Qc[gi][c] = ok ? ld16(qp + c * 32) : make_uint4(0, 0, 0, 0);
      L2[gi] = ok ? a.lse[row * a.hq + g * G + c16] * kLog2eW : 0.f;
    }
    for (int tile = 0; tile < n_tiles; ++tile) {
      const int64_t j = (int64_t)tile * 16 + c16;  // key row of this lane
      const int64_t jc = min(j, own * a.r - 1);
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int gi = 0; gi < kMaxGroups; ++gi) {
        if (gi >= ng) break;
        const uint16_t* kp = a.k + jc * kstride + (g0 + gi) * D + quad * 8;
        f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) S = mfma_16x16x32(ld16(kp + c * 32), Qc[gi][c], S);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = hv && (int64_t)tile * 16 + 4 * quad + i < own * a.r;
          acc[i] += ok ? exp2f(S[i] * a.scale_log2 - L2[gi]) : 0.f;
        }
      }
      // Sum over the heads (the 16 lanes of this quad group), then the max over the
      // block's 4 keys: block 4*tile + quad.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) acc[i] += __shfl_xor(acc[i], d, 64);
      }
      const float mx = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
      const int64_t b = (int64_t)tile * 4 + quad;
      if (c16 == 0 && b < own) trow[b] = g0 == 0 ? mx : trow[b] + mx;
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

// Block-major: a wave owns 16 pooled keys and walks the query rows that score any of
// them, 4 tokens (16 (token, head) rows) at a time: z = q.kbar^T (A = q, B = pooled
// keys), so a lane holds block c16 and rows 4*quad + i (token quad's heads); dz is the
// A operand of dkbar = dz^T.q (k = rows), B = the token's 4 heads x 8 dims.
template <int DI>
__global__ __launch_bounds__(256) void index_scores_bwd_dk_kernel(IdxBwdArgs a) {
  constexpr int NC = DI / 32;
  constexpr int NT = 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int64_t b0 = ((int64_t)blockIdx.x * 4 + wave) * 16;
  if (b0 >= a.nblk) return;
  const int64_t blk = b0 + c16;
  const bool bv = blk < a.nblk;
  uint4 Kc[NC];
  {
    const uint16_t* kp = a.kp + (bv ? blk : 0) * DI + quad * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) Kc[c] = bv ? ld16(kp + c * 32) : make_uint4(0, 0, 0, 0);
  }
  // Rows that score block b0: t / r > b0, i.e. t >= r * (b0 + 1).
  const int64_t t_first = (int64_t)a.r * (b0 + 1);
  const int64_t tok_begin = max((int64_t)0, t_first - a.q_pos0);
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t tok0 = tok_begin / 4 * 4; tok0 < a.lq; tok0 += 4) {
    // A: row c16 = (token tok0 + (c16 >> 2), head c16 & 3).
    const int64_t tka = tok0 + (c16 >> 2);
    const int ha = c16 & 3;
    const bool ra = tka < a.lq && ha < a.h_idx;
    const uint16_t* qp =
        a.q_idx + ((ra ? tka : 0) * a.h_idx + (ra ? ha : 0)) * DI + quad * 8;
    f32x4 Z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c)
      Z = mfma_16x16x32(ra ? ld16(qp + c * 32) : make_uint4(0, 0, 0, 0), Kc[c], Z);
    // Output rows 4*quad + i: token tok0 + quad, head i; column c16: block blk.
    const int64_t tk = tok0 + quad;
    const bool tv = tk < a.lq;
    const int64_t own = tv ? min((a.q_pos0 + tk) / a.r, a.nblk) : 0;
    const float g = (tv && bv && blk < own) ? a.dscores[tk * a.ld + blk] : 0.f;
    float dz[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float wi = (tv && i < a.h_idx) ? a.w[tk * a.h_idx + i] : 0.f;
      dz[i] = Z[i] > 0.f ? g * wi : 0.f;
    }
    const uint2 A = make_uint2(pack_bf16x2(dz[0], dz[1]), pack_bf16x2(dz[2], dz[3]));
    // B: token tok0 + quad, heads kk (k = rows 4*quad + kk), dims 8*c16 .. + 7.
    uint4 Qr[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bool ok = tv && kk < a.h_idx && c16 < DI / 8;
      Qr[kk] = ok ? ld16(a.q_idx + (tk * a.h_idx + kk) * DI + c16 * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < NT; ++e) acc[e] = mfma_16x16x16(A, w_repack(Qr, e), acc[e]);
  }
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

hipError_t launch_kl_target(const KlArgs& a, hipStream_t stream) {
  if (a.lq <= 0) return hipSuccess;
  const dim3 g1((unsigned)((a.lq * a.hkv + 3) / 4));
  const dim3 g2((unsigned)((a.lq + 3) / 4));
  if (a.d == 256) {
    hipLaunchKernelGGL(kl_lse_kernel<256>, g1, dim3(256), 0, stream, a);
    hipLaunchKernelGGL(kl_target_kernel<256>, g2, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(kl_lse_kernel<128>, g1, dim3(256), 0, stream, a);
    hipLaunchKernelGGL(kl_target_kernel<128>, g2, dim3(256), 0, stream, a);
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
    const dim3 gk((unsigned)((a.nblk + 63) / 64));
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

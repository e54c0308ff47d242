// Stages 1 and 2 of QSA: micro-block mean pooling of the indexer keys and the light
// MQA indexer's block scores.
//
// Method ("On the Design of Qwen3.8-Next Architecture", four architecture
// components, item 2 QSA): indexer keys are mean-pooled over micro-blocks of r = 4
// tokens and the indexer, with 4 MQA query heads, rates every block. Score reading
// (DeepSeek-DSA-style light indexer, which the page says QSA follows):
//   s[t][b] = sum_h w[t][h] * max(0, q_idx[t][h] . kbar[b]),  b < t / r.

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

// ------------------------------------------------------------------------------------
// Stage 1: pooling. One thread per (block, 8 consecutive dims). The r bf16 keys are
// summed in fp64 in token order (exact for bf16 inputs of any ordinary range),
// divided by r, and rounded once to bf16, nearest-even.
// ------------------------------------------------------------------------------------

__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  if (x == 0.0) return (__double_as_longlong(x) >> 48) & 0x8000u;
  int ex;
  frexp(x, &ex);                         // |x| = m * 2^ex, 0.5 <= m < 1
  const int qe = max(ex - 8, -133);      // exponent of the bf16 spacing at x
  const double y = ldexp(rint(ldexp(x, -qe)), qe);  // rint: ties to even
  return __float_as_uint((float)y) >> 16;  // y is exact in bf16, hence in fp32
}

__global__ __launch_bounds__(256) void pool_keys_kernel(const uint16_t* __restrict__ k,
                                                        int64_t ks, int64_t nb, int d, int r,
                                                        uint16_t* __restrict__ p, int64_t ps) {
  const int vec = d >> 3;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = gid / vec;
  if (b >= nb) return;
  const int c = (int)(gid - b * vec) * 8;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int j = 0; j < r; ++j) {
    const uint4 x = ld16(k + (b * r + j) * ks + c);
    const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += (double)bf16_bits_to_f32(w4[e] & 0xffffu);
      acc[2 * e + 1] += (double)bf16_bits_to_f32(w4[e] >> 16);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = f64_to_bf16_bits(acc[2 * e] / r) | (f64_to_bf16_bits(acc[2 * e + 1] / r) << 16);
  *reinterpret_cast<uint4*>(p + b * ps + c) = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_pool_keys(const uint16_t* k_idx, int64_t k_stride, int64_t n_blocks, int d_idx,
                            int r, uint16_t* k_pooled, int64_t p_stride, hipStream_t stream) {
  if (n_blocks <= 0) return hipSuccess;
  const int64_t threads = n_blocks * (d_idx / 8);
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(pool_keys_kernel, dim3((unsigned)grid), dim3(256), 0, stream, k_idx,
                     k_stride, n_blocks, d_idx, r, k_pooled, p_stride);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// Stage 2: block scores as a bf16 MFMA GEMM with a fused epilogue.
//
// Rows of the GEMM are (token, indexer head) pairs, 4 per token (heads >= H_I are
// zero rows), so with v_mfma_f32_16x16x32_bf16 the 4 heads of one token land in one
// lane's 4 accumulators and the weighted ReLU sum over heads is register-local.
// Workgroup: 4 waves x 16 tokens = 64 query rows; it walks its range of blocks in
// tiles of 64 pooled keys, double-buffered in LDS (one barrier per tile), each wave
// keeping its queries in registers. Columns are permuted so that within a tile, MFMA
// column c of sub-tile j is block 4c + j: each lane then owns 4 consecutive blocks
// of a token and writes them as one 16-byte store (a full 256-byte line per token per
// tile). Causal skipping: the workgroup stops at the last block any of its rows
// needs; stores wholly past a row's own block are skipped (the rest of a 16-byte
// store past the own block carries unspecified values, never read).
// ------------------------------------------------------------------------------------

constexpr int kScoreRows = 64;   // query rows per workgroup
constexpr int kScoreTileN = 64;  // pooled keys per LDS tile

template <int DI>
__global__ __launch_bounds__(256, 2) void index_scores_kernel(ScoreArgs a, int64_t n_per_wg) {
  constexpr int NC = DI / 32;      // 32-dim MFMA k-chunks
  constexpr int ROW = DI + 8;      // LDS row in bf16 elements, padded by 16 B
  constexpr int VPR = DI / 8;      // 16-byte vectors per pooled key
  constexpr int LPT = kScoreTileN * VPR / 256;  // 16-byte loads per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t tile[2][kScoreTileN * ROW];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int bi = blockIdx.z;
  const int64_t base = a.seq_lens ? (int64_t)a.seq_lens[bi] - a.lq : a.q_pos0;
  const int64_t i0 = (int64_t)blockIdx.x * kScoreRows;
  const int64_t t_last = base + min(i0 + kScoreRows - 1, a.lq - 1);
  if (t_last < 0) return;
  const int64_t nb_need = min(t_last / a.r, a.nblk);
  const int64_t n_begin = (int64_t)blockIdx.y * n_per_wg;
  const int64_t n_end = min(n_begin + n_per_wg, nb_need);
  if (n_begin >= n_end) return;
  const int n_tiles = (int)((n_end - n_begin + kScoreTileN - 1) / kScoreTileN);

  const uint16_t* qb = a.q_idx + (int64_t)bi * a.q_bs;
  const float* wb = a.w + (int64_t)bi * a.w_bs;
  const uint16_t* kpb = a.kp + (int64_t)bi * a.kp_bs;
  float* sb = a.scores + (int64_t)bi * a.s_bs;

  // Tile loader: thread -> LPT 16-byte vectors of the 64 x DI tile.
  uint4 stage[LPT];
  auto load_tile = [&](int64_t n0) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int v = threadIdx.x + 256 * u;
      const int row = v / VPR, cv = v - row * VPR;
      const int64_t blk = n0 + row;
      stage[u] = blk < a.nblk ? ld16(kpb + blk * DI + cv * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int v = threadIdx.x + 256 * u;
      const int row = v / VPR, cv = v - row * VPR;
      *reinterpret_cast<uint4*>(&tile[buf][row * ROW + cv * 8]) = stage[u];
    }
  };

  load_tile(n_begin);

  // A operands: this wave's 16 tokens as 4 M-tiles of (4 tokens x 4 heads).
  uint4 A[4][NC];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t tok = i0 + wave * 16 + mt * 4 + (c16 >> 2);
    const int h = c16 & 3;
    const bool ok = tok < a.lq && h < a.h_idx;
    const uint16_t* p = qb + (tok * a.h_idx + h) * DI + quad * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) A[mt][c] = ok ? ld16(p + c * 32) : make_uint4(0, 0, 0, 0);
  }
  // Epilogue data for the accumulator rows this lane holds: token (mt*4 + quad).
  float W[4][4];
  int64_t lim[4];
  float* orow[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t tok = i0 + wave * 16 + mt * 4 + quad;
    const int64_t t = base + tok;
    const bool valid = tok < a.lq && t >= 0;
    lim[mt] = valid ? min(t / a.r, a.nblk) : 0;
    orow[mt] = sb + (valid ? tok : 0) * a.ld;
#pragma unroll
    for (int h = 0; h < 4; ++h) W[mt][h] = (valid && h < a.h_idx) ? wb[tok * a.h_idx + h] : 0.f;
  }

  store_tile(0);
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    const int64_t n0 = n_begin + (int64_t)it * kScoreTileN;
    const bool more = it + 1 < n_tiles;
    if (more) load_tile(n0 + kScoreTileN);
    const uint16_t* tb = tile[it & 1];
    f32x4 acc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 B[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c)
        B[c] = *reinterpret_cast<const uint4*>(&tb[(4 * c16 + j) * ROW + c * 32 + quad * 8]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[mt][j] = mfma_16x16x32(A[mt][c], B[c], acc[mt][j]);
      }
    }
    const int64_t blk0 = n0 + 4 * c16;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      float s[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        s[j] = W[mt][0] * fmaxf(acc[mt][j][0], 0.f) + W[mt][1] * fmaxf(acc[mt][j][1], 0.f) +
               W[mt][2] * fmaxf(acc[mt][j][2], 0.f) + W[mt][3] * fmaxf(acc[mt][j][3], 0.f);
      if (blk0 < lim[mt])
        *reinterpret_cast<float4*>(orow[mt] + blk0) = make_float4(s[0], s[1], s[2], s[3]);
    }
    if (more) store_tile((it + 1) & 1);
    __syncthreads();
  }
}

hipError_t launch_index_scores(const ScoreArgs& a, hipStream_t stream) {
  if (a.lq <= 0 || a.batch <= 0 || a.nblk <= 0) return hipSuccess;
  // Blocks per workgroup along the key axis: enough workgroups to fill 256 CUs
  // even when few query rows are scored (decode), long walks otherwise.
  const int64_t row_tiles = (a.lq + kScoreRows - 1) / kScoreRows;
  int64_t n_per_wg = 2048;
  while (n_per_wg > kScoreTileN && row_tiles * a.batch * ((a.nblk + n_per_wg - 1) / n_per_wg) < 2048)
    n_per_wg /= 2;
  const int64_t ny = (a.nblk + n_per_wg - 1) / n_per_wg;
  dim3 grid((unsigned)row_tiles, (unsigned)ny, (unsigned)a.batch);
  if (a.d_idx == 128)
    hipLaunchKernelGGL(index_scores_kernel<128>, grid, dim3(256), 0, stream, a, n_per_wg);
  else
    hipLaunchKernelGGL(index_scores_kernel<64>, grid, dim3(256), 0, stream, a, n_per_wg);
  return hipGetLastError();
}

}  // namespace qsa

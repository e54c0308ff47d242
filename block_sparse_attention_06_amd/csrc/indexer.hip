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

// fp64 means of columns c..c+7 of pooled block b: keys b*r .. b*r+r-1 (row stride ks),
// summed exactly (each bf16 value and every partial sum fit fp64 without rounding).
__device__ __forceinline__ void pool_mean8(const uint16_t* __restrict__ k, int64_t ks, int64_t b,
                                           int c, int r, double (&m)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = 0.0;
  for (int j = 0; j < r; ++j) {
    const uint4 x = ld16(k + (b * r + j) * ks + c);
    const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m[2 * e] += (double)bf16_bits_to_f32(w4[e] & 0xffffu);
      m[2 * e + 1] += (double)bf16_bits_to_f32(w4[e] >> 16);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] /= r;
}

__device__ __forceinline__ void store_bf16x8(const double (&m)[8], uint16_t* __restrict__ dst) {
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = f64_to_bf16_bits(m[2 * e]) | (f64_to_bf16_bits(m[2 * e + 1]) << 16);
  *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
}

// Columns c..c+7 of pooled block b of a sequence (keys k, row stride ks) into row dst.
// With rope_dim > 0 the leading rope_dim columns are rotated at the block's position
// pos = (first_block + b) * r in the half-split convention: column i < h = rope_dim/2
// pairs with i + h at angle pos * theta^(-2i/rope_dim); the thread of columns c < h
// writes both halves of its pairs, the threads of columns h <= c < rope_dim nothing.
// Mean, rotation and angle are fp64; the result is rounded once to bf16.
constexpr int kMaxRopeHalf = 2048;  // rope_dim <= d_idx <= 4096

// inv[i] = theta^(-2i / rope_dim) for i < rope_dim / 2, once per workgroup in LDS.
__device__ __forceinline__ void rope_freqs(double* inv, int rope_dim, double theta) {
  for (int i = threadIdx.x; i < (rope_dim >> 1); i += blockDim.x)
    inv[i] = pow(theta, -2.0 * (double)i / (double)rope_dim);
  __syncthreads();
}

__device__ __forceinline__ void pool_block8(const uint16_t* __restrict__ k, int64_t ks, int64_t b,
                                            int c, int r, int64_t first_block, int rope_dim,
                                            const double* inv, uint16_t* __restrict__ dst_row) {
  const int h = rope_dim >> 1;
  if (c >= rope_dim) {
    double m[8];
    pool_mean8(k, ks, b, c, r, m);
    store_bf16x8(m, dst_row + c);
    return;
  }
  if (c >= h) return;
  double x1[8], x2[8];
  pool_mean8(k, ks, b, c, r, x1);
  pool_mean8(k, ks, b, c + h, r, x2);
  const double pos = (double)((first_block + b) * r);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    double sn, cs;
    sincos(pos * inv[c + e], &sn, &cs);
    const double a = x1[e], bb = x2[e];
    x1[e] = a * cs - bb * sn;
    x2[e] = bb * cs + a * sn;
  }
  store_bf16x8(x1, dst_row + c);
  store_bf16x8(x2, dst_row + c + h);
}

__global__ __launch_bounds__(256) void pool_keys_kernel(const uint16_t* __restrict__ k,
                                                        int64_t ks, int64_t nb, int d, int r,
                                                        uint16_t* __restrict__ p, int64_t ps,
                                                        int64_t first_block, int rope_dim,
                                                        double theta) {
  __shared__ double inv[kMaxRopeHalf];
  if (rope_dim) rope_freqs(inv, rope_dim, theta);
  const int vec = d >> 3;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = gid / vec;
  if (b >= nb) return;
  const int c = (int)(gid - b * vec) * 8;
  pool_block8(k, ks, b, c, r, first_block, rope_dim, inv, p + b * ps);
}

// Packed sequences: sequence blockIdx.y pools its complete blocks (at most max_nb) from
// its own key tokens into its slot of the padded output p[batch][max_nb][d]; block
// positions count from the sequence's first token.
__global__ __launch_bounds__(256) void pool_keys_varlen_kernel(const uint16_t* __restrict__ k,
                                                               const int32_t* __restrict__ cu_k,
                                                               int64_t max_nb, int d, int r,
                                                               uint16_t* __restrict__ p,
                                                               int rope_dim, double theta) {
  __shared__ double inv[kMaxRopeHalf];
  if (rope_dim) rope_freqs(inv, rope_dim, theta);
  const int vec = d >> 3;
  const int bi = blockIdx.y;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = gid / vec;
  const int64_t k0 = cu_k[bi];
  const int64_t nb = min(((int64_t)cu_k[bi + 1] - k0) / r, max_nb);
  if (b >= nb) return;
  const int c = (int)(gid - b * vec) * 8;
  pool_block8(k + k0 * d, d, b, c, r, 0, rope_dim, inv, p + ((int64_t)bi * max_nb + b) * d);
}

// Wave-row pooling, used when a row's d/8 threads (TPR) are a power of two <= 64, so no
// row straddles a wave, and r = 4. Compared with the per-thread form above: the four
// loads of a thread are issued together, a workgroup
// strides over the blocks, and with an encoding the angles of the wave's rows are
// spread over all 64 lanes (their sines and cosines go through wave-private LDS) while
// every lane rotates and stores its own 8 columns, taking its partner columns' means
// (c +- rope_dim/2, in the same row) from the partner lane. Arithmetic and rounding
// are those of pool_block8, value for value.
struct PoolWaveArgs {
  const uint16_t* k;
  int64_t ks;
  int64_t nb;  // blocks (plain); max blocks per sequence (packed)
  int d, r;
  uint16_t* p;
  int64_t ps;
  int64_t first_block;
  int rope_dim;
  double theta;
  const int32_t* cu_k;  // packed sequences (blockIdx.y) or null
};

constexpr int kPoolWaveMaxD = 512;  // TPR <= 64

// pool_mean8 with the r = 4 loads issued together.
__device__ __forceinline__ void pool_mean8_r4(const uint16_t* __restrict__ k, int64_t ks,
                                              int64_t b, int c, double (&m)[8]) {
  uint4 x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = ld16(k + (b * 4 + j) * ks + c);
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w4[4] = {x[j].x, x[j].y, x[j].z, x[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m[2 * e] += (double)bf16_bits_to_f32(w4[e] & 0xffffu);
      m[2 * e + 1] += (double)bf16_bits_to_f32(w4[e] >> 16);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] /= 4;
}

__global__ __launch_bounds__(256) void pool_keys_wave_kernel(PoolWaveArgs a) {
  __shared__ double inv[kPoolWaveMaxD / 2];
  __shared__ double2 sc_all[4][kWave * 4];  // per wave: rows_per_wave * rope_dim/2 <= 256
  const uint16_t* k = a.k;
  uint16_t* p = a.p;
  int64_t nb = a.nb, first_block = a.first_block;
  if (a.cu_k) {  // packed: sequence blockIdx.y, positions from its first token
    const int64_t k0 = a.cu_k[blockIdx.y];
    k += k0 * a.ks;
    nb = min(((int64_t)a.cu_k[blockIdx.y + 1] - k0) / a.r, a.nb);
    p += (int64_t)blockIdx.y * a.nb * a.ps;
    first_block = 0;
  }
  const int rope_dim = a.rope_dim, h = rope_dim >> 1;
  if (rope_dim) rope_freqs(inv, rope_dim, a.theta);
  const int tpr = a.d >> 3, rpw = kWave / tpr, rpi = 4 * rpw;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int rw = lane / tpr, c = (lane & (tpr - 1)) * 8;
  const bool rot = c < rope_dim, first_half = c < h;
  const int partner = rot ? lane + (first_half ? (h >> 3) : -(h >> 3)) : lane;
  const int ai = rw * h + (first_half ? c : c - h);  // this lane's first (sin, cos) entry
  double2* sc = sc_all[wave];
  for (int64_t base = (int64_t)blockIdx.x * rpi; base < nb; base += (int64_t)gridDim.x * rpi) {
    const int64_t row0 = base + wave * rpw;
    const int64_t b = row0 + rw, bl = min(b, nb - 1);
    double x[8];
    pool_mean8_r4(k, a.ks, bl, c, x);
    if (rope_dim) {
      for (int t = lane; t < rpw * h; t += kWave) {
        const int row = t / h, i = t - row * h;
        const int64_t bb = min(row0 + row, nb - 1);
        double sn, cs;
        sincos((double)((first_block + bb) * a.r) * inv[i], &sn, &cs);
        sc[t] = make_double2(sn, cs);
      }
      double y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = __shfl(x[e], partner);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (rot) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double2 v = sc[ai + e];
          // first half: a*cos - b*sin with b the partner; second half: b*cos + a*sin
          x[e] = first_half ? x[e] * v.y - y[e] * v.x : x[e] * v.y + y[e] * v.x;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    if (b < nb) store_bf16x8(x, p + b * a.ps + c);
  }
}

static bool pool_wave_fits(int d, int r) {
  const int tpr = d >> 3;
  return r == 4 && d <= kPoolWaveMaxD && (tpr & (tpr - 1)) == 0;
}

static hipError_t launch_pool_wave(const PoolWaveArgs& a, int64_t rows, int batch,
                                   hipStream_t stream) {
  const int rpi = 4 * (kWave / (a.d >> 3));
  const int64_t passes = (rows + rpi - 1) / rpi;
  // Up to 8 workgroups per CU (the most 256-thread workgroups a CU holds): 1M raw
  // keys on MI355X 59.1 -> 58.6 us plain, 82.2 -> 75.0 us with the encoding, against
  // 5 per CU.
  const int64_t cap = (int64_t)256 * 8 / batch + 1;
  const unsigned grid = (unsigned)(passes < cap ? passes : cap);
  hipLaunchKernelGGL(pool_keys_wave_kernel, dim3(grid, (unsigned)batch), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_pool_keys(const uint16_t* k_idx, int64_t k_stride, int64_t n_blocks, int d_idx,
                            int r, uint16_t* k_pooled, int64_t p_stride, const PooledPe& pe,
                            hipStream_t stream) {
  if (n_blocks <= 0) return hipSuccess;
  if (pool_wave_fits(d_idx, r))
    return launch_pool_wave({k_idx, k_stride, n_blocks, d_idx, r, k_pooled, p_stride, pe.first_block,
                          pe.rope_dim, pe.theta, nullptr},
                         n_blocks, 1, stream);
  const int64_t threads = n_blocks * (d_idx / 8);
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(pool_keys_kernel, dim3((unsigned)grid), dim3(256), 0, stream, k_idx,
                     k_stride, n_blocks, d_idx, r, k_pooled, p_stride, pe.first_block,
                     pe.rope_dim, pe.theta);
  return hipGetLastError();
}

hipError_t launch_pool_keys_varlen(const uint16_t* k_idx, const int32_t* cu_k, int batch,
                                   int64_t max_nb, int d_idx, int r, uint16_t* k_pooled,
                                   const PooledPe& pe, hipStream_t stream) {
  if (max_nb <= 0 || batch <= 0) return hipSuccess;
  if (pool_wave_fits(d_idx, r))
    return launch_pool_wave({k_idx, d_idx, max_nb, d_idx, r, k_pooled, d_idx, 0, pe.rope_dim, pe.theta,
                          cu_k},
                         max_nb, batch, stream);
  const int64_t grid = (max_nb * (d_idx / 8) + 255) / 256;
  hipLaunchKernelGGL(pool_keys_varlen_kernel, dim3((unsigned)grid, (unsigned)batch), dim3(256), 0,
                     stream, k_idx, cu_k, max_nb, d_idx, r, k_pooled, pe.rope_dim, pe.theta);
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
// store past the own block carries unspecified values, never read). The scores are
// stored non-temporal: a chunk's scores (2 GiB for 16K rows at 128K keys) are far
// larger than the caches, and kept out of L2 they leave it to the pooled-key tiles
// that every row tile re-reads (at 128K: 3.00 -> 2.66 ms a step on MI355X).
// ------------------------------------------------------------------------------------

// 16-byte store of four floats marked non-temporal: written once and read back only
// after much other traffic, so it should not displace data that is being reused.
__device__ __forceinline__ void st16_stream(float* p, float a, float b, float c, float d) {
  const f32x4 v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

constexpr int kScoreRows = 64;   // query rows per workgroup
constexpr int kScoreTileN = 64;  // pooled keys per LDS tile

template <int DI>
__global__ __launch_bounds__(256, 2) void index_scores_kernel(ScoreArgs a, int64_t n_per_wg) {
  constexpr int NC = DI / 32;      // 32-dim MFMA k-chunks
  constexpr int VPR = DI / 8;      // 16-byte vectors per pooled key
  constexpr int LPT = kScoreTileN * VPR / 256;  // 16-byte loads per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t tile[2][kScoreTileN * DI];  // key_tile_off layout

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int bi = blockIdx.z;
  int64_t base = a.seq_lens ? (int64_t)a.seq_lens[bi] - a.lq : a.q_pos0;
  int64_t lq = a.lq;
  const uint16_t* qb = a.q_idx + (int64_t)bi * a.q_bs;
  const float* wb = a.w + (int64_t)bi * a.w_bs;
  if (a.vl.cu_q) {  // packed sequences: this sequence's rows of the launch
    const SeqRows sr = varlen_rows(a.vl, bi, a.lq);
    lq = sr.n;
    base = sr.pos;
    qb = a.q_idx + sr.first * a.h_idx * DI;
    wb = a.w + sr.first * a.h_idx;
  }
  const int64_t i0 = (int64_t)blockIdx.x * kScoreRows;
  if (i0 >= lq) return;
  if (a.row_flags) {  // score only the tiles that hold a flagged row
    const int64_t rr = i0 + threadIdx.x;
    const int fl = (threadIdx.x < kScoreRows && rr < lq) ? a.row_flags[rr] : 0;
    if (!__syncthreads_or(fl)) return;
  }
  const int64_t t_last = base + min(i0 + kScoreRows - 1, lq - 1);
  if (t_last < 0) return;
  const int64_t nb_need = min(t_last / a.r, a.nblk);
  const int64_t n_begin = (int64_t)blockIdx.y * n_per_wg;
  const int64_t n_end = min(n_begin + n_per_wg, nb_need);
  if (n_begin >= n_end) return;
  const int n_tiles = (int)((n_end - n_begin + kScoreTileN - 1) / kScoreTileN);

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
      *reinterpret_cast<uint4*>(&tile[buf][key_tile_off<DI>(row, cv)]) = stage[u];
    }
  };

  load_tile(n_begin);

  // A operands: this wave's 16 tokens as 4 M-tiles of (4 tokens x 4 heads).
  uint4 A[4][NC];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t tok = i0 + wave * 16 + mt * 4 + (c16 >> 2);
    const int h = c16 & 3;
    const bool ok = tok < lq && h < a.h_idx;
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
    const bool valid = tok < lq && t >= 0;
    lim[mt] = valid ? min(t / a.r, a.nblk) : 0;
    orow[mt] = sb + (valid ? tok : 0) * a.ld;
#pragma unroll
    for (int h = 0; h < 4; ++h) W[mt][h] = (valid && h < a.h_idx) ? wb[tok * a.h_idx + h] : 0.f;
  }

  store_tile(0);
  __syncthreads();
  for (int it = 0; it < n_tiles; ++it) {
    const int64_t n0 = n_begin + (int64_t)it * kScoreTileN;
    // The next tile's loads and LDS writes run on every pass, the last one's going
    // to a buffer nothing reads: with both under one condition the compiler could not
    // tell that the writes had waited for the loads and waited again at the top.
    load_tile(n0 + kScoreTileN);
    const uint16_t* tb = tile[it & 1];
    f32x4 acc[4][4];
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
    const int64_t blk0 = n0 + 4 * c16;
    float s[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[mt][j] = score_of_heads(W[mt], acc[mt][j]);
    // The next tile goes to LDS (the other buffer, read by no wave until the barrier)
    // before the score stores: loads and stores share one counter, so a wait for the
    // tile's loads placed after the stores would wait for the stores too.
    store_tile((it + 1) & 1);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      if (blk0 < lim[mt]) st16_stream(orow[mt] + blk0, s[mt][0], s[mt][1], s[mt][2], s[mt][3]);
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------
// Stage 2 for a few query rows per sequence (decode): a streaming scan of the pooled
// keys. One wave per (sequence, row, range of blocks), no barriers: the wave keeps its
// token's 4 heads as the A operand (rows 0-3 of the MFMA tile, the rest zero). A tile
// of 64 pooled keys is read from memory contiguously (instruction u, lane L: bytes
// 1024 u + 16 L of the tile for d_I = 128, whole rows per 16 lanes) and turned into B
// operands (lane (c16, quad) of column set j needs chunk quad + 4c of row 16 j + c16)
// through a wave-private LDS half tile whose 16-byte chunks are XOR-swizzled by the
// row, so that both the contiguous writes and the strided reads hit distinct banks.
// Two tiles are in flight: a tile's loads are issued before the previous one is staged
// and multiplied.
// ------------------------------------------------------------------------------------

template <int DI, bool CAND>
__global__ __launch_bounds__(256, 2) void index_scores_scan_kernel(ScoreArgs a, int n_ranges,
                                                                int blocks_per_wave) {
  // With CAND, a wave's range is one top-k segment (kTopkWaveSeg blocks, tiles of 64):
  // each tile's scores wait in LDS (one per lane and tile), and at the end the wave
  // writes them and extracts the segment's kTopkWaveKeep best for the top-k merge.
  constexpr int kSegTiles = kTopkWaveSeg / 64;
  constexpr int NC = DI / 32;
  constexpr int CPR = DI / 8;  // 16-byte chunks per pooled key = loads per lane per tile
  __shared__ uint4 stage[4][32 * CPR];  // half a tile per wave
  __shared__ float scores_lds[4][kSegTiles * 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  const int64_t per_seq = a.lq * n_ranges;
  const int bi = (int)(item / per_seq);
  if (bi >= a.batch) return;
  const int64_t rem = item - (int64_t)bi * per_seq;
  const int64_t row = rem / n_ranges;
  const int rg = (int)(rem - row * n_ranges);
  const int64_t base = a.seq_lens ? (int64_t)a.seq_lens[bi] - a.lq : a.q_pos0;
  const int64_t t = base + row;
  if (t < 0) return;
  const int64_t lim = min(t / a.r, a.nblk);
  const int64_t n0 = (int64_t)rg * blocks_per_wave;
  const int64_t n1 = min(n0 + blocks_per_wave, lim);
  const int64_t cslot = ((int64_t)bi * a.lq + row) * a.cand.n_seg + rg;
  if (n0 >= n1) {
    if (CAND && lane < kTopkWaveKeep) {  // an empty segment: padding only
      a.cand.cand_val[cslot * kTopkWaveKeep + lane] = __builtin_nanf("");
      a.cand.cand_idx[cslot * kTopkWaveKeep + lane] = -1;
      if (lane == 0) a.cand.bnd_idx[cslot] = -1;
    }
    return;
  }

  const uint16_t* kpb = a.kp + (int64_t)bi * a.kp_bs;
  float* orow = a.scores + (int64_t)bi * a.s_bs + row * a.ld;
  // A: row c16 is head c16 of this token (zero beyond the indexer heads).
  uint4 A[NC];
  {
    const bool ok = c16 < min(a.h_idx, 4);
    const uint16_t* p = a.q_idx + (int64_t)bi * a.q_bs + (row * a.h_idx + (ok ? c16 : 0)) * DI +
                        quad * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) A[c] = ok ? ld16(p + c * 32) : make_uint4(0, 0, 0, 0);
  }
  float W[4];
#pragma unroll
  for (int h = 0; h < 4; ++h)
    W[h] = h < a.h_idx ? a.w[(int64_t)bi * a.w_bs + row * a.h_idx + h] : 0.f;

  uint4* st = stage[wave];
  uint4 R0[CPR], R1[CPR];
  // Unconditional loads (rows past the range clamp to its last one, never used), so
  // that every wait counts exactly one tile.
  auto load = [&](uint4 (&R)[CPR], int64_t nb) {
#pragma unroll
    for (int u = 0; u < CPR; ++u) {
      const int e = u * 64 + lane;
      const int64_t blk = min(nb + e / CPR, n1 - 1);
      R[u] = ld16_stream(kpb + blk * DI + (e % CPR) * 8);  // read once per pass
    }
  };
  // Stage a tile and multiply it, half a tile (32 rows, two MFMA column sets) at a time:
  // returns the scores of blocks nb + 16 j + c16 (valid in the quad-0 lanes).
  auto compute = [&](const uint4 (&R)[CPR], float (&s)[4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int u = h * CPR / 2; u < (h + 1) * CPR / 2; ++u) {
        const int e = u * 64 + lane;
        const int r = e / CPR - 32 * h, ch = e % CPR;
        st[r * CPR + (ch ^ (r & (CPR - 1)))] = R[u];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int r = 16 * jj + c16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c)
          acc = mfma_16x16x32(A[c], st[r * CPR + ((quad + 4 * c) ^ (r & (CPR - 1)))], acc);
        s[2 * h + jj] = score_of_heads(W, acc);
      }
      // The next half's stores must not pass these reads.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  };
  const int n_tiles = (int)((n1 - n0 + 63) / 64);

  // Lane L's score: block nb + L of the tile (element L / 16 of quad-0 lane L % 16).
  auto lane_score = [&](const uint4 (&R)[CPR]) -> float {
    float s[4];
    compute(R, s);
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __shfl(s[j], c16, 64);
    return quad == 0 ? v[0] : (quad == 1 ? v[1] : (quad == 2 ? v[2] : v[3]));
  };

  // Streams up to kSegTiles tiles from block c0 with two tiles in flight, parking one
  // score per lane and tile in the wave's LDS slots (no global stores in the stream: a
  // store among the loads would make every wait a full drain).
  float* sc = scores_lds[wave];
  auto stream = [&](int64_t c0, int nt) {
    load(R0, c0);
    load(R1, c0 + 64);
#pragma unroll
    for (int it = 0; it < kSegTiles; it += 2) {
      if (it >= nt) break;
      const int64_t nb = c0 + (int64_t)it * 64;
      sc[it * 64 + lane] = lane_score(R0);
      if (it + 2 < kSegTiles) load(R0, nb + 128);
      __builtin_amdgcn_sched_barrier(0);
      if (it + 1 < nt) sc[(it + 1) * 64 + lane] = lane_score(R1);
      if (it + 3 < kSegTiles) load(R1, nb + 192);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (!CAND) {
    // Chunks of kSegTiles tiles, each streamed, then stored in one burst.
    for (int64_t c0 = n0; c0 < n1; c0 += 64 * kSegTiles) {
      const int nv = (int)min(n1 - c0, (int64_t)64 * kSegTiles);
      stream(c0, (nv + 63) / 64);
#pragma unroll
      for (int i = 0; i < kSegTiles; ++i)
        if (i * 64 + lane < nv) orow[c0 + i * 64 + lane] = sc[i * 64 + lane];  // own slots
    }
  } else {
    stream(n0, n_tiles);
    const int n_valid = (int)(n1 - n0);
    // The segment's scores leave in one burst of coalesced stores after its loads
    // (stores interleaved with the key stream cost HBM read/write turnarounds); a -0
    // leaves as +0, as the rank keys see it.
    uint64_t rk[kSegTiles];
#pragma unroll
    for (int i = 0; i < kSegTiles; ++i) {
      const int p = i * 64 + lane;
      rk[i] = p < n_valid ? rank_key(sc[p], (int32_t)(n0 + p)) : 0ull;
      if (p < n_valid) orow[n0 + p] = key_to_float((uint32_t)(rk[i] >> 32));
    }
    const int keep = min(n_valid, kTopkWaveKeep);
    float* cv = a.cand.cand_val + cslot * kTopkWaveKeep;
    int32_t* ci = a.cand.cand_idx + cslot * kTopkWaveKeep;
    // The extraction packs its survivors into 64 wave-private slots: the staging tile.
    const uint64_t last =
        wave_extract_top<kSegTiles>(rk, keep, reinterpret_cast<uint64_t*>(st), [&](int k, uint64_t w) {
          cv[k] = key_to_float((uint32_t)(w >> 32));
          ci[k] = rank_key_id(w);
        });
    if (lane == 0) {
      for (int k = keep; k < kTopkWaveKeep; ++k) {
        cv[k] = __builtin_nanf("");
        ci[k] = -1;
      }
      const bool truncated = n_valid > keep;
      a.cand.bnd_val[cslot] = truncated ? key_to_float((uint32_t)(last >> 32)) : 0.f;
      a.cand.bnd_idx[cslot] = truncated ? rank_key_id(last) : -1;
    }
  }
}

hipError_t launch_index_scores(const ScoreArgs& a, hipStream_t stream) {
  if (a.lq <= 0 || a.batch <= 0 || a.nblk <= 0) return hipSuccess;
  if ((a.lq <= 4 || a.cand.cand_val) && !a.vl.cu_q && !a.row_flags) {
    // About 2048 waves (two per SIMD): one round over the GPU, 64-block tiles. With
    // candidates, a wave covers exactly one top-k segment.
    const int64_t rows = (int64_t)a.batch * a.lq;
    int64_t bpw = (rows * a.nblk + 2047) / 2048;
    bpw = (bpw + 63) / 64 * 64;
    if (bpw < 64) bpw = 64;
    if (a.cand.cand_val) bpw = kTopkWaveSeg;
    const int n_ranges = (int)((a.nblk + bpw - 1) / bpw);
    const int64_t waves = rows * n_ranges;
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (a.cand.cand_val) {
      if (a.d_idx == 128)
        hipLaunchKernelGGL((index_scores_scan_kernel<128, true>), grid, dim3(256), 0, stream, a,
                           n_ranges, (int)bpw);
      else
        hipLaunchKernelGGL((index_scores_scan_kernel<64, true>), grid, dim3(256), 0, stream, a,
                           n_ranges, (int)bpw);
    } else if (a.d_idx == 128) {
      hipLaunchKernelGGL((index_scores_scan_kernel<128, false>), grid, dim3(256), 0, stream, a,
                         n_ranges, (int)bpw);
    } else {
      hipLaunchKernelGGL((index_scores_scan_kernel<64, false>), grid, dim3(256), 0, stream, a,
                         n_ranges, (int)bpw);
    }
    return hipGetLastError();
  }
  // Blocks per workgroup along the key axis: enough workgroups to fill 256 CUs
  // even when few query rows are scored, long walks otherwise.
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

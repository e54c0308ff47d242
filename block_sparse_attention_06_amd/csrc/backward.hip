// Backward of stage 4: gradients of the sparse attention with respect to q, k and v
// over fixed selection rows.
//
// Method ("Qwen3.8-Flash-Next" Miles recipe, section 1 "Model Introduction"): the
// recipe trains through a forward and a backward sparse-attention kernel whose
// selection rows are built outside the kernel. The selection is a constant of the
// backward pass: no gradient reaches the indexer through the top-k.
//
// With P = softmax(scale q k^T) over each row's kept tokens and dO the output gradient:
//   dV_j = sum_t P_tj dO_t,   dP_tj = dO_t . v_j,   D_t = dO_t . O_t (= sum_j P_tj dP_tj),
//   dS_tj = P_tj (dP_tj - D_t),   dQ_t = scale sum_j dS_tj k_j,   dK_j = scale sum_t dS_tj q_t.
// P is recomputed from the forward's lse; D comes from the forward's bf16 output.
//
// Query side: one wave per (query row, KV group) walks the row's kept blocks 4 at a
// time, like the forward kernel: S^T = K.Q^T and dP^T = V.dO^T on
// v_mfma_f32_16x16x32_bf16 (keys as rows), dS in the S^T layout, which is the A
// operand of dQ = dS.K on v_mfma_f32_16x16x16_bf16 (K read a second time with 4 keys
// per lane, output columns permuted as in the forward). The wave also stores D.
//
// Key side: one wave per (key block, KV group) over the rows that kept the block. The
// inverse selection is built by a stable radix sort of the (block, row) pairs, so a
// block's rows come in ascending order and every sum has a fixed order (the results
// do not depend on scheduling). Per row: S = Q.K^T and dP = dO.V^T with the block's 4
// keys as MFMA columns (12 of 16 rows are heads, 4 of 16 columns are keys), so P and
// dS land in the A-operand layout of dV = P^T.dO and dK = dS^T.Q, whose B operands
// are the row's dO and q with 4 heads per lane. A row's q and dO are read from memory
// once, two rows ahead, and staged in the wave's LDS tile, from which both layouts are
// read; the block's K and V sit in LDS too.

#include <cstring>  // rocPRIM's host code uses memset

#include <rocprim/device/device_radix_sort.hpp>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t bwd_half(uint32_t w, int hi) {
  return hi ? (w >> 16) : (w & 0xffffu);
}

__device__ __forceinline__ uint32_t bwd_word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// B operand of a 16x16x16 MFMA from 4 rows (k) of 8 consecutive bf16 each: column e
// of the 8 (output dim tile hf*8 + e) packs element e of the 4 rows.
__device__ __forceinline__ uint2 bwd_repack(const uint4 (&r)[4], int e) {
  const int wi = e >> 1, hi = e & 1;
  const uint32_t lo = bwd_half(bwd_word(r[0], wi), hi) | (bwd_half(bwd_word(r[1], wi), hi) << 16);
  const uint32_t up = bwd_half(bwd_word(r[2], wi), hi) | (bwd_half(bwd_word(r[3], wi), hi) << 16);
  return make_uint2(lo, up);
}

__device__ __forceinline__ float bf16_dot8(const uint4& a, const uint4& b) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w};
  const uint32_t y[4] = {b.x, b.y, b.z, b.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += bf16_bits_to_f32(x[i] & 0xffffu) * bf16_bits_to_f32(y[i] & 0xffffu);
    s += bf16_bits_to_f32(x[i] >> 16) * bf16_bits_to_f32(y[i] >> 16);
  }
  return s;
}

}  // namespace

// ---- query side: dQ and D ------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void sparse_attn_bwd_dq_kernel(BwdArgs a) {
  constexpr int NC = D / 32;
  constexpr int NH = D / 128;
  constexpr int NT = D / 16;
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
  const int n_steps = (a.n_sel + 3) / 4;
  const int32_t* srow = a.sel + row * a.n_sel;
  const int64_t kstride = (int64_t)a.hkv * D;

  // Head c16 of the group as a B operand (k = dims 32c + 8*quad + [0..7]): q, dO, O.
  const bool hv = c16 < G;
  const int64_t hrow = (row * a.hq + g * G + (hv ? c16 : 0)) * (int64_t)D + quad * 8;
  uint4 Qc[NC], dOc[NC];
  float dsum = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    Qc[c] = hv ? ld16(a.q + hrow + c * 32) : make_uint4(0, 0, 0, 0);
    dOc[c] = hv ? ld16(a.dout + hrow + c * 32) : make_uint4(0, 0, 0, 0);
    const uint4 Oc = hv ? ld16(a.out + hrow + c * 32) : make_uint4(0, 0, 0, 0);
    dsum += bf16_dot8(dOc[c], Oc);
  }
  dsum = wave_xor_sum(dsum, 16);
  dsum = wave_xor_sum(dsum, 32);  // D of head c16, in every quad
  const float Dh = dsum;
  const float L2 = hv ? a.lse[row * a.hq + g * G + c16] * kLog2e : 0.f;
  if (quad == 0 && hv) a.dbuf[row * a.hq + g * G + c16] = Dh;

  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.scale_log2;

  // Steps of 4 kept blocks (16 keys: key x = token x % 4 of block slot x / 4), two in
  // flight. A step's block ids are scalar loads (the selection row is read-only here
  // and uniform per wave); its K and V rows are read whole (load u, lane L: 16-byte
  // chunk L % 32 of key 2u + L / 32, padding reads token 0, masked) and staged in the
  // wave's LDS tiles ([key][chunk], chunks XOR-swizzled by key & 7), which give the A
  // operands of S^T = K.Q^T and dP^T = V.dO^T (key c16, chunk quad + 4c) and the B
  // operand of dQ = dS.K (4 keys per lane, 8 dims each): K is read from memory once.
  constexpr int CPK = D / 8;         // 16-byte chunks per key row
  constexpr int LPS = 16 * CPK / 64;  // loads per lane per step, each of K and V
  __shared__ uint4 dq_tile_k[4][16 * CPK], dq_tile_v[4][16 * CPK];
  uint4* tk_ = dq_tile_k[wave];
  uint4* tv_ = dq_tile_v[wave];
  const auto* ssel = reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(srow));
  struct Step {
    uint4 Kr[LPS], Vr[LPS];
    int first, bq;  // block of slot 0 (-1: padding reached), block of slot `quad`
  };
  auto issue = [&](Step& st, int s) {
    int b4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b4[j] = (4 * s + j < a.n_sel) ? ssel[4 * s + j] : -1;
    st.first = b4[0];
    st.bq = quad == 0 ? b4[0] : (quad == 1 ? b4[1] : (quad == 2 ? b4[2] : b4[3]));
#pragma unroll
    for (int u = 0; u < LPS; ++u) {
      const int key = u * (64 / CPK) + lane / CPK;
      const int slot = key >> 2;
      const int bk = slot == 0 ? b4[0] : (slot == 1 ? b4[1] : (slot == 2 ? b4[2] : b4[3]));
      int64_t tok = (int64_t)bk * 4 + (key & 3);
      tok = bk < 0 ? 0 : min(tok, t);
      const int64_t off = tok * kstride + g * D + (lane % CPK) * 8;
      st.Kr[u] = ld16(a.k + off);
      st.Vr[u] = ld16(a.v + off);
    }
  };
  auto compute = [&](const Step& st) {
#pragma unroll
    for (int u = 0; u < LPS; ++u) {
      const int key = u * (64 / CPK) + lane / CPK;
      const int ch = (lane % CPK) ^ (key & 7);
      tk_[key * CPK + ch] = st.Kr[u];
      tv_[key * CPK + ch] = st.Vr[u];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4 S = {0.f, 0.f, 0.f, 0.f}, dP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = (quad + 4 * c) ^ (c16 & 7);
      S = mfma_16x16x32(tk_[c16 * CPK + ch], Qc[c], S);
      dP = mfma_16x16x32(tv_[c16 * CPK + ch], dOc[c], dP);
    }
    // Row 4*quad+i of S^T is token bq*4 + i; column c16 is head c16.
    float ds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = hv && st.bq >= 0 && (int64_t)st.bq * 4 + i <= t;
      const float p = ok ? exp2f(S[i] * sl2 - L2) : 0.f;
      ds[i] = p * (dP[i] - Dh);
    }
    const uint2 A = make_uint2(pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]));
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      uint4 Kq[4];  // the tokens of block slot `quad`, dims hf*128 + 8*c16 ..
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = 4 * quad + kk;
        Kq[kk] = tk_[key * CPK + ((c16 + 16 * hf) ^ (key & 7))];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        acc[hf * 8 + e] = mfma_16x16x16(A, bwd_repack(Kq, e), acc[hf * 8 + e]);
    }
    // The next step's tile stores must not pass these reads.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  Step A0, A1;
  issue(A0, 0);
  issue(A1, 1);
  for (int s = 0; s < n_steps; s += 2) {
    if (A0.first < 0) break;  // -1 padding reached
    compute(A0);
    issue(A0, s + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 >= n_steps || A1.first < 0) break;
    compute(A1);
    issue(A1, s + 3);
    __builtin_amdgcn_sched_barrier(0);
  }

  // dq = scale * dS.K; lane holds heads 4*quad + i, dims hf*128 + 8*c16 + e.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hl = 4 * quad + i;
    if (hl < G) {
      float* op = a.dq + (row * a.hq + g * G + hl) * (int64_t)D + c16 * 8;
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        *reinterpret_cast<float4*>(op + hf * 128) =
            make_float4(acc[hf * 8 + 0][i] * a.scale, acc[hf * 8 + 1][i] * a.scale,
                        acc[hf * 8 + 2][i] * a.scale, acc[hf * 8 + 3][i] * a.scale);
        *reinterpret_cast<float4*>(op + hf * 128 + 4) =
            make_float4(acc[hf * 8 + 4][i] * a.scale, acc[hf * 8 + 5][i] * a.scale,
                        acc[hf * 8 + 6][i] * a.scale, acc[hf * 8 + 7][i] * a.scale);
      }
    }
  }
}

// ---- inverse selection ----------------------------------------------------------------

// Pair p = (row i, slot s): key = kept block (n_kb for padding: sorts last), value = i.
__global__ __launch_bounds__(256) void bwd_pairs_kernel(const int32_t* __restrict__ sel,
                                                         int64_t n_pairs, int n_sel,
                                                         int32_t n_kb, int32_t* __restrict__ keys,
                                                         int32_t* __restrict__ rows) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= n_pairs) return;
  const int32_t b = sel[p];
  keys[p] = (b >= 0 && b < n_kb) ? b : n_kb;
  rows[p] = (int32_t)(p / n_sel);
}

// start[b] = first position of key b in the sorted keys (b = 0 .. n_kb).
__global__ __launch_bounds__(256) void bwd_starts_kernel(const int32_t* __restrict__ keys,
                                                          int64_t n_pairs, int32_t n_kb,
                                                          int32_t* __restrict__ start) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b > n_kb) return;
  int64_t lo = 0, hi = n_pairs;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (keys[mid] < b) lo = mid + 1;
    else hi = mid;
  }
  start[b] = (int32_t)lo;
}

// ---- key side: dK and dV --------------------------------------------------------------

// NL: 1 KiB loads that cover a row's G heads of one group, ceil(G * D / 512).
template <int D, int NL>
__global__ __launch_bounds__(256) void sparse_attn_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NC = D / 32;
  constexpr int NH = D / 128;
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int G = a.hq / a.hkv;

  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  const int64_t kb = item / a.hkv;
  const int g = (int)(item - kb * a.hkv);
  if (kb >= a.n_kb) return;
  const int64_t kstride = (int64_t)a.hkv * D;

  // The block's 4 keys as B columns (k = dims 32c + 8*quad + [0..7]); other columns 0.
  __shared__ uint4 bwd_tile_q[4][16 * D / 8], bwd_tile_do[4][16 * D / 8];
  __shared__ uint4 bwd_tile_kv[4][2][4 * D / 8];
  // The block's 4 keys (K, then V) in the wave's LDS, chunks XOR-swizzled by the key:
  // B columns c16 read key c16 % 4 (columns past the 4 keys are masked out of P and dS
  // later; keys past lk read the last key, also masked).
  uint4* tkv = &bwd_tile_kv[wave][0][0];
  {
    const int64_t tok = min(kb * 4 + (lane & 3), a.lk - 1);
    const int part = (lane >> 2) & 1;  // 0: K, 1: V
    const uint16_t* src = (part ? a.v : a.k) + tok * kstride + g * D;
#pragma unroll
    for (int u = lane >> 3; u < D / 8; u += 8)
      tkv[(part * 4 + (lane & 3)) * (D / 8) + (u ^ (lane & 3))] = ld16(src + u * 8);
  }

  f32x4 dK[NT], dV[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    dK[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    dV[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = a.scale_log2;
  const int32_t p0 = a.start[kb], p1 = a.start[kb + 1];
  const bool hv = c16 < G;  // A rows: head c16

  // Rows are loaded two ahead into registers: a row's q and dO of the group's heads
  // (contiguous chunks) with its lse and D of heads 4*quad + i. On arrival they go to
  // the wave's LDS tile ([head][16-byte chunk], chunks XOR-swizzled by head & 7 so that
  // all three access shapes are free of bank conflicts), the registers take the row
  // after next, and the row is computed from the tile: the A operands of S and dP (head
  // c16, k = dims 32c + 8*quad + [0..7]) and the B operands of dV and dK (4 heads per
  // lane, 8 dims each). The tile is private to the wave: no workgroup barrier.
  struct RowBuf {
    uint4 Qa[NL], dOa[NL];
    float L2[4], Dh[4];
    int64_t row;
  };
  // Every load is unconditional (past the group's heads: its last head again; those
  // S and dP rows are masked out of P and dS), so that the waits count loads exactly.
  // The pair list is read-only here and p is uniform: scalar loads, which the vector
  // loads in flight need not wait for.
  const auto* prow = reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(a.pair_rows));
  // The group's G heads of a row are G * D contiguous bf16 in q and in dout: load u,
  // lane L takes 16-byte chunk 64u + L of them (whole 1 KiB per instruction; chunks past
  // the group's last re-read it).
  constexpr int CPR = D / 8;  // 16-byte chunks per head
  const int n_chunks = G * CPR;
  auto load_row = [&](RowBuf& rb, int32_t p) {
    rb.row = prow[p];
    const int64_t hbase = (rb.row * a.hq + g * G) * (int64_t)D;
    const uint16_t* qp = a.q + hbase + lane * 8;
    const uint16_t* dp = a.dout + hbase + lane * 8;
#pragma unroll
    for (int u = 0; u < NL - 1; ++u) {
      rb.Qa[u] = ld16(qp + u * 512);
      rb.dOa[u] = ld16(dp + u * 512);
    }
    const int64_t last = (int64_t)min(64 * (NL - 1) + lane, n_chunks - 1) * 8;
    rb.Qa[NL - 1] = ld16(a.q + hbase + last);
    rb.dOa[NL - 1] = ld16(a.dout + hbase + last);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = min(4 * quad + i, G - 1);
      rb.L2[i] = a.lse[rb.row * a.hq + g * G + h] * kLog2e;
      rb.Dh[i] = a.dbuf[rb.row * a.hq + g * G + h];
    }
  };
  uint4* tq = bwd_tile_q[wave];
  uint4* tdo = bwd_tile_do[wave];
  for (int c = 64 * NL + lane; c < 16 * CPR; c += 64) {
    tq[c] = make_uint4(0, 0, 0, 0);
    tdo[c] = make_uint4(0, 0, 0, 0);
  }
  struct RowState {
    float l2[4], dh[4];
    int64_t t;
  };
  auto stage = [&](const RowBuf& rb, RowState& rs) {
    // Rows past the group's heads that the last load reaches get copies of its last
    // chunk (finite; they meet P = dS = 0); the rest were zeroed at the start.
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int c = 64 * u + lane;
      const int h = c / CPR, ch = c % CPR;
      tq[h * CPR + (ch ^ (h & 7))] = rb.Qa[u];
      tdo[h * CPR + (ch ^ (h & 7))] = rb.dOa[u];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rs.l2[i] = rb.L2[i];
      rs.dh[i] = rb.Dh[i];
    }
    rs.t = a.q_pos0 + rb.row;
  };
  auto compute = [&](const RowState& rs) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4 S = {0.f, 0.f, 0.f, 0.f}, dP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = (quad + 4 * c) ^ (c16 & 7);
      const int kch = (quad + 4 * c) ^ (c16 & 3);
      S = mfma_16x16x32(tq[c16 * (D / 8) + ch], tkv[(c16 & 3) * (D / 8) + kch], S);
      dP = mfma_16x16x32(tdo[c16 * (D / 8) + ch], tkv[(4 + (c16 & 3)) * (D / 8) + kch], dP);
    }
    // Row 4*quad+i is head 4*quad+i; column c16 is token kb*4 + c16.
    float pv[4], ds[4];
    const bool key_ok = c16 < 4 && kb * 4 + c16 <= rs.t && kb * 4 + c16 < a.lk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = key_ok && 4 * quad + i < G;
      pv[i] = ok ? exp2f(S[i] * sl2 - rs.l2[i]) : 0.f;
      ds[i] = pv[i] * (dP[i] - rs.dh[i]);
    }
    const uint2 Ap = make_uint2(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]));
    const uint2 As = make_uint2(pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]));
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      uint4 Rr[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int h = 4 * quad + kk;
        Rr[kk] = tdo[h * (D / 8) + ((c16 + 16 * hf) ^ (h & 7))];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) dV[hf * 8 + e] = mfma_16x16x16(Ap, bwd_repack(Rr, e), dV[hf * 8 + e]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int h = 4 * quad + kk;
        Rr[kk] = tq[h * (D / 8) + ((c16 + 16 * hf) ^ (h & 7))];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) dK[hf * 8 + e] = mfma_16x16x16(As, bwd_repack(Rr, e), dK[hf * 8 + e]);
    }
    // The next row's tile stores must not pass these reads.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  if (p0 < p1) {
    // Loads are unconditional (past the list: the last row again, in bounds), so that
    // every wait counts exactly one row's loads.
    RowBuf B0, B1;
    RowState st;
    load_row(B0, p0);
    load_row(B1, min(p0 + 1, p1 - 1));
    for (int32_t p = p0; p < p1; p += 2) {
      stage(B0, st);
      load_row(B0, min(p + 2, p1 - 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(st);
      stage(B1, st);
      load_row(B1, min(p + 3, p1 - 1));
      __builtin_amdgcn_sched_barrier(0);
      if (p + 1 < p1) compute(st);
    }
  }

  // Rows 0..3 of the accumulators are the block's keys (quad 0 lanes): dims
  // hf*128 + 8*c16 + e. Keys of the block nobody kept get zeros.
  if (quad == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t tk = kb * 4 + i;
      if (tk >= a.lk) break;
      float* kp = a.dk + (tk * a.hkv + g) * (int64_t)D + c16 * 8;
      float* vp = a.dv + (tk * a.hkv + g) * (int64_t)D + c16 * 8;
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        *reinterpret_cast<float4*>(kp + hf * 128) =
            make_float4(dK[hf * 8 + 0][i] * a.scale, dK[hf * 8 + 1][i] * a.scale,
                        dK[hf * 8 + 2][i] * a.scale, dK[hf * 8 + 3][i] * a.scale);
        *reinterpret_cast<float4*>(kp + hf * 128 + 4) =
            make_float4(dK[hf * 8 + 4][i] * a.scale, dK[hf * 8 + 5][i] * a.scale,
                        dK[hf * 8 + 6][i] * a.scale, dK[hf * 8 + 7][i] * a.scale);
        *reinterpret_cast<float4*>(vp + hf * 128) =
            make_float4(dV[hf * 8 + 0][i], dV[hf * 8 + 1][i], dV[hf * 8 + 2][i], dV[hf * 8 + 3][i]);
        *reinterpret_cast<float4*>(vp + hf * 128 + 4) =
            make_float4(dV[hf * 8 + 4][i], dV[hf * 8 + 5][i], dV[hf * 8 + 6][i], dV[hf * 8 + 7][i]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.f;
}

// ---- host side ------------------------------------------------------------------------

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = min((n + 255) / 256, (int64_t)65536);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

static size_t bwd_align(size_t n) { return (n + 255) & ~size_t(255); }

static int bwd_key_bits(int64_t n_kb) {
  int bits = 1;
  while (((int64_t)1 << bits) <= n_kb) ++bits;  // keys 0 .. n_kb (padding) fit
  return bits;
}

// Radix-sort scratch: queried from rocPRIM when a device answers, else a bound.
static size_t bwd_sort_temp_bytes(int64_t n_pairs, int64_t n_kb) {
  size_t bytes = 0;
  rocprim::double_buffer<int32_t> kd(nullptr, nullptr), vd(nullptr, nullptr);
  const hipError_t e = rocprim::radix_sort_pairs(nullptr, bytes, kd, vd, (unsigned)n_pairs, 0,
                                                 bwd_key_bits(n_kb), (hipStream_t)0);
  if (e == hipSuccess) return bytes;
  (void)hipGetLastError();  // no device here: the sort's histograms and look-back state
  return (size_t)(n_pairs / 8) + ((size_t)64 << 20);
}

BwdLayout bwd_layout(int64_t lq, int64_t lk, int hq, int n_sel, int r) {
  BwdLayout L{};
  const int64_t n_pairs = lq * n_sel;
  const int64_t n_kb = (lk + r - 1) / r;
  size_t off = 0;
  L.dbuf = off;
  off += bwd_align((size_t)lq * hq * sizeof(float));
  L.keys0 = off;
  off += bwd_align((size_t)n_pairs * sizeof(int32_t));
  L.keys1 = off;
  off += bwd_align((size_t)n_pairs * sizeof(int32_t));
  L.rows0 = off;
  off += bwd_align((size_t)n_pairs * sizeof(int32_t));
  L.rows1 = off;
  off += bwd_align((size_t)n_pairs * sizeof(int32_t));
  L.start = off;
  off += bwd_align((size_t)(n_kb + 1) * sizeof(int32_t));
  L.temp = off;
  L.temp_bytes = bwd_sort_temp_bytes(n_pairs, n_kb);
  off += bwd_align(L.temp_bytes);
  L.total = off;
  return L;
}

hipError_t launch_sparse_attn_bwd(BwdArgs a, char* ws, size_t ws_bytes, hipStream_t stream) {
  if (a.lq <= 0) return hipSuccess;
  const BwdLayout L = bwd_layout(a.lq, a.lk, a.hq, a.n_sel, 4);
  const int64_t n_pairs = a.lq * a.n_sel;
  a.dbuf = reinterpret_cast<float*>(ws + L.dbuf);
  int32_t* keys0 = reinterpret_cast<int32_t*>(ws + L.keys0);
  int32_t* keys1 = reinterpret_cast<int32_t*>(ws + L.keys1);
  int32_t* rows0 = reinterpret_cast<int32_t*>(ws + L.rows0);
  int32_t* rows1 = reinterpret_cast<int32_t*>(ws + L.rows1);
  a.start = reinterpret_cast<int32_t*>(ws + L.start);

  hipLaunchKernelGGL(bwd_pairs_kernel, dim3((unsigned)((n_pairs + 255) / 256)), dim3(256), 0,
                     stream, a.sel, n_pairs, a.n_sel, (int32_t)a.n_kb, keys0, rows0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The scratch the sort needs on this device must fit the reserved part.
  size_t need = 0;
  rocprim::double_buffer<int32_t> kd(keys0, keys1), vd(rows0, rows1);
  e = rocprim::radix_sort_pairs(nullptr, need, kd, vd, (unsigned)n_pairs, 0,
                                bwd_key_bits(a.n_kb), stream);
  if (e != hipSuccess) return e;
  if (need > L.temp_bytes || L.total > ws_bytes) return hipErrorInvalidValue;
  size_t have = L.temp_bytes;
  e = rocprim::radix_sort_pairs(ws + L.temp, have, kd, vd, (unsigned)n_pairs, 0,
                                bwd_key_bits(a.n_kb), stream);
  if (e != hipSuccess) return e;
  a.pair_rows = vd.current();
  hipLaunchKernelGGL(bwd_starts_kernel, dim3((unsigned)((a.n_kb + 1 + 255) / 256)), dim3(256), 0,
                     stream, kd.current(), n_pairs, (int32_t)a.n_kb, a.start);
  const dim3 gq((unsigned)((a.lq * a.hkv + 3) / 4));
  const dim3 gk((unsigned)((a.n_kb * a.hkv + 3) / 4));
  const int nl = (a.hq / a.hkv * a.d + 511) / 512;  // 1 KiB loads per row and group
  if (a.d == 256) {
    hipLaunchKernelGGL(sparse_attn_bwd_dq_kernel<256>, gq, dim3(256), 0, stream, a);
    switch (nl) {
#define QSA_DKDV(N) \
  case N: hipLaunchKernelGGL((sparse_attn_bwd_dkdv_kernel<256, N>), gk, dim3(256), 0, stream, a); break;
      QSA_DKDV(1) QSA_DKDV(2) QSA_DKDV(3) QSA_DKDV(4) QSA_DKDV(5) QSA_DKDV(6) QSA_DKDV(7)
      QSA_DKDV(8)
#undef QSA_DKDV
      default: return hipErrorInvalidValue;
    }
  } else {
    hipLaunchKernelGGL(sparse_attn_bwd_dq_kernel<128>, gq, dim3(256), 0, stream, a);
    switch (nl) {
#define QSA_DKDV(N) \
  case N: hipLaunchKernelGGL((sparse_attn_bwd_dkdv_kernel<128, N>), gk, dim3(256), 0, stream, a); break;
      QSA_DKDV(1) QSA_DKDV(2) QSA_DKDV(3) QSA_DKDV(4)
#undef QSA_DKDV
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace qsa

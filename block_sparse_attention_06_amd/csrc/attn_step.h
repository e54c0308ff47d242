// One step of the prefill and decode attention: 4 kept blocks (16 keys) of one
// (query, KV group), gathered into MFMA operands, and the online-softmax update
// that consumes them. Shared by the per-row kernels and the multi-row tile.
//
// Method ("Qwen3.8-Flash-Next" Miles recipe, section 1 "Model Introduction"):
// attention reads only the key tokens the indexer kept for each query.
//
//   S^T[16 keys x 16 heads] = K[16 x d] . Q^T        d/32 x v_mfma_f32_16x16x32_bf16
//   O[16 heads x d] += P[16 x 16 keys] . V[16 keys x d]   d/16 x v_mfma_f32_16x16x16_bf16
// (the operand layouts and the permuted output columns are described where the
// kernels are.)
#pragma once

#include "qsa_device.h"

namespace qsa {

constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ uint32_t half_of(uint32_t w, int hi) { return hi ? (w >> 16) : (w & 0xffffu); }

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// One step = 4 kept blocks (16 keys) of one (query, KV group): the operands of a
// step, gathered straight from global memory.
template <int D>
struct AttnStep {
  static constexpr int NC = D / 32;   // k-chunks of Q.K^T
  static constexpr int NH = D / 128;  // 128-dim halves
  uint4 Kc[NC];
  uint4 Vr[4][NH];
};

__device__ __forceinline__ int pick4(int b0, int b1, int b2, int b3, int i) {
  return i == 0 ? b0 : (i == 1 ? b1 : (i == 2 ? b2 : b3));
}

// Row of kb/vb holding token `i` (0..3) of kept block b: the token clamped to the
// query's position t, at that block's place p (in units of 4 rows) in a paged pool, or
// at its own position in a contiguous cache. Padding (b < 0) reads row 0. For a paged
// pool the offset stays inside the block, so a block after t (not a valid selection)
// still reads inside the pool.
__device__ __forceinline__ int64_t attn_row(int b, int p, int i, int64_t t, bool paged) {
  if (b < 0) return 0;
  const int64_t tl = min((int64_t)b * 4 + i, t);
  if (!paged) return tl;
  const int64_t off = tl - (int64_t)b * 4;
  return (int64_t)p * 4 + (off < 0 ? 0 : off);
}

// V rows of one step: this lane's 4 keys are the 4 tokens of block slot `quad`, 16
// contiguous bytes (8 dims) of each per 128-dim half.
template <int D>
__device__ __forceinline__ void attn_load_v(AttnStep<D>& st, const int (&b4)[4], const int (&p4)[4],
                                            bool paged, const uint16_t* vb, int64_t kstride, int g,
                                            int64_t t, int c16, int quad) {
  const int bv = pick4(b4[0], b4[1], b4[2], b4[3], quad);
  const int pv = pick4(p4[0], p4[1], p4[2], p4[3], quad);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int64_t tv = attn_row(bv, pv, kk, t, paged);
    const uint16_t* vp = vb + tv * kstride + g * D + c16 * 8;
#pragma unroll
    for (int hf = 0; hf < AttnStep<D>::NH; ++hf) st.Vr[kk][hf] = ld16(vp + hf * 128);
  }
}

// Issues the loads of one step. Block ids < 0 (padding) and keys after position t
// read an in-bounds row that the softmax masks. b4 holds the kept blocks' ids (token
// positions); with a paged pool, p4 holds their places in it (units of 4 rows).
template <int D>
__device__ __forceinline__ void attn_load_step(AttnStep<D>& st, const int (&b4)[4],
                                               const int (&p4)[4], bool paged,
                                               const uint16_t* kb, const uint16_t* vb,
                                               int64_t kstride, int g, int64_t t, int c16,
                                               int quad) {
  // K rows: key (c16) = token (c16 & 3) of block slot (c16 >> 2).
  const int bk = pick4(b4[0], b4[1], b4[2], b4[3], c16 >> 2);
  const int pk = pick4(p4[0], p4[1], p4[2], p4[3], c16 >> 2);
  const int64_t tk = attn_row(bk, pk, c16 & 3, t, paged);
  const uint16_t* kp = kb + tk * kstride + g * D + quad * 8;
#pragma unroll
  for (int c = 0; c < AttnStep<D>::NC; ++c) st.Kc[c] = ld16(kp + c * 32);
  attn_load_v<D>(st, b4, p4, paged, vb, kstride, g, t, c16, quad);
}

// S^T = K.Q^T, online softmax update of (m_run, l_run), O = O*alpha + P.V.
template <int D>
__device__ __forceinline__ void attn_compute_step(const AttnStep<D>& st, const int (&b4)[4],
                                                  const uint4 (&Qc)[D / 32], f32x4 (&O)[D / 16],
                                                  float& m_run, float& l_run, float sl2,
                                                  int64_t t, int quad) {
  constexpr int NC = D / 32, NH = D / 128, NT = D / 16;
  f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NC; ++c) S = mfma_16x16x32(st.Kc[c], Qc[c], S);

  // Row 4*quad+i of S^T is token bv*4 + i.
  const int bv = pick4(b4[0], b4[1], b4[2], b4[3], quad);
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = bv >= 0 && (int64_t)bv * 4 + i <= t;
    x[i] = ok ? S[i] * sl2 : -INFINITY;
  }
  float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  mt = wave_xor_max(mt, 16);
  mt = wave_xor_max(mt, 32);
  const float m_new = fmaxf(m_run, mt);
  const float alpha = exp2f(m_run - m_new);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = exp2f(x[i] - m_new);
  l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
  const bool moved = m_new != m_run;
  m_run = m_new;

  // Rescale O only when some head's running max moved: otherwise every alpha is
  // exactly 1 and the multiplies change nothing. After the first steps a new maximum
  // is rare, so most steps skip the 64 multiplies (the result is bit-identical).
  if (__any(moved)) {
    float ai[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * quad + i, kWave);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) O[n][i] *= ai[i];
    }
  }

  const uint2 P = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int wi = e >> 1, hi = e & 1;
      const uint32_t lo =
          half_of(word_of(st.Vr[0][hf], wi), hi) | (half_of(word_of(st.Vr[1][hf], wi), hi) << 16);
      const uint32_t up =
          half_of(word_of(st.Vr[2][hf], wi), hi) | (half_of(word_of(st.Vr[3][hf], wi), hi) << 16);
      O[hf * 8 + e] = mfma_16x16x16(P, make_uint2(lo, up), O[hf * 8 + e]);
    }
  }
}

// Q^T as the B operand: column = head c16 of the group, k = dims 32c + 8*quad + [0..7].
template <int D>
__device__ __forceinline__ void attn_load_q(uint4 (&Qc)[D / 32], const uint16_t* qrow, int g,
                                            int G, int c16, int quad) {
  const bool hv = c16 < G;
  const uint16_t* qp = qrow + (int64_t)(g * G + (hv ? c16 : 0)) * D + quad * 8;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) Qc[c] = hv ? ld16(qp + c * 32) : make_uint4(0, 0, 0, 0);
}

}  // namespace qsa

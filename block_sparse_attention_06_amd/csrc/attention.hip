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
// time (16 keys); the kept blocks of neighbouring queries are unrelated, so each
// wave gathers its own K/V straight from global memory into MFMA operands -- no
// LDS round trip and no cross-wave synchronisation.
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
// Decode splits each sequence's kept blocks over waves and writes (m, l, o)
// partials that a second kernel combines.

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ uint32_t half_of(uint32_t w, int hi) { return hi ? (w >> 16) : (w & 0xffffu); }

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <int D, bool DECODE>
__global__ __launch_bounds__(256) void sparse_attn_kernel(AttnArgs a) {
  constexpr int NC = D / 32;   // k-chunks of Q.K^T
  constexpr int NH = D / 128;  // 128-dim halves
  constexpr int NT = D / 16;   // output dim tiles
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int quad = lane >> 4;
  const int G = a.hq / a.hkv;

  const int64_t item = (int64_t)blockIdx.x * 4 + wave;
  int64_t row, t;
  int g, split = 0, s_begin, s_end;
  const uint16_t *kb, *vb;
  const int n_steps = (a.n_sel + 3) / 4;
  if (!DECODE) {
    row = item / a.hkv;
    g = (int)(item - row * a.hkv);
    if (row >= a.lq) return;
    t = a.q_pos0 + row;
    kb = a.k;
    vb = a.v;
    s_begin = 0;
    s_end = n_steps;
  } else {
    const int64_t per_seq = (int64_t)a.hkv * a.n_split;
    row = item / per_seq;
    if (row >= a.lq) return;
    const int rem = (int)(item - row * per_seq);
    g = rem / a.n_split;
    split = rem - g * a.n_split;
    t = (int64_t)a.seq_lens[row] - 1;
    kb = a.k + row * a.cache_bs;
    vb = a.v + row * a.cache_bs;
    s_begin = split * a.steps_per_split;
    s_end = min(s_begin + a.steps_per_split, n_steps);
    if (t < 0) s_end = s_begin;
  }
  const int32_t* srow = a.sel + row * a.n_sel;
  const uint16_t* qrow = a.q + row * (int64_t)a.hq * D;
  const int64_t kstride = (int64_t)a.hkv * D;  // elements between consecutive tokens

  // Q^T as the B operand: column = head c16 of this group, k = dims 32c + 8*quad + [0..7].
  uint4 Qc[NC];
  {
    const bool hv = c16 < G;
    const uint16_t* qp = qrow + (int64_t)(g * G + (hv ? c16 : 0)) * D + quad * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) Qc[c] = hv ? ld16(qp + c * 32) : make_uint4(0, 0, 0, 0);
  }

  f32x4 O[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) O[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max (log2 domain) of head c16
  float l_run = 0.f;        // this lane's partial sum for head c16

  const float sl2 = a.scale_log2;
  for (int s = s_begin; s < s_end; ++s) {
    int b4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b4[j] = (4 * s + j < a.n_sel) ? srow[4 * s + j] : -1;
    if (b4[0] < 0) break;  // -1 padding reached

    // K rows: key (c16) = token (c16 & 3) of block slot (c16 >> 2).
    const int slot_k = c16 >> 2;
    const int bk = slot_k == 0 ? b4[0] : (slot_k == 1 ? b4[1] : (slot_k == 2 ? b4[2] : b4[3]));
    int64_t tk = (int64_t)bk * 4 + (c16 & 3);
    tk = bk < 0 ? 0 : min(tk, t);  // masked keys read an in-bounds row
    const uint16_t* kp = kb + tk * kstride + g * D + quad * 8;
    uint4 Kc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) Kc[c] = ld16(kp + c * 32);

    // V rows: this lane's 4 keys are the 4 tokens of block slot `quad`.
    const int bv = quad == 0 ? b4[0] : (quad == 1 ? b4[1] : (quad == 2 ? b4[2] : b4[3]));
    uint4 Vr[4][NH];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      int64_t tv = (int64_t)bv * 4 + kk;
      tv = bv < 0 ? 0 : min(tv, t);
      const uint16_t* vp = vb + tv * kstride + g * D + c16 * 8;
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) Vr[kk][hf] = ld16(vp + hf * 128);
    }

    f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) S = mfma_16x16x32(Kc[c], Qc[c], S);

    // Row 4*quad+i of S^T is token bv*4 + i.
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
    m_run = m_new;

    float ai[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * quad + i, kWave);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) O[n][i] *= ai[i];
    }

    const uint2 P = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1, hi = e & 1;
        const uint32_t lo = half_of(word_of(Vr[0][hf], wi), hi) | (half_of(word_of(Vr[1][hf], wi), hi) << 16);
        const uint32_t up = half_of(word_of(Vr[2][hf], wi), hi) | (half_of(word_of(Vr[3][hf], wi), hi) << 16);
        O[hf * 8 + e] = mfma_16x16x16(P, make_uint2(lo, up), O[hf * 8 + e]);
      }
    }
  }

  float l_tot = wave_xor_sum(l_run, 16);
  l_tot = wave_xor_sum(l_tot, 32);
  float lh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lh[i] = __shfl(l_tot, 4 * quad + i, kWave);

  if (!DECODE) {
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
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hl = 4 * quad + i;
      if (hl < G) {
        const int64_t slot = (row * a.hq + g * G + hl) * (int64_t)a.n_split + split;
        float* op = a.part_o + slot * D + c16 * 8;
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
          *reinterpret_cast<float4*>(op + hf * 128) =
              make_float4(O[hf * 8 + 0][i], O[hf * 8 + 1][i], O[hf * 8 + 2][i], O[hf * 8 + 3][i]);
          *reinterpret_cast<float4*>(op + hf * 128 + 4) =
              make_float4(O[hf * 8 + 4][i], O[hf * 8 + 5][i], O[hf * 8 + 6][i], O[hf * 8 + 7][i]);
        }
      }
    }
    if (quad == 0 && c16 < G) {
      const int64_t slot = (row * a.hq + g * G + c16) * (int64_t)a.n_split + split;
      a.part_ml[slot * 2 + 0] = m_run;
      a.part_ml[slot * 2 + 1] = l_tot;
    }
  }
}

// Combine the decode partials of one (sequence, head): rescale each split's
// (m, l, o) to the common max and normalise. Thread s first holds split s's (m, l)
// (n_split <= D), so every partial is requested at once rather than one after the
// other; then thread `dim` sums its column over the splits, eight loads in flight.
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(AttnArgs a) {
  constexpr int NW = D / 64;
  __shared__ float wgt[D];
  __shared__ float red[2][NW];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = a.n_split;
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
  const float* po = a.part_o + bh * ns * D + tid;
  float acc = 0.f;
  int s = 0;
  for (; s + 8 <= ns; s += 8) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = po[(int64_t)(s + u) * D];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += wgt[s + u] * x[u];
  }
  for (; s < ns; ++s) acc += wgt[s] * po[(int64_t)s * D];
  const float o = L > 0.f ? acc / L : 0.f;
  a.out[bh * D + tid] = (uint16_t)(pack_bf16x2(o, 0.f) & 0xffffu);
  if (a.lse && tid == 0) a.lse[bh] = L > 0.f ? M * kLn2 + logf(L) : -INFINITY;
}

hipError_t launch_sparse_attn_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.lq <= 0) return hipSuccess;
  const int64_t items = a.lq * a.hkv;
  const dim3 grid((unsigned)((items + 3) / 4));
  if (a.d == 256)
    hipLaunchKernelGGL((sparse_attn_kernel<256, false>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((sparse_attn_kernel<128, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

int decode_steps_per_split(int n_sel) {
  const int steps = (n_sel + 3) / 4;
  const int target_splits = 64;
  return steps <= target_splits ? 1 : (steps + target_splits - 1) / target_splits;
}

int decode_num_splits(int n_sel) {
  const int steps = (n_sel + 3) / 4;
  const int sps = decode_steps_per_split(n_sel);
  return (steps + sps - 1) / sps;
}

hipError_t launch_sparse_attn_decode(const AttnArgs& a, hipStream_t stream) {
  if (a.lq <= 0) return hipSuccess;
  if (a.n_split < 1 || a.n_split > a.d) return hipErrorInvalidValue;  // combine: a split per thread
  const int64_t items = a.lq * a.hkv * a.n_split;
  const dim3 grid((unsigned)((items + 3) / 4));
  const dim3 cgrid((unsigned)(a.lq * a.hq));
  if (a.d == 256) {
    hipLaunchKernelGGL((sparse_attn_kernel<256, true>), grid, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((attn_combine_kernel<256>), cgrid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((sparse_attn_kernel<128, true>), grid, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((attn_combine_kernel<128>), cgrid, dim3(128), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace qsa

// The C ABI of libqsa (declared in include/qsa.h): argument checking, error
// reporting, workspace sizing, and the two whole-path drivers. Every check runs
// on the host before anything is enqueued; nothing here allocates, synchronises
// or reads device memory.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "qsa.h"
#include "qsa_internal.h"

// Scratch of qsa_decode_forward_noalloc, for callers that cannot allocate: one copy on
// every GPU the library runs on, held until the process ends. In host code its name
// is a host-side stand-in; only the device address that hipGetSymbolAddress returns
// (noalloc_scratch below) is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[QSA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

qsa_status fail(qsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

qsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return QSA_OK;
  return fail(QSA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define QSA_REQUIRE(cond, st, ...) \
  do {                             \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define QSA_TRY(expr)                    \
  do {                                   \
    const qsa_status st_ = (expr);       \
    if (st_ != QSA_OK) return st_;       \
  } while (0)

// Device address of `scratch` on the current device, looked up once per device (with
// that device current) and kept.
qsa_status noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(QSA_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (es != hipSuccess) return hip_status(es, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(QSA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    addr[dev] = p;
  }
  *out = addr[dev];
  return QSA_OK;
}

qsa_status check_r(int r) {
  QSA_REQUIRE(r == 4, QSA_ERR_UNSUPPORTED, "micro-block size r=%d: only r=4 is supported", r);
  return QSA_OK;
}

qsa_status check_budget(int budget_tokens, int r) {
  QSA_REQUIRE(budget_tokens > 0 && budget_tokens % r == 0, QSA_ERR_INVALID_ARGUMENT,
              "budget_tokens=%d must be a positive multiple of r=%d", budget_tokens, r);
  const int n_sel = budget_tokens / r;
  QSA_REQUIRE(n_sel >= 4 && n_sel <= 1024, QSA_ERR_UNSUPPORTED,
              "budget_tokens/r=%d blocks: supported range is 4..1024", n_sel);
  return QSA_OK;
}

qsa_status check_indexer_shape(int h_idx, int d_idx) {
  QSA_REQUIRE(h_idx >= 1 && h_idx <= 4, QSA_ERR_UNSUPPORTED,
              "indexer heads h_idx=%d: supported 1..4", h_idx);
  QSA_REQUIRE(d_idx == 64 || d_idx == 128, QSA_ERR_UNSUPPORTED,
              "indexer dim d_idx=%d: supported 64 or 128", d_idx);
  return QSA_OK;
}

qsa_status check_attn_shape(int hq, int hkv, int d) {
  QSA_REQUIRE(hq > 0 && hkv > 0 && hq % hkv == 0, QSA_ERR_INVALID_ARGUMENT,
              "hq=%d must be a positive multiple of hkv=%d", hq, hkv);
  QSA_REQUIRE(hq / hkv <= 16, QSA_ERR_UNSUPPORTED, "heads per KV group %d > 16", hq / hkv);
  QSA_REQUIRE(d == 128 || d == 256, QSA_ERR_UNSUPPORTED, "head dim d=%d: supported 128 or 256",
              d);
  return QSA_OK;
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

int64_t score_ld(int64_t nblk) { return (nblk + 3) & ~int64_t(3); }

// The pooled-key encoding of a call: none for NULL or rope_dim 0.
qsa_status pooled_pe(const qsa_pooled_pe* pe, int d_idx, qsa::PooledPe* out) {
  *out = qsa::PooledPe{0, 0.0, 0};
  if (!pe || pe->rope_dim == 0) return QSA_OK;
  QSA_REQUIRE(pe->rope_dim % 16 == 0 && pe->rope_dim >= 16 && pe->rope_dim <= d_idx,
              QSA_ERR_UNSUPPORTED, "rope_dim=%d: a multiple of 16 in 16..d_idx=%d, or 0",
              pe->rope_dim, d_idx);
  QSA_REQUIRE(isfinite(pe->rope_theta) && pe->rope_theta > 1.f, QSA_ERR_INVALID_ARGUMENT,
              "rope_theta=%g must be finite and > 1", (double)pe->rope_theta);
  out->rope_dim = pe->rope_dim;
  out->theta = (double)pe->rope_theta;
  return QSA_OK;
}

}  // namespace

extern "C" {

int qsa_abi_version(void) { return QSA_ABI_VERSION; }

const char* qsa_last_error(void) { return g_err; }

qsa_status qsa_pool_keys(const void* k_idx, int64_t k_idx_row_stride, int64_t n_blocks,
                         int d_idx, int r, void* k_pooled, int64_t k_pooled_row_stride,
                         void* stream) {
  QSA_TRY(check_r(r));
  QSA_REQUIRE(n_blocks >= 0, QSA_ERR_INVALID_ARGUMENT, "n_blocks=%lld < 0", (long long)n_blocks);
  QSA_REQUIRE(d_idx > 0 && d_idx % 8 == 0 && d_idx <= 4096, QSA_ERR_UNSUPPORTED,
              "d_idx=%d must be a multiple of 8 in 8..4096", d_idx);
  if (n_blocks == 0) return QSA_OK;
  QSA_REQUIRE(k_idx && k_pooled, QSA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  QSA_REQUIRE(aligned16(k_idx) && aligned16(k_pooled), QSA_ERR_INVALID_ARGUMENT,
              "k_idx and k_pooled must be 16-byte aligned");
  QSA_REQUIRE(k_idx_row_stride >= d_idx && k_idx_row_stride % 8 == 0 &&
                  k_pooled_row_stride >= d_idx && k_pooled_row_stride % 8 == 0,
              QSA_ERR_INVALID_ARGUMENT,
              "row strides (%lld, %lld) must be >= d_idx and multiples of 8 elements",
              (long long)k_idx_row_stride, (long long)k_pooled_row_stride);
  return hip_status(
      qsa::launch_pool_keys(static_cast<const uint16_t*>(k_idx), k_idx_row_stride, n_blocks,
                            d_idx, r, static_cast<uint16_t*>(k_pooled), k_pooled_row_stride,
                            qsa::PooledPe{0, 0.0, 0}, static_cast<hipStream_t>(stream)),
      "qsa_pool_keys launch");
}

qsa_status qsa_pool_keys_pe(const void* k_idx, int64_t k_idx_row_stride, int64_t n_blocks,
                            int d_idx, int r, int64_t first_block, const qsa_pooled_pe* pe,
                            void* k_pooled, int64_t k_pooled_row_stride, void* stream) {
  qsa::PooledPe p{};
  QSA_TRY(pooled_pe(pe, d_idx, &p));
  QSA_REQUIRE(first_block >= 0, QSA_ERR_INVALID_ARGUMENT, "first_block=%lld < 0",
              (long long)first_block);
  p.first_block = first_block;
  if (p.rope_dim == 0)
    return qsa_pool_keys(k_idx, k_idx_row_stride, n_blocks, d_idx, r, k_pooled,
                         k_pooled_row_stride, stream);
  QSA_TRY(check_r(r));
  QSA_REQUIRE(n_blocks >= 0, QSA_ERR_INVALID_ARGUMENT, "n_blocks=%lld < 0", (long long)n_blocks);
  QSA_REQUIRE(d_idx > 0 && d_idx % 8 == 0 && d_idx <= 4096, QSA_ERR_UNSUPPORTED,
              "d_idx=%d must be a multiple of 8 in 8..4096", d_idx);
  if (n_blocks == 0) return QSA_OK;
  QSA_REQUIRE(k_idx && k_pooled, QSA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  QSA_REQUIRE(aligned16(k_idx) && aligned16(k_pooled), QSA_ERR_INVALID_ARGUMENT,
              "k_idx and k_pooled must be 16-byte aligned");
  QSA_REQUIRE(k_idx_row_stride >= d_idx && k_idx_row_stride % 8 == 0 &&
                  k_pooled_row_stride >= d_idx && k_pooled_row_stride % 8 == 0,
              QSA_ERR_INVALID_ARGUMENT,
              "row strides (%lld, %lld) must be >= d_idx and multiples of 8 elements",
              (long long)k_idx_row_stride, (long long)k_pooled_row_stride);
  return hip_status(
      qsa::launch_pool_keys(static_cast<const uint16_t*>(k_idx), k_idx_row_stride, n_blocks,
                            d_idx, r, static_cast<uint16_t*>(k_pooled), k_pooled_row_stride, p,
                            static_cast<hipStream_t>(stream)),
      "qsa_pool_keys_pe launch");
}

qsa_status qsa_index_scores(int batch, int64_t lq, int h_idx, int d_idx, int r,
                            const void* q_idx, int64_t q_idx_batch_stride, const float* w,
                            int64_t w_batch_stride, const void* k_pooled,
                            int64_t k_pooled_batch_stride, int64_t nblk, int64_t q_pos0,
                            const int32_t* seq_lens, float* scores, int64_t ld,
                            int64_t scores_batch_stride, void* stream) {
  QSA_TRY(check_r(r));
  QSA_TRY(check_indexer_shape(h_idx, d_idx));
  QSA_REQUIRE(batch >= 1 && batch <= 65535, QSA_ERR_INVALID_ARGUMENT, "batch=%d", batch);
  QSA_REQUIRE(lq >= 0 && lq <= ((int64_t)1 << 31) - 64, QSA_ERR_INVALID_ARGUMENT, "lq=%lld",
              (long long)lq);
  QSA_REQUIRE(nblk >= 0 && nblk < ((int64_t)1 << 30), QSA_ERR_INVALID_ARGUMENT, "nblk=%lld",
              (long long)nblk);
  QSA_REQUIRE(seq_lens || q_pos0 >= 0, QSA_ERR_INVALID_ARGUMENT, "q_pos0=%lld < 0",
              (long long)q_pos0);
  QSA_REQUIRE(ld >= nblk && ld % 4 == 0, QSA_ERR_INVALID_ARGUMENT,
              "ld=%lld must be >= nblk=%lld and a multiple of 4", (long long)ld,
              (long long)nblk);
  if (lq == 0 || nblk == 0) return QSA_OK;
  QSA_REQUIRE(q_idx && w && k_pooled && scores, QSA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  QSA_REQUIRE(aligned16(q_idx) && aligned16(k_pooled) && aligned16(scores),
              QSA_ERR_INVALID_ARGUMENT, "q_idx, k_pooled and scores must be 16-byte aligned");
  if (batch > 1) {
    QSA_REQUIRE(q_idx_batch_stride % 8 == 0 && k_pooled_batch_stride % 8 == 0 &&
                    scores_batch_stride % 4 == 0,
                QSA_ERR_INVALID_ARGUMENT, "batch strides break 16-byte alignment");
    QSA_REQUIRE(q_idx_batch_stride >= lq * h_idx * d_idx && w_batch_stride >= lq * h_idx &&
                    k_pooled_batch_stride >= nblk * d_idx && scores_batch_stride >= lq * ld,
                QSA_ERR_INVALID_ARGUMENT, "batch strides overlap consecutive sequences");
  }
  if (!seq_lens) {
    QSA_REQUIRE((q_pos0 + lq - 1) / r <= nblk + (int64_t)0x7fffffff, QSA_ERR_INVALID_ARGUMENT,
                "positions overflow");
  }
  qsa::ScoreArgs a{static_cast<const uint16_t*>(q_idx), q_idx_batch_stride, w, w_batch_stride,
                   static_cast<const uint16_t*>(k_pooled), k_pooled_batch_stride, nblk, lq,
                   h_idx, d_idx, r, q_pos0, seq_lens, scores, ld, scores_batch_stride, batch};
  return hip_status(qsa::launch_index_scores(a, static_cast<hipStream_t>(stream)),
                    "qsa_index_scores launch");
}

qsa::TopkArgs topk_args(int batch, int64_t lq, int r, int budget_tokens, const float* scores,
                        int64_t ld, int64_t sbs, int64_t nblk, int64_t q_pos0,
                        const int32_t* seq_lens, int32_t* sel) {
  return qsa::TopkArgs{scores, ld, sbs, lq, nblk, q_pos0, seq_lens, r, budget_tokens / r, sel,
                       batch};
}

size_t qsa_topk_workspace_bytes(int batch, int64_t lq, int64_t nblk, int budget_tokens, int r) {
  if (batch <= 0 || lq <= 0 || nblk <= 0 || r <= 0 || budget_tokens < r) return 0;
  // Sized for rows whose positions reach the last block (the device may hold seq_lens).
  qsa::TopkArgs a = topk_args(batch, lq, r, budget_tokens, nullptr, nblk, 0, nblk,
                              nblk * (int64_t)r, nullptr, nullptr);
  a.seq_lens = reinterpret_cast<const int32_t*>(1);  // bound by nblk, not by positions
  return qsa::topk_workspace_bytes(a);
}

qsa_status qsa_topk_blocks(int batch, int64_t lq, int r, int budget_tokens, const float* scores,
                           int64_t ld, int64_t scores_batch_stride, int64_t nblk, int64_t q_pos0,
                           const int32_t* seq_lens, int32_t* sel, void* workspace,
                           size_t workspace_bytes, void* stream) {
  QSA_TRY(check_r(r));
  QSA_TRY(check_budget(budget_tokens, r));
  QSA_REQUIRE(batch >= 1 && batch <= 65535, QSA_ERR_INVALID_ARGUMENT, "batch=%d", batch);
  QSA_REQUIRE(lq >= 0 && lq <= ((int64_t)1 << 31) - 1, QSA_ERR_INVALID_ARGUMENT, "lq=%lld",
              (long long)lq);
  QSA_REQUIRE(nblk >= 0 && nblk < ((int64_t)1 << 22), QSA_ERR_UNSUPPORTED,
              "nblk=%lld: top-k supports fewer than 2^22 blocks", (long long)nblk);
  QSA_REQUIRE(seq_lens || q_pos0 >= 0, QSA_ERR_INVALID_ARGUMENT, "q_pos0=%lld < 0",
              (long long)q_pos0);
  QSA_REQUIRE(ld >= nblk && ld % 4 == 0, QSA_ERR_INVALID_ARGUMENT,
              "ld=%lld must be >= nblk and a multiple of 4", (long long)ld);
  if (lq == 0) return QSA_OK;
  QSA_REQUIRE(sel && (scores || nblk == 0), QSA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  QSA_REQUIRE(!scores || aligned16(scores), QSA_ERR_INVALID_ARGUMENT,
              "scores must be 16-byte aligned");
  if (batch > 1)
    QSA_REQUIRE(scores_batch_stride % 4 == 0 && scores_batch_stride >= lq * ld,
                QSA_ERR_INVALID_ARGUMENT, "scores_batch_stride=%lld",
                (long long)scores_batch_stride);
  if (!seq_lens)
    QSA_REQUIRE((q_pos0 + lq - 1) / r < ((int64_t)1 << 31), QSA_ERR_INVALID_ARGUMENT,
                "positions overflow int32 block ids");
  const qsa::TopkArgs a = topk_args(batch, lq, r, budget_tokens, scores, ld,
                                    scores_batch_stride, nblk, q_pos0, seq_lens, sel);
  QSA_REQUIRE(qsa::topk_supported(a), QSA_ERR_UNSUPPORTED,
              "rows of %lld blocks with %d kept blocks exceed the two-level selection",
              (long long)nblk, budget_tokens / r);
  const size_t need = qsa::topk_workspace_bytes(a);
  QSA_REQUIRE(need == 0 || (workspace && workspace_bytes >= need && aligned16(workspace)),
              QSA_ERR_WORKSPACE, "top-k workspace: need %zu bytes (16-byte aligned), got %zu",
              need, workspace_bytes);
  return hip_status(qsa::launch_topk_blocks(a, workspace, static_cast<hipStream_t>(stream)),
                    "qsa_topk_blocks launch");
}

namespace {

// Argument checks of the sparse attention forward, shared by every entry point that
// launches it, so that a call fails before it has launched anything.
qsa_status check_attn_fwd(int64_t lq, int64_t lk, int hq, int hkv, int d, int r, int n_sel,
                          const void* q, const void* k, const void* v, const int32_t* sel,
                          int64_t q_pos0, float softmax_scale, const void* out) {
  QSA_TRY(check_r(r));
  QSA_TRY(check_attn_shape(hq, hkv, d));
  QSA_REQUIRE(n_sel >= 1 && n_sel <= 1024, QSA_ERR_UNSUPPORTED, "n_sel=%d: supported 1..1024",
              n_sel);
  QSA_REQUIRE(lq >= 0 && lq < ((int64_t)1 << 31), QSA_ERR_INVALID_ARGUMENT, "lq=%lld",
              (long long)lq);
  QSA_REQUIRE(q_pos0 >= 0 && q_pos0 + lq <= lk, QSA_ERR_INVALID_ARGUMENT,
              "query positions [%lld, %lld) must lie inside the %lld keys", (long long)q_pos0,
              (long long)(q_pos0 + lq), (long long)lk);
  QSA_REQUIRE(isfinite(softmax_scale), QSA_ERR_INVALID_ARGUMENT, "softmax_scale not finite");
  if (lq == 0) return QSA_OK;
  QSA_REQUIRE(q && k && v && sel && out, QSA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  QSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out),
              QSA_ERR_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
  QSA_REQUIRE(lq * hkv / 4 < ((int64_t)1 << 31), QSA_ERR_INVALID_ARGUMENT, "grid too large");
  return QSA_OK;
}

}  // namespace

qsa_status qsa_sparse_attn_fwd(int64_t lq, int64_t lk, int hq, int hkv, int d, int r, int n_sel,
                               const void* q, const void* k, const void* v, const int32_t* sel,
                               int64_t q_pos0, float softmax_scale, void* out, float* lse,
                               void* stream) {
  QSA_TRY(check_attn_fwd(lq, lk, hq, hkv, d, r, n_sel, q, k, v, sel, q_pos0, softmax_scale,
                         out));
  if (lq == 0) return QSA_OK;
  qsa::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.sel = sel;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.lq = lq;
  a.lk = lk;
  a.q_pos0 = q_pos0;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.n_sel = n_sel;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  return hip_status(qsa::launch_sparse_attn_fwd(a, static_cast<hipStream_t>(stream)),
                    "qsa_sparse_attn_fwd launch");
}

qsa_status qsa_sparse_attn_fwd_tiled(int64_t lq, int64_t lk, int hq, int hkv, int d, int r,
                                     int n_sel, const void* q, const void* k, const void* v,
                                     const int32_t* sel, int64_t q_pos0, float softmax_scale,
                                     int min_shared, void* out, float* lse, void* stream) {
  QSA_TRY(check_attn_fwd(lq, lk, hq, hkv, d, r, n_sel, q, k, v, sel, q_pos0, softmax_scale,
                         out));
  QSA_REQUIRE(n_sel <= qsa::kTileMaxSel, QSA_ERR_UNSUPPORTED,
              "n_sel=%d: the tiled attention holds kept lists of up to %d blocks", n_sel,
              qsa::kTileMaxSel);
  QSA_REQUIRE(min_shared >= 0 && min_shared <= 65, QSA_ERR_INVALID_ARGUMENT,
              "min_shared=%d: 0..64 of 64 sampled blocks, or 65 for never", min_shared);
  if (lq == 0) return QSA_OK;
  qsa::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.sel = sel;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.lq = lq;
  a.lk = lk;
  a.q_pos0 = q_pos0;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.n_sel = n_sel;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  return hip_status(qsa::launch_sparse_attn_fwd_tiled(a, min_shared, static_cast<hipStream_t>(stream)),
                    "qsa_sparse_attn_fwd_tiled launch");
}

int64_t qsa_sparse_attn_fwd_rows_per_launch(int hkv, int d) {
  if (hkv < 1 || (d != 128 && d != 256)) return 0;
  return qsa::sparse_attn_fwd_rows_per_launch(hkv, d);
}

int64_t qsa_sparse_attn_fwd_launches(int64_t lq, int64_t lk, int hkv, int d) {
  if (lq < 0 || lk < 0 || hkv < 1 || (d != 128 && d != 256)) return -1;
  return qsa::sparse_attn_fwd_launches(lq, lk, hkv, d);
}

size_t qsa_sparse_attn_bwd_workspace_bytes(int64_t lq, int64_t lk, int hq, int r, int n_sel) {
  if (lq <= 0 || lk <= 0 || hq <= 0 || r <= 0 || n_sel <= 0) return 0;
  return qsa::bwd_layout(lq, lk, hq, n_sel, r).total;
}

qsa_status qsa_sparse_attn_bwd(int64_t lq, int64_t lk, int hq, int hkv, int d, int r, int n_sel,
                               const void* q, const void* k, const void* v, const int32_t* sel,
                               int64_t q_pos0, float softmax_scale, const void* out,
                               const float* lse, const void* dout, float* dq, float* dk,
                               float* dv, void* workspace, size_t workspace_bytes, void* stream) {
  QSA_TRY(check_r(r));
  QSA_TRY(check_attn_shape(hq, hkv, d));
  QSA_REQUIRE(n_sel >= 1 && n_sel <= 1024, QSA_ERR_UNSUPPORTED, "n_sel=%d: supported 1..1024",
              n_sel);
  QSA_REQUIRE(lq >= 0 && lq * (int64_t)n_sel < ((int64_t)1 << 31), QSA_ERR_INVALID_ARGUMENT,
              "lq=%lld: lq * n_sel must stay below 2^31", (long long)lq);
  QSA_REQUIRE(lk >= 1 && lk < ((int64_t)1 << 31), QSA_ERR_INVALID_ARGUMENT, "lk=%lld",
              (long long)lk);
  QSA_REQUIRE(q_pos0 >= 0 && q_pos0 + lq <= lk, QSA_ERR_INVALID_ARGUMENT,
              "query positions [%lld, %lld) must lie inside the %lld keys", (long long)q_pos0,
              (long long)(q_pos0 + lq), (long long)lk);
  QSA_REQUIRE(isfinite(softmax_scale), QSA_ERR_INVALID_ARGUMENT, "softmax_scale not finite");
  QSA_REQUIRE(k && v && dk && dv, QSA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  QSA_REQUIRE(aligned16(k) && aligned16(v) && aligned16(dk) && aligned16(dv),
              QSA_ERR_INVALID_ARGUMENT, "k, v, dk and dv must be 16-byte aligned");
  QSA_REQUIRE(lq == 0 || (q && sel && out && lse && dout && dq), QSA_ERR_INVALID_ARGUMENT,
              "null tensor pointer");
  QSA_REQUIRE(lq == 0 || (aligned16(q) && aligned16(out) && aligned16(dout) && aligned16(dq)),
              QSA_ERR_INVALID_ARGUMENT, "q, out, dout and dq must be 16-byte aligned");
  const size_t need = qsa_sparse_attn_bwd_workspace_bytes(lq, lk, hq, r, n_sel);
  QSA_REQUIRE(lq == 0 || (workspace && workspace_bytes >= need && aligned16(workspace)),
              QSA_ERR_WORKSPACE, "backward workspace: need %zu bytes (16-byte aligned), got %zu",
              need, workspace_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (lq == 0) {  // no query reads any key: zero gradients (a fill kernel, not a memset)
    QSA_TRY(hip_status(qsa::launch_fill_zero(dk, lk * hkv * d, s), "dk clear"));
    return hip_status(qsa::launch_fill_zero(dv, lk * hkv * d, s), "dv clear");
  }
  qsa::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.sel = sel;
  a.out = static_cast<const uint16_t*>(out);
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.lq = lq;
  a.lk = lk;
  a.q_pos0 = q_pos0;
  a.n_kb = (lk + r - 1) / r;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.n_sel = n_sel;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  return hip_status(qsa::launch_sparse_attn_bwd(a, static_cast<char*>(workspace), workspace_bytes,
                                                s),
                    "qsa_sparse_attn_bwd launch (or sort scratch larger than reserved)");
}

// ---- indexer warm-up ----

qsa_status qsa_indexer_kl_target(int64_t lq, int64_t lk, int hq, int hkv, int d, int r,
                                 const void* q, const void* k, int64_t q_pos0,
                                 float softmax_scale, float* lse, float* target, int64_t ld,
                                 void* stream) {
  QSA_TRY(check_r(r));
  QSA_TRY(check_attn_shape(hq, hkv, d));
  QSA_REQUIRE(hkv <= qsa::kKlMaxGroups, QSA_ERR_UNSUPPORTED,
              "hkv=%d: the dense KL passes take up to %d KV groups", hkv, qsa::kKlMaxGroups);
  QSA_REQUIRE(lq >= 0 && lq < ((int64_t)1 << 31) && lk >= 1, QSA_ERR_INVALID_ARGUMENT,
              "lq=%lld lk=%lld", (long long)lq, (long long)lk);
  QSA_REQUIRE(q_pos0 >= 0 && q_pos0 + lq <= lk, QSA_ERR_INVALID_ARGUMENT,
              "query positions [%lld, %lld) must lie inside the %lld keys", (long long)q_pos0,
              (long long)(q_pos0 + lq), (long long)lk);
  QSA_REQUIRE(isfinite(softmax_scale), QSA_ERR_INVALID_ARGUMENT, "softmax_scale not finite");
  const int64_t nblk = lk / r;
  QSA_REQUIRE(ld >= nblk && ld % 4 == 0, QSA_ERR_INVALID_ARGUMENT,
              "ld=%lld: needs ld >= lk / r = %lld and ld %% 4 == 0", (long long)ld,
              (long long)nblk);
  if (lq == 0) return QSA_OK;
  QSA_REQUIRE(q && k && lse && target, QSA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  QSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(target), QSA_ERR_INVALID_ARGUMENT,
              "q, k and target must be 16-byte aligned");
  qsa::KlArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), lse, target,
                lq, lk, q_pos0, nblk, ld, hq, hkv, d, r,
                softmax_scale * 1.4426950408889634f};
  return hip_status(qsa::launch_kl_target(a, static_cast<hipStream_t>(stream)),
                    "qsa_indexer_kl_target launch");
}

qsa_status qsa_indexer_kl_loss(int64_t lq, int64_t nblk, int r, int64_t q_pos0,
                               const float* scores, const float* target, int64_t ld,
                               float* loss, float* dscores, void* stream) {
  QSA_TRY(check_r(r));
  QSA_REQUIRE(lq >= 0 && lq < ((int64_t)1 << 31) && nblk >= 0 && q_pos0 >= 0,
              QSA_ERR_INVALID_ARGUMENT, "lq=%lld nblk=%lld q_pos0=%lld", (long long)lq,
              (long long)nblk, (long long)q_pos0);
  QSA_REQUIRE(ld >= nblk && ld % 4 == 0, QSA_ERR_INVALID_ARGUMENT, "ld=%lld", (long long)ld);
  if (lq == 0) return QSA_OK;
  QSA_REQUIRE(scores && target && loss && dscores, QSA_ERR_INVALID_ARGUMENT,
              "null tensor pointer");
  qsa::KlLossArgs a{scores, target, loss, dscores, lq, q_pos0, nblk, ld, r};
  return hip_status(qsa::launch_kl_loss(a, static_cast<hipStream_t>(stream)),
                    "qsa_indexer_kl_loss launch");
}

qsa_status qsa_index_scores_bwd(int64_t lq, int h_idx, int d_idx, int r, const void* q_idx,
                                const float* w, const void* k_pooled, int64_t nblk,
                                int64_t q_pos0, const float* dscores, int64_t ld,
                                float* dq_idx, float* dw, float* dk_pooled, float* dk_idx,
                                int64_t n_tokens, void* stream) {
  QSA_TRY(check_r(r));
  QSA_TRY(check_indexer_shape(h_idx, d_idx));
  QSA_REQUIRE(lq >= 0 && lq < ((int64_t)1 << 31) && nblk >= 0 && nblk < ((int64_t)1 << 31) &&
                  q_pos0 >= 0,
              QSA_ERR_INVALID_ARGUMENT, "lq=%lld nblk=%lld q_pos0=%lld", (long long)lq,
              (long long)nblk, (long long)q_pos0);
  QSA_REQUIRE(ld >= nblk && ld % 4 == 0, QSA_ERR_INVALID_ARGUMENT, "ld=%lld", (long long)ld);
  QSA_REQUIRE(!dk_idx || (n_tokens >= 0 && n_tokens < ((int64_t)1 << 40)),
              QSA_ERR_INVALID_ARGUMENT, "n_tokens=%lld", (long long)n_tokens);
  QSA_REQUIRE(q_idx && w && dscores && dq_idx && dw && (nblk == 0 || (k_pooled && dk_pooled)),
              QSA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  QSA_REQUIRE(aligned16(q_idx) && aligned16(dscores) && aligned16(dq_idx) &&
                  (nblk == 0 || (aligned16(k_pooled) && aligned16(dk_pooled))),
              QSA_ERR_INVALID_ARGUMENT, "q_idx, k_pooled, dscores and outputs must be 16-byte aligned");
  qsa::IdxBwdArgs a{static_cast<const uint16_t*>(q_idx), w,
                    static_cast<const uint16_t*>(k_pooled), dscores, dq_idx, dw, dk_pooled,
                    dk_idx, lq, q_pos0, nblk, ld, dk_idx ? n_tokens : 0, h_idx, d_idx, r};
  return hip_status(qsa::launch_index_scores_bwd(a, static_cast<hipStream_t>(stream)),
                    "qsa_index_scores_bwd launch");
}

size_t qsa_sparse_attn_decode_workspace_bytes(int batch, int hq, int d, int n_sel) {
  if (batch <= 0 || hq <= 0 || d <= 0 || n_sel <= 0) return 0;
  const size_t ns = (size_t)qsa::decode_num_splits(n_sel);
  const size_t slots = (size_t)batch * hq * ns;
  return align256(slots * d * sizeof(float)) + align256(slots * 2 * sizeof(float));
}

namespace {

// A paged K/V cache: pools of num_pages pages of page_size tokens ([slot][hkv][d],
// slot = page * page_size + offset); page p of sequence s is table[s * table_stride + p].
struct PagedKV {
  const int32_t* table;
  int64_t table_stride;
  int page_size;
  int64_t num_pages;
};

qsa_status check_paged(const PagedKV& p, int r, int64_t lmax) {
  QSA_REQUIRE(p.table, QSA_ERR_INVALID_ARGUMENT, "null block table");
  QSA_REQUIRE(p.page_size >= r && p.page_size % r == 0 && p.page_size <= (1 << 20),
              QSA_ERR_UNSUPPORTED, "page_size=%d: a multiple of r=%d up to 2^20 (a block of r "
              "tokens must not straddle pages)", p.page_size, r);
  QSA_REQUIRE(p.num_pages >= 1 && p.num_pages * (p.page_size / r) < ((int64_t)1 << 31),
              QSA_ERR_INVALID_ARGUMENT, "num_pages=%lld", (long long)p.num_pages);
  QSA_REQUIRE(p.table_stride >= (lmax + p.page_size - 1) / p.page_size,
              QSA_ERR_INVALID_ARGUMENT,
              "table_stride=%lld holds fewer pages than lmax=%lld tokens need",
              (long long)p.table_stride, (long long)lmax);
  return QSA_OK;
}

qsa_status sparse_attn_decode_impl(int batch, int hq, int hkv, int d, int r, int n_sel,
                                   const void* q, const void* k_cache, const void* v_cache,
                                   int64_t cache_batch_stride, int64_t lmax,
                                   const PagedKV* paged, const int32_t* seq_lens,
                                   const int32_t* sel, float softmax_scale, void* out,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  QSA_TRY(check_r(r));
  QSA_TRY(check_attn_shape(hq, hkv, d));
  QSA_REQUIRE(n_sel >= 1 && n_sel <= 1024, QSA_ERR_UNSUPPORTED, "n_sel=%d: supported 1..1024",
              n_sel);
  QSA_REQUIRE(batch >= 1 && batch <= (1 << 20), QSA_ERR_INVALID_ARGUMENT, "batch=%d", batch);
  QSA_REQUIRE(lmax >= 1, QSA_ERR_INVALID_ARGUMENT, "lmax=%lld", (long long)lmax);
  QSA_REQUIRE(isfinite(softmax_scale), QSA_ERR_INVALID_ARGUMENT, "softmax_scale not finite");
  QSA_REQUIRE(q && k_cache && v_cache && seq_lens && sel && out, QSA_ERR_INVALID_ARGUMENT,
              "null tensor pointer");
  QSA_REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(out),
              QSA_ERR_INVALID_ARGUMENT, "q, caches and out must be 16-byte aligned");
  if (paged) {
    QSA_TRY(check_paged(*paged, r, lmax));
  } else {
    QSA_REQUIRE(batch == 1 || (cache_batch_stride % 8 == 0 &&
                               cache_batch_stride >= lmax * (int64_t)hkv * d),
                QSA_ERR_INVALID_ARGUMENT, "cache_batch_stride=%lld",
                (long long)cache_batch_stride);
  }
  const size_t need = qsa_sparse_attn_decode_workspace_bytes(batch, hq, d, n_sel);
  QSA_REQUIRE(workspace && workspace_bytes >= need && aligned16(workspace), QSA_ERR_WORKSPACE,
              "decode workspace: need %zu bytes (16-byte aligned), got %zu", need,
              workspace_bytes);
  const int ns = qsa::decode_num_splits(n_sel);
  const size_t slots = (size_t)batch * hq * ns;
  qsa::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.sel = sel;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.lq = batch;
  a.lk = lmax;
  a.seq_lens = seq_lens;
  a.cache_bs = cache_batch_stride;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.n_sel = n_sel;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       align256(slots * d * sizeof(float)));
  a.n_split = ns;
  a.steps_per_split = qsa::decode_steps_per_split(n_sel);
  if (paged) {
    a.block_table = paged->table;
    a.table_stride = paged->table_stride;
    a.page_blocks = paged->page_size / r;
    a.num_pages = (int)paged->num_pages;
  }
  return hip_status(qsa::launch_sparse_attn_decode(a, static_cast<hipStream_t>(stream)),
                    "decode attention launch");
}

}  // namespace

qsa_status qsa_sparse_attn_decode(int batch, int hq, int hkv, int d, int r, int n_sel,
                                  const void* q, const void* k_cache, const void* v_cache,
                                  int64_t cache_batch_stride, int64_t lmax,
                                  const int32_t* seq_lens, const int32_t* sel,
                                  float softmax_scale, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return sparse_attn_decode_impl(batch, hq, hkv, d, r, n_sel, q, k_cache, v_cache,
                                 cache_batch_stride, lmax, nullptr, seq_lens, sel,
                                 softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

qsa_status qsa_sparse_attn_decode_paged(int batch, int hq, int hkv, int d, int r, int n_sel,
                                        const void* q, const void* k_pool, const void* v_pool,
                                        int64_t num_pages, int page_size,
                                        const int32_t* block_table, int64_t table_stride,
                                        int64_t lmax, const int32_t* seq_lens,
                                        const int32_t* sel, float softmax_scale, void* out,
                                        float* lse, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  const PagedKV pk{block_table, table_stride, page_size, num_pages};
  return sparse_attn_decode_impl(batch, hq, hkv, d, r, n_sel, q, k_pool, v_pool, 0, lmax, &pk,
                                 seq_lens, sel, softmax_scale, out, lse, workspace,
                                 workspace_bytes, stream);
}

// ---- whole prefill path ----

size_t qsa_prefill_workspace_bytes(int64_t lq, int64_t lk, int r, int budget_tokens,
                                   int64_t row_chunk) {
  if (lq <= 0 || lk <= 0 || r <= 0) return 0;
  const int64_t rc = row_chunk > 0 ? (row_chunk < lq ? row_chunk : lq) : lq;
  return align256((size_t)rc * (size_t)score_ld(lk / r) * sizeof(float)) +
         qsa_topk_workspace_bytes(1, rc, lk / r, budget_tokens, r);
}

namespace {

// Checks shared by both prefill selections, then the pooling of the new blocks (and
// the copy of a pooled prefix into k_pooled).
qsa_status prefill_pool(int64_t lq, int64_t lk, int64_t q_pos0, int h_idx, int d_idx, int r,
                        int budget_tokens, const void* k_idx, int64_t first_raw_token,
                        const void* k_pooled_prefix, void* k_pooled, const qsa_pooled_pe* pe,
                        size_t need, void* workspace, size_t workspace_bytes, void* stream) {
  QSA_TRY(check_r(r));
  qsa::PooledPe ppe{};
  QSA_TRY(pooled_pe(pe, d_idx, &ppe));
  QSA_TRY(check_budget(budget_tokens, r));
  QSA_TRY(check_indexer_shape(h_idx, d_idx));
  QSA_REQUIRE(lq >= 0 && lk >= 1 && q_pos0 >= 0 && q_pos0 + lq <= lk, QSA_ERR_INVALID_ARGUMENT,
              "query positions [%lld, %lld) must lie inside the %lld keys", (long long)q_pos0,
              (long long)(q_pos0 + lq), (long long)lk);
  QSA_REQUIRE(first_raw_token >= 0 && first_raw_token % r == 0 && first_raw_token <= lk,
              QSA_ERR_INVALID_ARGUMENT, "first_raw_token=%lld must be a multiple of r in [0, lk]",
              (long long)first_raw_token);
  QSA_REQUIRE(first_raw_token == 0 || k_pooled_prefix, QSA_ERR_INVALID_ARGUMENT,
              "k_pooled_prefix is required when first_raw_token > 0");
  QSA_REQUIRE(k_pooled && (k_idx || first_raw_token / r == lk / r), QSA_ERR_INVALID_ARGUMENT,
              "null k_pooled or k_idx");
  QSA_REQUIRE(aligned16(k_pooled) && (!k_pooled_prefix || aligned16(k_pooled_prefix)),
              QSA_ERR_INVALID_ARGUMENT, "pooled-key buffers must be 16-byte aligned");
  QSA_REQUIRE(lq == 0 || (workspace && workspace_bytes >= need && aligned16(workspace)),
              QSA_ERR_WORKSPACE, "prefill workspace: need %zu bytes (16-byte aligned), got %zu",
              need, workspace_bytes);
  const int64_t nblk = lk / r;
  const int64_t prefix_blocks = first_raw_token / r;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (prefix_blocks > 0 && k_pooled_prefix != k_pooled) {
    QSA_TRY(hip_status(hipMemcpyAsync(k_pooled, k_pooled_prefix,
                                      (size_t)prefix_blocks * d_idx * sizeof(uint16_t),
                                      hipMemcpyDeviceToDevice, s),
                       "copy of the pooled prefix"));
  }
  const int64_t new_blocks = nblk - prefix_blocks;
  if (new_blocks > 0)
    QSA_TRY(qsa_pool_keys_pe(k_idx, d_idx, new_blocks, d_idx, r, prefix_blocks, pe,
                             static_cast<uint16_t*>(k_pooled) + prefix_blocks * d_idx, d_idx,
                             stream));
  return QSA_OK;
}

// List entries of the fused selection's largest chunk: rows x pieces x piece capacity.
size_t fused_list_bytes(int64_t lq, int64_t rc) {
  const int64_t last = lq % rc == 0 ? rc : lq % rc;
  const int64_t a = rc * qsa::fused_n_split(rc), b = last * qsa::fused_n_split(last);
  return (size_t)(a > b ? a : b) * qsa::kFusedListCap * sizeof(uint64_t);
}

}  // namespace

qsa_status qsa_prefill_select(int64_t lq, int64_t lk, int64_t q_pos0, int h_idx, int d_idx,
                              int r, int budget_tokens, const void* q_idx, const float* w,
                              const void* k_idx, int64_t first_raw_token,
                              const void* k_pooled_prefix, void* k_pooled, int32_t* sel,
                              int64_t row_chunk, void* workspace, size_t workspace_bytes,
                              const qsa_pooled_pe* pe, void* stream) {
  const size_t need = qsa_prefill_workspace_bytes(lq, lk, r, budget_tokens, row_chunk);
  QSA_TRY(prefill_pool(lq, lk, q_pos0, h_idx, d_idx, r, budget_tokens, k_idx, first_raw_token,
                       k_pooled_prefix, k_pooled, pe, need, workspace, workspace_bytes, stream));
  if (lq == 0) return QSA_OK;
  const int64_t nblk = lk / r;
  const int64_t rc = row_chunk > 0 ? (row_chunk < lq ? row_chunk : lq) : lq;
  const int64_t ld = score_ld(nblk);
  float* sc = static_cast<float*>(workspace);
  const size_t sc_bytes = align256((size_t)rc * (size_t)ld * sizeof(float));
  const int n_sel = budget_tokens / r;
  for (int64_t c0 = 0; c0 < lq; c0 += rc) {
    const int64_t n = (lq - c0) < rc ? (lq - c0) : rc;
    QSA_TRY(qsa_index_scores(1, n, h_idx, d_idx, r,
                             static_cast<const uint16_t*>(q_idx) + c0 * h_idx * d_idx, 0,
                             w + c0 * h_idx, 0, k_pooled, 0, nblk, q_pos0 + c0, nullptr, sc, ld,
                             0, stream));
    QSA_TRY(qsa_topk_blocks(1, n, r, budget_tokens, sc, ld, 0, nblk, q_pos0 + c0, nullptr,
                            sel + c0 * n_sel, static_cast<char*>(workspace) + sc_bytes,
                            workspace_bytes - sc_bytes, stream));
  }
  return QSA_OK;
}

size_t qsa_prefill_fused_workspace_bytes(int64_t lq, int64_t lk, int r, int budget_tokens,
                                         int64_t row_chunk) {
  if (lq <= 0 || lk <= 0 || r <= 0) return 0;
  const int64_t rc = row_chunk > 0 ? (row_chunk < lq ? row_chunk : lq) : lq;
  // scores, lists, list counts, row flags, sampled keys and sample counts per
  // (row, piece, lane)
  return align256((size_t)rc * (size_t)score_ld(lk / r) * sizeof(float)) +
         align256(fused_list_bytes(lq, rc)) + align256((size_t)rc * 4 * 16 * sizeof(int32_t)) +
         align256((size_t)rc * sizeof(int32_t)) + align256((size_t)rc * 4 * 16 * 32) +
         align256((size_t)rc * 4 * 16 * sizeof(int32_t));
}

qsa_status qsa_prefill_select_fused(int64_t lq, int64_t lk, int64_t q_pos0, int h_idx,
                                    int d_idx, int r, int budget_tokens, const void* q_idx,
                                    const float* w, const void* k_idx, int64_t first_raw_token,
                                    const void* k_pooled_prefix, void* k_pooled, int32_t* sel,
                                    int64_t row_chunk, void* workspace, size_t workspace_bytes,
                                    const qsa_pooled_pe* pe, const qsa_fused_tuning* tuning,
                                    void* stream) {
  const int64_t nblk = lk / r > 0 ? lk / r : 0;
  QSA_REQUIRE(nblk < ((int64_t)1 << 24), QSA_ERR_UNSUPPORTED,
              "%lld blocks: the fused selection takes fewer than 2^24", (long long)nblk);
  const int n_sel = r > 0 ? budget_tokens / r : 0;
  qsa_fused_tuning tn{2 * (n_sel > 1 ? n_sel - 1 : 1), 64, qsa::kFusedListCap};
  if (tuning) {
    if (tuning->target > 0) tn.target = tuning->target;
    if (tuning->sample_k > 0) tn.sample_k = tuning->sample_k;
    if (tuning->cap > 0) tn.cap = tuning->cap;
  }
  QSA_REQUIRE(tn.cap <= qsa::kFusedListCap, QSA_ERR_UNSUPPORTED, "cap=%d: at most %d", tn.cap,
              qsa::kFusedListCap);
  const size_t need = qsa_prefill_fused_workspace_bytes(lq, lk, r, budget_tokens, row_chunk);
  QSA_TRY(prefill_pool(lq, lk, q_pos0, h_idx, d_idx, r, budget_tokens, k_idx, first_raw_token,
                       k_pooled_prefix, k_pooled, pe, need, workspace, workspace_bytes, stream));
  if (lq == 0) return QSA_OK;
  QSA_REQUIRE(q_idx && w && sel && aligned16(q_idx), QSA_ERR_INVALID_ARGUMENT,
              "null or misaligned q_idx, w or sel");
  const int64_t rc = row_chunk > 0 ? (row_chunk < lq ? row_chunk : lq) : lq;
  const int64_t ld = score_ld(nblk);
  char* ws = static_cast<char*>(workspace);
  float* sc = reinterpret_cast<float*>(ws);
  ws += align256((size_t)rc * (size_t)ld * sizeof(float));
  uint2* lists = reinterpret_cast<uint2*>(ws);
  ws += align256(fused_list_bytes(lq, rc));
  int32_t* counts = reinterpret_cast<int32_t*>(ws);
  ws += align256((size_t)rc * 4 * 16 * sizeof(int32_t));
  int32_t* flags = reinterpret_cast<int32_t*>(ws);
  ws += align256((size_t)rc * sizeof(int32_t));
  uint4* s_top = reinterpret_cast<uint4*>(ws);
  ws += align256((size_t)rc * 4 * 16 * 32);
  int32_t* s_nv = reinterpret_cast<int32_t*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t c0 = 0; c0 < lq; c0 += rc) {
    const int64_t n = (lq - c0) < rc ? (lq - c0) : rc;
    qsa::FusedSelArgs f{};
    f.q_idx = static_cast<const uint16_t*>(q_idx) + c0 * h_idx * d_idx;
    f.w = w + c0 * h_idx;
    f.kp = static_cast<const uint16_t*>(k_pooled);
    f.nblk = nblk;
    f.lq = n;
    f.q_pos0 = q_pos0 + c0;
    f.h_idx = h_idx;
    f.d_idx = d_idx;
    f.r = r;
    f.n_sel = n_sel;
    f.lists = lists;
    f.counts = counts;
    f.flags = flags;
    f.s_top = s_top;
    f.s_nv = s_nv;
    f.n_split = qsa::fused_n_split(n);
    f.lane_cap = qsa::kFusedListCap / 16;  // 16 lane lists of a (row, piece): 2048 in all
    f.cap = tn.cap;
    f.target = tn.target;
    f.sample_k = tn.sample_k;
    f.scores = sc;
    f.ld = ld;
    f.sel = sel + c0 * n_sel;
    QSA_TRY(hip_status(qsa::launch_select_fused(f, s), "fused selection launch"));
  }
  return QSA_OK;
}

qsa_status qsa_prefill_forward(int64_t lq, int64_t lk, int64_t q_pos0, int hq, int hkv, int d,
                               int h_idx, int d_idx, int r, int budget_tokens, const void* q,
                               const void* k, const void* v, const void* q_idx, const float* w,
                               const void* k_idx, int64_t first_raw_token,
                               const void* k_pooled_prefix, void* k_pooled, float softmax_scale,
                               int32_t* sel, void* out, float* lse, int64_t row_chunk,
                               void* workspace, size_t workspace_bytes,
                               const qsa_pooled_pe* pe, void* stream) {
  QSA_TRY(check_budget(budget_tokens, r));
  QSA_TRY(check_attn_fwd(lq, lk, hq, hkv, d, r, budget_tokens / r, q, k, v, sel, q_pos0,
                         softmax_scale, out));
  QSA_TRY(qsa_prefill_select(lq, lk, q_pos0, h_idx, d_idx, r, budget_tokens, q_idx, w, k_idx,
                             first_raw_token, k_pooled_prefix, k_pooled, sel, row_chunk,
                             workspace, workspace_bytes, pe, stream));
  return qsa_sparse_attn_fwd(lq, lk, hq, hkv, d, r, budget_tokens / r, q, k, v, sel, q_pos0,
                             softmax_scale, out, lse, stream);
}

// ---- packed variable-length sequences ----

namespace {

qsa::TopkArgs varlen_topk_args(int batch, int64_t rows, int r, int budget_tokens,
                               const float* scores, int64_t ld, int64_t sbs, int64_t max_nblk,
                               int32_t* sel, qsa::Varlen vl) {
  qsa::TopkArgs a = topk_args(batch, rows, r, budget_tokens, scores, ld, sbs, max_nblk, 0,
                              nullptr, sel);
  a.vl = vl;
  return a;
}

int64_t varlen_row_chunk(int64_t max_lq, int64_t row_chunk) {
  return row_chunk > 0 ? (row_chunk < max_lq ? row_chunk : max_lq) : max_lq;
}

qsa_status check_varlen(int batch, const int32_t* cu_q, const int32_t* cu_k, int64_t max_lq,
                        int64_t max_lk, int r) {
  QSA_TRY(check_r(r));
  QSA_REQUIRE(batch >= 1 && batch <= 65535, QSA_ERR_INVALID_ARGUMENT, "batch=%d", batch);
  QSA_REQUIRE(cu_q && cu_k, QSA_ERR_INVALID_ARGUMENT, "null cu_seqlens");
  QSA_REQUIRE(max_lq >= 0 && max_lk >= 0 && max_lq <= max_lk && max_lk < ((int64_t)1 << 31),
              QSA_ERR_INVALID_ARGUMENT, "max_lq=%lld, max_lk=%lld", (long long)max_lq,
              (long long)max_lk);
  QSA_REQUIRE(max_lk / r < ((int64_t)1 << 22), QSA_ERR_UNSUPPORTED,
              "max_lk=%lld: top-k supports fewer than 2^22 blocks", (long long)max_lk);
  return QSA_OK;
}

}  // namespace

size_t qsa_prefill_varlen_workspace_bytes(int batch, int64_t max_lq, int64_t max_lk, int r,
                                          int budget_tokens, int64_t row_chunk) {
  if (batch <= 0 || max_lq <= 0 || max_lk <= 0 || r <= 0 || budget_tokens < r) return 0;
  const int64_t rc = varlen_row_chunk(max_lq, row_chunk);
  const int64_t nblk = max_lk / r;
  const int64_t ld = score_ld(nblk);
  // Sized for rows whose positions reach the last block (lengths live on the device).
  const qsa::Varlen any{reinterpret_cast<const int32_t*>(1), nullptr, 0};
  const qsa::TopkArgs ta =
      varlen_topk_args(batch, rc, r, budget_tokens, nullptr, ld, rc * ld, nblk, nullptr, any);
  return align256((size_t)batch * rc * ld * sizeof(float)) + qsa::topk_workspace_bytes(ta);
}

qsa_status qsa_prefill_varlen_select(int batch, const int32_t* cu_seqlens_q,
                                     const int32_t* cu_seqlens_k, int64_t max_lq,
                                     int64_t max_lk, int h_idx, int d_idx, int r,
                                     int budget_tokens, const void* q_idx, const float* w,
                                     const void* k_idx, void* k_pooled, int32_t* sel,
                                     int64_t row_chunk, void* workspace, size_t workspace_bytes,
                                     const qsa_pooled_pe* pe, void* stream) {
  QSA_TRY(check_varlen(batch, cu_seqlens_q, cu_seqlens_k, max_lq, max_lk, r));
  QSA_TRY(check_budget(budget_tokens, r));
  QSA_TRY(check_indexer_shape(h_idx, d_idx));
  qsa::PooledPe ppe{};
  QSA_TRY(pooled_pe(pe, d_idx, &ppe));
  const int64_t nblk = max_lk / r;
  QSA_REQUIRE(k_pooled && (k_idx || nblk == 0), QSA_ERR_INVALID_ARGUMENT,
              "null k_pooled or k_idx");
  QSA_REQUIRE(aligned16(k_pooled) && (!k_idx || aligned16(k_idx)), QSA_ERR_INVALID_ARGUMENT,
              "k_idx and k_pooled must be 16-byte aligned");
  if (max_lq > 0) {
    QSA_REQUIRE(q_idx && w && sel, QSA_ERR_INVALID_ARGUMENT, "null tensor pointer");
    QSA_REQUIRE(aligned16(q_idx), QSA_ERR_INVALID_ARGUMENT, "q_idx must be 16-byte aligned");
    const size_t need =
        qsa_prefill_varlen_workspace_bytes(batch, max_lq, max_lk, r, budget_tokens, row_chunk);
    QSA_REQUIRE(need == 0 || (workspace && workspace_bytes >= need && aligned16(workspace)),
                QSA_ERR_WORKSPACE,
                "varlen prefill workspace: need %zu bytes (16-byte aligned), got %zu", need,
                workspace_bytes);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  QSA_TRY(hip_status(qsa::launch_pool_keys_varlen(static_cast<const uint16_t*>(k_idx),
                                                  cu_seqlens_k, batch, nblk, d_idx, r,
                                                  static_cast<uint16_t*>(k_pooled), ppe, s),
                     "varlen pooling launch"));
  if (max_lq == 0) return QSA_OK;
  const int64_t rc = varlen_row_chunk(max_lq, row_chunk);
  const int64_t ld = score_ld(nblk);
  float* sc = static_cast<float*>(workspace);
  char* tk = static_cast<char*>(workspace) + align256((size_t)batch * rc * ld * sizeof(float));
  for (int64_t c0 = 0; c0 < max_lq; c0 += rc) {
    const int64_t n = (max_lq - c0) < rc ? (max_lq - c0) : rc;
    const qsa::Varlen vl{cu_seqlens_q, cu_seqlens_k, c0};
    qsa::ScoreArgs sa{static_cast<const uint16_t*>(q_idx), 0, w, 0,
                      static_cast<const uint16_t*>(k_pooled), nblk * d_idx, nblk, n, h_idx,
                      d_idx, r, 0, nullptr, sc, ld, rc * ld, batch, {}, vl};
    QSA_TRY(hip_status(qsa::launch_index_scores(sa, s), "varlen score launch"));
    const qsa::TopkArgs ta =
        varlen_topk_args(batch, n, r, budget_tokens, sc, ld, rc * ld, nblk, sel, vl);
    QSA_TRY(hip_status(qsa::launch_topk_blocks(ta, tk, s), "varlen top-k launch"));
  }
  return QSA_OK;
}

qsa_status qsa_sparse_attn_varlen_fwd(int batch, const int32_t* cu_seqlens_q,
                                      const int32_t* cu_seqlens_k, int64_t total_q,
                                      int64_t max_lk, int hq, int hkv, int d, int r, int n_sel,
                                      const void* q, const void* k, const void* v,
                                      const int32_t* sel, float softmax_scale, void* out,
                                      float* lse, void* stream) {
  QSA_TRY(check_r(r));
  QSA_TRY(check_attn_shape(hq, hkv, d));
  QSA_REQUIRE(batch >= 1 && batch <= 65535, QSA_ERR_INVALID_ARGUMENT, "batch=%d", batch);
  QSA_REQUIRE(cu_seqlens_q && cu_seqlens_k, QSA_ERR_INVALID_ARGUMENT, "null cu_seqlens");
  QSA_REQUIRE(n_sel >= 1 && n_sel <= 1024, QSA_ERR_UNSUPPORTED, "n_sel=%d: supported 1..1024",
              n_sel);
  QSA_REQUIRE(total_q >= 0 && total_q < ((int64_t)1 << 31), QSA_ERR_INVALID_ARGUMENT,
              "total_q=%lld", (long long)total_q);
  QSA_REQUIRE(max_lk >= 0, QSA_ERR_INVALID_ARGUMENT, "max_lk=%lld", (long long)max_lk);
  QSA_REQUIRE(isfinite(softmax_scale), QSA_ERR_INVALID_ARGUMENT, "softmax_scale not finite");
  if (total_q == 0) return QSA_OK;
  QSA_REQUIRE(q && k && v && sel && out, QSA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  QSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out),
              QSA_ERR_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
  qsa::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.sel = sel;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.lq = total_q;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.n_sel = n_sel;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.batch_vl = batch;
  a.keys_hint = max_lk;
  return hip_status(qsa::launch_sparse_attn_fwd(a, static_cast<hipStream_t>(stream)),
                    "qsa_sparse_attn_varlen_fwd launch");
}

qsa_status qsa_prefill_varlen_forward(int batch, const int32_t* cu_seqlens_q,
                                      const int32_t* cu_seqlens_k, int64_t total_q,
                                      int64_t max_lq, int64_t max_lk, int hq, int hkv, int d,
                                      int h_idx, int d_idx, int r, int budget_tokens,
                                      const void* q, const void* k, const void* v,
                                      const void* q_idx, const float* w, const void* k_idx,
                                      void* k_pooled, float softmax_scale, int32_t* sel,
                                      void* out, float* lse, int64_t row_chunk,
                                      void* workspace, size_t workspace_bytes,
                                      const qsa_pooled_pe* pe, void* stream) {
  QSA_TRY(check_budget(budget_tokens, r));
  QSA_TRY(check_attn_shape(hq, hkv, d));
  QSA_REQUIRE(total_q >= 0 && total_q < ((int64_t)1 << 31), QSA_ERR_INVALID_ARGUMENT,
              "total_q=%lld", (long long)total_q);
  QSA_REQUIRE(isfinite(softmax_scale), QSA_ERR_INVALID_ARGUMENT, "softmax_scale not finite");
  QSA_REQUIRE(total_q == 0 || (q && k && v && out && aligned16(q) && aligned16(k) &&
                               aligned16(v) && aligned16(out)),
              QSA_ERR_INVALID_ARGUMENT, "q, k, v and out must be non-null and 16-byte aligned");
  QSA_TRY(qsa_prefill_varlen_select(batch, cu_seqlens_q, cu_seqlens_k, max_lq, max_lk, h_idx,
                                    d_idx, r, budget_tokens, q_idx, w, k_idx, k_pooled, sel,
                                    row_chunk, workspace, workspace_bytes, pe, stream));
  return qsa_sparse_attn_varlen_fwd(batch, cu_seqlens_q, cu_seqlens_k, total_q, max_lk, hq,
                                    hkv, d, r, budget_tokens / r, q, k, v, sel, softmax_scale,
                                    out, lse, stream);
}

// ---- whole decode step ----

size_t qsa_decode_workspace_bytes(int batch, int hq, int d, int64_t lmax, int r,
                                  int budget_tokens) {
  if (batch <= 0 || r <= 0 || budget_tokens <= 0) return 0;
  const size_t sc = align256((size_t)batch * (size_t)score_ld(lmax / r) * sizeof(float));
  const size_t tk = align256(qsa_topk_workspace_bytes(batch, 1, lmax / r, budget_tokens, r));
  return sc + tk + qsa_sparse_attn_decode_workspace_bytes(batch, hq, d, budget_tokens / r);
}

namespace {

qsa_status decode_forward_impl(int batch, int hq, int hkv, int d, int h_idx, int d_idx, int r,
                               int budget_tokens, const void* q, const void* q_idx,
                               const float* w, const void* k_pooled,
                               int64_t k_pooled_batch_stride, const void* k_cache,
                               const void* v_cache, int64_t cache_batch_stride,
                               const PagedKV* paged, int64_t lmax, const int32_t* seq_lens,
                               float softmax_scale, int32_t* sel, void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream,
                               bool use_scratch = false) {
  QSA_TRY(check_r(r));
  if (paged) QSA_TRY(check_paged(*paged, r, lmax));
  QSA_REQUIRE(q && k_cache && v_cache && out && aligned16(q) && aligned16(k_cache) &&
                  aligned16(v_cache) && aligned16(out),
              QSA_ERR_INVALID_ARGUMENT, "q, caches and out must be non-null and 16-byte aligned");
  QSA_REQUIRE(isfinite(softmax_scale), QSA_ERR_INVALID_ARGUMENT, "softmax_scale not finite");
  QSA_TRY(check_budget(budget_tokens, r));
  QSA_TRY(check_indexer_shape(h_idx, d_idx));
  QSA_TRY(check_attn_shape(hq, hkv, d));
  QSA_REQUIRE(batch >= 1 && batch <= 65535, QSA_ERR_INVALID_ARGUMENT, "batch=%d", batch);
  QSA_REQUIRE(lmax >= r && lmax / r < ((int64_t)1 << 22), QSA_ERR_UNSUPPORTED,
              "lmax=%lld: 4 <= lmax and lmax / r < 2^22", (long long)lmax);
  QSA_REQUIRE(q_idx && w && k_pooled && seq_lens && sel, QSA_ERR_INVALID_ARGUMENT,
              "null tensor pointer");
  QSA_REQUIRE(aligned16(q_idx) && aligned16(k_pooled), QSA_ERR_INVALID_ARGUMENT,
              "q_idx and k_pooled must be 16-byte aligned");
  QSA_REQUIRE(batch == 1 || (k_pooled_batch_stride % 8 == 0 &&
                             k_pooled_batch_stride >= (lmax / r) * (int64_t)d_idx),
              QSA_ERR_INVALID_ARGUMENT, "k_pooled_batch_stride=%lld",
              (long long)k_pooled_batch_stride);
  const size_t need = qsa_decode_workspace_bytes(batch, hq, d, lmax, r, budget_tokens);
  if (use_scratch) {  // every argument checked: only now touch the device
    QSA_TRY(noalloc_scratch(&workspace));
    workspace_bytes = (size_t)QSA_NOALLOC_SCRATCH_BYTES;
  }
  QSA_REQUIRE(workspace && workspace_bytes >= need && aligned16(workspace), QSA_ERR_WORKSPACE,
              "decode workspace: need %zu bytes (16-byte aligned), got %zu", need,
              workspace_bytes);
  const int64_t nblk = lmax / r;
  const int64_t ld = score_ld(nblk);
  float* sc = static_cast<float*>(workspace);
  const size_t sc_bytes = align256((size_t)batch * (size_t)ld * sizeof(float));
  const size_t tk_bytes = align256(qsa_topk_workspace_bytes(batch, 1, nblk, budget_tokens, r));
  char* tk = static_cast<char*>(workspace) + sc_bytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  qsa::ScoreArgs sa{static_cast<const uint16_t*>(q_idx), (int64_t)h_idx * d_idx, w, h_idx,
                    static_cast<const uint16_t*>(k_pooled), k_pooled_batch_stride, nblk, 1,
                    h_idx, d_idx, r, 0, seq_lens, sc, ld, ld, batch, {}};
  const qsa::TopkArgs ta = topk_args(batch, 1, r, budget_tokens, sc, ld, ld, nblk, 0, seq_lens,
                                     sel);
  QSA_REQUIRE(qsa::topk_supported(ta), QSA_ERR_UNSUPPORTED, "rows of %lld blocks",
              (long long)nblk);
  if (tk_bytes > 0) {
    // Long rows: the scan also emits per-segment candidates, then one merge launch.
    sa.cand = qsa::topk_candidates(ta, tk);
    QSA_TRY(hip_status(qsa::launch_index_scores(sa, s), "decode score scan launch"));
    QSA_TRY(hip_status(qsa::launch_topk_merge(ta, tk, s), "decode top-k merge launch"));
  } else {
    QSA_TRY(hip_status(qsa::launch_index_scores(sa, s), "decode score scan launch"));
    QSA_TRY(hip_status(qsa::launch_topk_blocks(ta, tk, s), "decode top-k launch"));
  }
  return sparse_attn_decode_impl(batch, hq, hkv, d, r, budget_tokens / r, q, k_cache, v_cache,
                                 cache_batch_stride, lmax, paged, seq_lens, sel, softmax_scale,
                                 out, lse, tk + tk_bytes, workspace_bytes - sc_bytes - tk_bytes,
                                 stream);
}

}  // namespace

qsa_status qsa_decode_forward(int batch, int hq, int hkv, int d, int h_idx, int d_idx, int r,
                              int budget_tokens, const void* q, const void* q_idx,
                              const float* w, const void* k_pooled,
                              int64_t k_pooled_batch_stride, const void* k_cache,
                              const void* v_cache, int64_t cache_batch_stride, int64_t lmax,
                              const int32_t* seq_lens, float softmax_scale, int32_t* sel,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (batch > 1)
    QSA_REQUIRE(cache_batch_stride % 8 == 0 && cache_batch_stride >= lmax * (int64_t)hkv * d,
                QSA_ERR_INVALID_ARGUMENT, "cache_batch_stride=%lld",
                (long long)cache_batch_stride);
  return decode_forward_impl(batch, hq, hkv, d, h_idx, d_idx, r, budget_tokens, q, q_idx, w,
                             k_pooled, k_pooled_batch_stride, k_cache, v_cache,
                             cache_batch_stride, nullptr, lmax, seq_lens, softmax_scale, sel,
                             out, lse, workspace, workspace_bytes, stream);
}

qsa_status qsa_decode_forward_noalloc(int batch, int hq, int hkv, int d, int h_idx, int d_idx,
                                      int r, int budget_tokens, const void* q,
                                      const void* q_idx, const float* w, const void* k_pooled,
                                      int64_t k_pooled_batch_stride, const void* k_cache,
                                      const void* v_cache, int64_t cache_batch_stride,
                                      int64_t lmax, const int32_t* seq_lens,
                                      float softmax_scale, int32_t* sel, void* out, float* lse,
                                      void* stream) {
  QSA_REQUIRE(batch >= 1 && r > 0 && budget_tokens > 0 && lmax >= 0,
              QSA_ERR_INVALID_ARGUMENT, "batch=%d r=%d budget=%d lmax=%lld", batch, r,
              budget_tokens, (long long)lmax);
  const size_t need = qsa_decode_workspace_bytes(batch, hq, d, lmax, r, budget_tokens);
  QSA_REQUIRE(need <= (size_t)QSA_NOALLOC_SCRATCH_BYTES, QSA_ERR_WORKSPACE,
              "qsa_decode_forward_noalloc: batch %d x lmax %lld needs %zu bytes of scratch; "
              "the static scratch holds %zu (use qsa_decode_forward with a workspace)",
              batch, (long long)lmax, need, (size_t)QSA_NOALLOC_SCRATCH_BYTES);
  if (batch > 1)
    QSA_REQUIRE(cache_batch_stride % 8 == 0 && cache_batch_stride >= lmax * (int64_t)hkv * d,
                QSA_ERR_INVALID_ARGUMENT, "cache_batch_stride=%lld",
                (long long)cache_batch_stride);
  return decode_forward_impl(batch, hq, hkv, d, h_idx, d_idx, r, budget_tokens, q, q_idx, w,
                             k_pooled, k_pooled_batch_stride, k_cache, v_cache,
                             cache_batch_stride, nullptr, lmax, seq_lens, softmax_scale, sel,
                             out, lse, nullptr, 0, stream, /*use_scratch=*/true);
}

qsa_status qsa_decode_forward_paged(int batch, int hq, int hkv, int d, int h_idx, int d_idx,
                                    int r, int budget_tokens, const void* q, const void* q_idx,
                                    const float* w, const void* k_pooled,
                                    int64_t k_pooled_batch_stride, const void* k_pool,
                                    const void* v_pool, int64_t num_pages, int page_size,
                                    const int32_t* block_table, int64_t table_stride,
                                    int64_t lmax, const int32_t* seq_lens, float softmax_scale,
                                    int32_t* sel, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  const PagedKV pk{block_table, table_stride, page_size, num_pages};
  return decode_forward_impl(batch, hq, hkv, d, h_idx, d_idx, r, budget_tokens, q, q_idx, w,
                             k_pooled, k_pooled_batch_stride, k_pool, v_pool, 0, &pk, lmax,
                             seq_lens, softmax_scale, sel, out, lse, workspace, workspace_bytes,
                             stream);
}

}  // extern "C"

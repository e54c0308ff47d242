/*
 * qsa.h -- C ABI of the Qwen Sparse Attention (QSA) forward path on MI355X (gfx950).
 *
 * QSA keeps exact softmax attention but reads only part of the context: a light
 * indexer scores micro-blocks of r = 4 tokens from mean-pooled keys and keeps the
 * best blocks up to a token budget; attention then reads only the kept tokens.
 * Sources, cited by page title and section:
 *   [DR] "On the Design of Qwen3.8-Next Architecture" (summary page), "four
 *        architecture components", item 2 "Qwen Sparse Attention (QSA)":
 *        micro-blocks of r=4, keys mean-pooled, 4 MQA indexer heads, K=2048,
 *        DeepSeek-DSA-style light indexer + top-k.
 *   [MR] "Qwen3.8-Flash-Next" (Miles RL recipe), section 1 "Model Introduction":
 *        each layer projects indexer queries and compressed keys, scores them,
 *        keeps indexer_budget key tokens per query, attention reads only those;
 *        selection rows are built outside the attention kernel; 24 heads,
 *        2 query groups, kv-channels 256.
 *   [MR5] same page, section 5.3 "Rollout & SGLang": packed THD tensors.
 *   [RA] release article "Qwen3.8-Flash-Next开源", section "GDN+QSA".
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers; bf16 tensors are passed as void* and
 *     hold IEEE bfloat16 bit patterns. Strides are in ELEMENTS. Every pointer to a
 *     bf16 or fp32 tensor must be 16-byte aligned, as must every row stride times
 *     the element size where a stride is taken.
 *   - `stream` is a hipStream_t (NULL = the null stream). Every call only enqueues
 *     work on it and returns; nothing is synchronised, no device memory is read on
 *     the host, and the library allocates nothing: the caller owns every input,
 *     output and workspace buffer. Calls are thread-safe.
 *   - Errors detectable on the host (null pointers, shapes, alignment, unsupported
 *     sizes, short workspace) return a non-zero qsa_status BEFORE any launch, and
 *     qsa_last_error() then describes it (thread-local text). A failed launch
 *     returns QSA_ERR_HIP. Faults inside a kernel surface at the caller's next
 *     synchronisation.
 *   - Supported sizes: r = 4; attention head dim d in {128, 256}; heads per KV
 *     group Hq/Hkv in 1..16; indexer heads H_I in 1..4 with dim d_I in {64, 128};
 *     budget K a multiple of r with 4 <= K/r <= 1024.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 3

typedef enum qsa_status {
  QSA_OK = 0,
  QSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad shape, stride or alignment */
  QSA_ERR_UNSUPPORTED = 2,      /* a size outside the supported set above */
  QSA_ERR_WORKSPACE = 3,        /* workspace null or smaller than the query says */
  QSA_ERR_HIP = 4               /* a HIP launch failed; the message names the error */
} qsa_status;

/* Version of this ABI (QSA_ABI_VERSION of the built library). */
int qsa_abi_version(void);

/* Text describing the last non-OK status returned on the calling thread ("" if none). */
const char* qsa_last_error(void);

/*
 * Stage 1 -- micro-block mean pooling of the indexer keys [DR].
 * kbar[b][c] = bf16( (k_idx[r*b][c] + ... + k_idx[r*b+r-1][c]) / r ), b < n_blocks,
 * summed in fp64 (exact for bf16 keys), divided by r and rounded once to nearest
 * even. Only complete blocks are
 * passed: the caller points k_idx at the first token of the first block to pool and
 * k_pooled at that block's row. qsa_pool_keys adds no positional encoding;
 * qsa_pool_keys_pe adds the one below.
 *   k_idx     bf16 [r*n_blocks rows][d_idx], row i at k_idx + i*k_idx_row_stride
 *   k_pooled  bf16 [n_blocks][d_idx],        row b at k_pooled + b*k_pooled_row_stride
 */
qsa_status qsa_pool_keys(const void* k_idx, int64_t k_idx_row_stride, int64_t n_blocks,
                         int d_idx, int r, void* k_pooled, int64_t k_pooled_row_stride,
                         void* stream);

/*
 * Positional encoding of the pooled keys [DR]: the keys are mean-pooled first and the
 * position is encoded afterwards (the pages name no form; the reading here is the
 * partial rotary encoding of the model's attention): the leading rope_dim columns of
 * kbar[b] are rotated at the block's position p = (first_block + b) * r, the position
 * of its first token, in the half-split convention: for i < h = rope_dim / 2,
 *   a = p * rope_theta^(-2i / rope_dim)
 *   kbar[i]     <- kbar[i] cos a - kbar[i+h] sin a
 *   kbar[i + h] <- kbar[i+h] cos a + kbar[i] sin a
 * The mean, the angle and the rotation are fp64; the result is rounded once to bf16.
 * The indexer queries are expected rotated the same way at their own positions (the
 * caller's projection does that, as for q and k of the attention), so that a score
 * depends on the query's offset from the block. rope_dim = 0 (or a NULL pointer
 * wherever a qsa_pooled_pe* is taken) means no encoding.
 *   rope_dim    multiple of 16 with 16 <= rope_dim <= d_idx, or 0
 *   rope_theta  rotary base, finite and > 1
 * qsa_pool_keys_pe: as qsa_pool_keys; first_block is the index of the first pooled
 * block within its sequence (nonzero when pooling the tail of a cached prefix).
 */
typedef struct qsa_pooled_pe {
  int rope_dim;
  float rope_theta;
} qsa_pooled_pe;
qsa_status qsa_pool_keys_pe(const void* k_idx, int64_t k_idx_row_stride, int64_t n_blocks,
                            int d_idx, int r, int64_t first_block, const qsa_pooled_pe* pe,
                            void* k_pooled, int64_t k_pooled_row_stride, void* stream);

/*
 * Stage 2 -- light MQA indexer block scores [DR], [RA] (DSA-style reading):
 *   s[t][b] = sum_{h < h_idx} w[t][h] * max(0, q_idx[t][h] . kbar[b])
 * for every block b < min(pos(t) / r, nblk), i.e. every complete block strictly
 * before the query's own block. Entries at b >= pos(t)/r hold unspecified values
 * (up to the next multiple of 4; never read by stage 3).
 * Query row i of sequence s sits at position pos = q_pos0 + i when seq_lens is NULL,
 * else at pos = seq_lens[s] - lq + i (seq_lens is a device array of `batch` int32;
 * rows with pos < 0 score nothing).
 *   q_idx    bf16 [batch][lq][h_idx][d_idx], sequence s at q_idx + s*q_idx_batch_stride
 *   w        fp32 [batch][lq][h_idx],        sequence s at w + s*w_batch_stride
 *   k_pooled bf16 [batch][nblk][d_idx],      sequence s at k_pooled + s*k_pooled_batch_stride
 *   scores   fp32 [batch][lq][ld], ld >= nblk and ld % 4 == 0,
 *            sequence s at scores + s*scores_batch_stride
 */
qsa_status qsa_index_scores(int batch, int64_t lq, int h_idx, int d_idx, int r,
                            const void* q_idx, int64_t q_idx_batch_stride,
                            const float* w, int64_t w_batch_stride,
                            const void* k_pooled, int64_t k_pooled_batch_stride, int64_t nblk,
                            int64_t q_pos0, const int32_t* seq_lens,
                            float* scores, int64_t ld, int64_t scores_batch_stride,
                            void* stream);

/*
 * Stage 3 -- block top-k under the token budget [MR], [DR].
 * For each query row (positions as in stage 2) with own block o = pos / r and
 * C = min(o, nblk) candidate blocks 0..C-1: keep the m = min(K/r - 1, C) best
 * candidates ranked by score (descending, -0.0 == +0.0) then block id (ascending),
 * plus the own block o. Output row: the kept ids in ascending order (o last),
 * then -1 up to K/r entries. Exact; no host round trip. Scores must be finite.
 *   scores  fp32 as written by stage 2
 *   sel     int32 [batch][lq][K/r], contiguous
 *   workspace: qsa_topk_workspace_bytes() bytes, 16-byte aligned (0 when every row
 *   has at most 32768 candidates: then it may be NULL). Requires nblk < 2^22.
 */
size_t qsa_topk_workspace_bytes(int batch, int64_t lq, int64_t nblk, int budget_tokens, int r);
qsa_status qsa_topk_blocks(int batch, int64_t lq, int r, int budget_tokens,
                           const float* scores, int64_t ld, int64_t scores_batch_stride,
                           int64_t nblk, int64_t q_pos0, const int32_t* seq_lens,
                           int32_t* sel, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Stage 4 -- exact softmax attention over the kept tokens, prefill [MR], [MR5].
 * For query row i at t = q_pos0 + i and head h (KV group g = h / (hq/hkv)):
 *   J = { j : j/r is a kept block of row i, j <= t, j < lk }
 *   out[i][h] = sum_{j in J} softmax_j(scale * q[i][h] . k[j][g]) v[j][g]
 *   lse[i][h] = ln sum_{j in J} exp(scale * q[i][h] . k[j][g])
 * The kernel needs no causal or segment logic beyond masking j > t in the own block.
 *   q    bf16 [lq][hq][d] (THD), k/v bf16 [lk][hkv][d] (THD), contiguous
 *   sel  int32 [lq][n_sel] as written by stage 3 (ascending ids, -1 padded)
 *   out  bf16 [lq][hq][d]; lse fp32 [lq][hq] or NULL
 * The rows go to the GPU in launches of one generation of the workgroups the device
 * holds at once, so that rows in flight walk their ascending block lists together
 * and share the blocks they have in common through L2. When the K/V of a sequence
 * (lk * hkv * d * 4 bytes) exceed 128 MB, the launches take one KV group at a time,
 * qsa_sparse_attn_fwd_rows_per_launch() rows of that group each (hkv * ceil(lq / rows)
 * launches a call), so that a group's K/V stays in the last-level cache; otherwise
 * each launch takes both groups of rows / hkv rows. A row's result does not depend on
 * how the rows are split.
 */
qsa_status qsa_sparse_attn_fwd(int64_t lq, int64_t lk, int hq, int hkv, int d, int r, int n_sel,
                               const void* q, const void* k, const void* v,
                               const int32_t* sel, int64_t q_pos0, float softmax_scale,
                               void* out, float* lse, void* stream);
/*
 * Stage 4 as a multi-row tile [MR], [DR] (MTP reuse of the kept blocks): the same
 * outputs as qsa_sparse_attn_fwd up to the order of the online softmax (fp32 rounding).
 * A workgroup takes four neighbouring rows of one KV group; where they share enough
 * kept blocks it stages the sorted union of their blocks in LDS once, 16 keys at a
 * time, and each row attends over it with the blocks it did not keep masked, so a block
 * kept by several of the rows is read once. Where they share too little, each row
 * walks its own blocks as in qsa_sparse_attn_fwd.
 *   arguments as for qsa_sparse_attn_fwd, with n_sel <= 512 (QSA_ERR_UNSUPPORTED above)
 *   min_shared  0: always the union; 1..64: the union when at least min_shared of 64
 *               evenly spaced kept blocks of the tile's first row are kept by its second
 *               row too; 65: never
 * Launches: one KV group and one resident generation of tiles at a time. On random
 * selections the rows share few blocks and the per-row kernel is faster; the tile is
 * for inputs whose neighbouring rows keep mostly the same blocks.
 */
qsa_status qsa_sparse_attn_fwd_tiled(int64_t lq, int64_t lk, int hq, int hkv, int d, int r,
                                     int n_sel, const void* q, const void* k, const void* v,
                                     const int32_t* sel, int64_t q_pos0, float softmax_scale,
                                     int min_shared, void* out, float* lse, void* stream);
/*
 * Rows per launch of qsa_sparse_attn_fwd on the current device when each launch takes
 * one KV group of its rows (hkv KV heads, head dim d = 128 or 256); 0 when the
 * arguments are unsupported, -1 when the runtime cannot report the device's occupancy
 * (then all rows go in one launch).
 */
int64_t qsa_sparse_attn_fwd_rows_per_launch(int hkv, int d);
/*
 * Kernel launches one qsa_sparse_attn_fwd call issues for lq rows over a sequence of
 * lk keys (for packed rows: the longest sequence's key count) on the current device,
 * by the rule above; 0 for lq = 0, -1 for unsupported arguments. A measurement aid:
 * the average launch duration is the call's duration over this count.
 */
int64_t qsa_sparse_attn_fwd_launches(int64_t lq, int64_t lk, int hkv, int d);

/*
 * Stage 4 backward -- gradients of the stage-4 attention with respect to q, k and v
 * over the same selection rows, which are constants here ([MR]: the recipe trains
 * through a forward and a backward sparse-attention kernel fed with selection rows
 * built outside the kernel; no gradient reaches the indexer through the top-k).
 * With P the softmax weights of row i over its kept tokens J_i:
 *   dv[j][g] = sum_{i: j in J_i} sum_{h in g} P[i][h][j] dout[i][h]
 *   dS[i][h][j] = P[i][h][j] (dout[i][h] . v[j][g] - dout[i][h] . out[i][h])
 *   dq[i][h] = scale sum_{j in J_i} dS[i][h][j] k[j][g]
 *   dk[j][g] = scale sum_{i: j in J_i} sum_{h in g} dS[i][h][j] q[i][h]
 * P is recomputed from lse; the row term dout . out uses the forward's bf16 output.
 * Every sum runs in a fixed order: results do not depend on scheduling.
 *   q, k, v, sel, q_pos0, softmax_scale: as for qsa_sparse_attn_fwd
 *   out  bf16 [lq][hq][d], lse fp32 [lq][hq]: the forward's outputs (both required)
 *   dout bf16 [lq][hq][d]: gradient of the loss with respect to out
 *   dq   fp32 [lq][hq][d]; dk, dv fp32 [lk][hkv][d], fully written (keys that no row
 *        reads get 0)
 *   workspace: qsa_sparse_attn_bwd_workspace_bytes() bytes, 16-byte aligned (an
 *   upper bound when no GPU is visible to the query; the call checks that the sort's
 *   scratch on its device fits and returns QSA_ERR_HIP if not). lq * n_sel < 2^31.
 */
size_t qsa_sparse_attn_bwd_workspace_bytes(int64_t lq, int64_t lk, int hq, int r, int n_sel);
qsa_status qsa_sparse_attn_bwd(int64_t lq, int64_t lk, int hq, int hkv, int d, int r, int n_sel,
                               const void* q, const void* k, const void* v,
                               const int32_t* sel, int64_t q_pos0, float softmax_scale,
                               const void* out, const float* lse, const void* dout,
                               float* dq, float* dk, float* dv, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Indexer warm-up -- KL distillation of the full attention onto the block scores
 * ([DR]: before sparse training the indexer is warmed up by distilling the full
 * attention distribution, max-pooled to blocks, into it with a KL loss). Readings:
 * the heads' probabilities are summed; the target lives on the blocks the indexer
 * scores for row i (b < B_i = min(t_i / r, lk / r), t_i = q_pos0 + i) and is
 * normalised there; the indexer's distribution is softmax(s[i][b]) over the same
 * blocks; the loss of row i is KL(target || indexer); the target is a constant.
 *
 * qsa_indexer_kl_target: dense causal attention statistics of the main heads.
 *   lse[i][h] = ln sum_{j <= t_i} exp(scale q[i][h] . k[j][g]), fp32 [lq][hq];
 *   target[i][b] = max_{j in block b} sum_h exp(scale q[i][h] . k[j][g] - lse[i][h])
 *   for b < B_i (unnormalised), fp32 [lq][ld] (ld >= lk / r, ld % 4 == 0; entries
 *   b >= B_i are not written). q, k as for qsa_sparse_attn_fwd; hkv <= 4
 *   (QSA_ERR_UNSUPPORTED otherwise: the head sum of a row stays in one wave).
 * qsa_indexer_kl_loss: from the indexer scores s [lq][ld] (stage 2) and target,
 *   loss[i] = KL(p_i || softmax(s_i)) with p_i = target_i / sum_b target_i[b] (0 when
 *   B_i = 0), fp32 [lq]; dscores[i][b] = softmax(s_i)[b] - p_i[b] for b < B_i,
 *   fp32 [lq][ld] (the rest not written). Sums in fp64. nblk = lk / r.
 * qsa_index_scores_bwd: gradients of the stage-2 scores with respect to the
 *   indexer's inputs given dscores (entries b >= B_i are ignored). With
 *   z = q_idx[i][h] . k_pooled[b]: dw[i][h] = sum_b dscores[i][b] max(0, z);
 *   dz = dscores[i][b] w[i][h] [z > 0] (bf16 in the MFMA products);
 *   dq_idx[i][h] = sum_b dz k_pooled[b]; dk_pooled[b] = sum_{i,h} dz q_idx[i][h]; all
 *   fp32, q_idx/w/k_pooled laid out as for qsa_index_scores (unbatched). dk_idx, if
 *   not NULL, receives the raw indexer keys' gradient through the mean pooling,
 *   fp32 [n_tokens][d_idx]: dk_pooled[j / r] / r for tokens of complete blocks, 0
 *   for the rest (the pooled key's bf16 rounding is passed straight through). The
 *   ReLU's derivative at 0 is 0. Every sum has a fixed order (no atomics).
 */
qsa_status qsa_indexer_kl_target(int64_t lq, int64_t lk, int hq, int hkv, int d, int r,
                                 const void* q, const void* k, int64_t q_pos0,
                                 float softmax_scale, float* lse, float* target, int64_t ld,
                                 void* stream);
qsa_status qsa_indexer_kl_loss(int64_t lq, int64_t nblk, int r, int64_t q_pos0,
                               const float* scores, const float* target, int64_t ld,
                               float* loss, float* dscores, void* stream);
qsa_status qsa_index_scores_bwd(int64_t lq, int h_idx, int d_idx, int r, const void* q_idx,
                                const float* w, const void* k_pooled, int64_t nblk,
                                int64_t q_pos0, const float* dscores, int64_t ld,
                                float* dq_idx, float* dw, float* dk_pooled, float* dk_idx,
                                int64_t n_tokens, void* stream);

/*
 * Stage 4' -- decode: one new query token per sequence at t = seq_lens[s] - 1, the
 * same attention as stage 4 over a KV cache, split over the kept blocks into
 * partial softmax states that a second kernel combines.
 *   q        bf16 [batch][hq][d]
 *   k_cache, v_cache bf16 [batch][lmax][hkv][d], sequence s at +s*cache_batch_stride
 *   seq_lens int32 [batch] on the device, 1 <= seq_lens[s] <= lmax
 *   sel      int32 [batch][n_sel]
 *   out      bf16 [batch][hq][d]; lse fp32 [batch][hq] or NULL
 *   workspace: qsa_sparse_attn_decode_workspace_bytes() bytes
 */
size_t qsa_sparse_attn_decode_workspace_bytes(int batch, int hq, int d, int n_sel);
qsa_status qsa_sparse_attn_decode(int batch, int hq, int hkv, int d, int r, int n_sel,
                                  const void* q, const void* k_cache, const void* v_cache,
                                  int64_t cache_batch_stride, int64_t lmax,
                                  const int32_t* seq_lens, const int32_t* sel,
                                  float softmax_scale, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Selection half of the prefill path: pool the new blocks, then for query rows in
 * chunks of `row_chunk` compute the block scores and the top-k. Inputs as in stages
 * 1-3; k_idx holds the raw indexer keys of tokens first_raw_token .. lk-1 (tokens
 * before it are covered by k_pooled_prefix, first_raw_token / r rows, which may be
 * NULL when first_raw_token == 0). Outputs: k_pooled [lk/r][d_idx] (prefix rows
 * copied, new rows pooled) and sel [lq][K/r]. Query row i sits at q_pos0 + i.
 * workspace: qsa_prefill_workspace_bytes() bytes (one chunk's scores + top-k space).
 * The result does not depend on row_chunk; larger chunks mean fewer launches (on
 * MI355X at 128K, 65536-row chunks, 8 GiB of scores, were the fastest measured).
 * pe: positional encoding of the new pooled rows (see qsa_pool_keys_pe; their first
 * block is first_raw_token / r), or NULL for none. Prefix rows are copied as given,
 * so a prefix pooled with the same encoding stays consistent.
 */
size_t qsa_prefill_workspace_bytes(int64_t lq, int64_t lk, int r, int budget_tokens,
                                   int64_t row_chunk);
qsa_status qsa_prefill_select(int64_t lq, int64_t lk, int64_t q_pos0, int h_idx, int d_idx,
                              int r, int budget_tokens, const void* q_idx, const float* w,
                              const void* k_idx, int64_t first_raw_token,
                              const void* k_pooled_prefix, void* k_pooled, int32_t* sel,
                              int64_t row_chunk, void* workspace, size_t workspace_bytes,
                              const qsa_pooled_pe* pe, void* stream);

/*
 * Stages 2 + 3 fused (prefill): the same selection as qsa_prefill_select, bit for
 * bit (the same fp32 scores, the same exact top-k and tie rule), without writing the
 * whole score matrix. Per row, a strided sample of its blocks' scores sets a threshold
 * about `target` of the row's scores reach; the scoring pass appends only the scores
 * at or above it to a short per-row list, and the m = K/r - 1 best are selected from
 * the list. A list that came out shorter than m or longer than `cap` makes that row
 * fall back to materialised scores and an exact select (the same result, slower).
 * ("On the Design of Qwen3.8-Next Architecture", item 2 QSA: the indexer rates
 * micro-blocks and each query keeps the best up to its budget; the release article's
 * GDN+QSA section counts finding the important context as a cost of its own.)
 * Arguments as qsa_prefill_select; blocks (lk / r) must be fewer than 2^24. tuning may
 * be NULL (defaults: target 2 (K/r - 1), sample_k 64, cap 2048); a field <= 0 takes
 * its default; cap <= 2048. The workspace holds one chunk's scores (for the fallback),
 * its lists, counts, flags and sampled keys: qsa_prefill_fused_workspace_bytes().
 */
typedef struct qsa_fused_tuning {
  int target;    /* list entries a row aims at */
  int sample_k;  /* the threshold is about the sample_k-th best sampled score */
  int cap;       /* most list entries a row may hold before it falls back */
} qsa_fused_tuning;
size_t qsa_prefill_fused_workspace_bytes(int64_t lq, int64_t lk, int r, int budget_tokens,
                                         int64_t row_chunk);
qsa_status qsa_prefill_select_fused(int64_t lq, int64_t lk, int64_t q_pos0, int h_idx,
                                    int d_idx, int r, int budget_tokens, const void* q_idx,
                                    const float* w, const void* k_idx, int64_t first_raw_token,
                                    const void* k_pooled_prefix, void* k_pooled, int32_t* sel,
                                    int64_t row_chunk, void* workspace, size_t workspace_bytes,
                                    const qsa_pooled_pe* pe, const qsa_fused_tuning* tuning,
                                    void* stream);

/*
 * Whole prefill path: qsa_prefill_select followed by qsa_sparse_attn_fwd on the same
 * stream. Arguments as in those two calls.
 */
qsa_status qsa_prefill_forward(int64_t lq, int64_t lk, int64_t q_pos0, int hq, int hkv, int d,
                               int h_idx, int d_idx, int r, int budget_tokens,
                               const void* q, const void* k, const void* v,
                               const void* q_idx, const float* w,
                               const void* k_idx, int64_t first_raw_token,
                               const void* k_pooled_prefix, void* k_pooled,
                               float softmax_scale, int32_t* sel, void* out, float* lse,
                               int64_t row_chunk, void* workspace, size_t workspace_bytes,
                               const qsa_pooled_pe* pe, void* stream);

/*
 * Packed variable-length batches (THD) [MR5]: `batch` sequences packed along the token
 * axis. Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q, q_idx,
 * w, sel, out and lse, and key tokens cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k, v
 * and k_idx; its queries are its LAST lq_b = cu_q[b+1]-cu_q[b] tokens, so query row
 * i of the sequence sits at position lk_b - lq_b + i among its own lk_b keys (a
 * sequence with lq_b = lk_b is a plain prefill, lq_b < lk_b a chunk after a prefix
 * whose keys are packed in too). Every step is the single-sequence one applied to
 * each sequence on its own: no block, score or key crosses a sequence boundary.
 *   cu_seqlens_q, cu_seqlens_k  device int32 [batch + 1], non-decreasing from 0;
 *                cu_k[b+1]-cu_k[b] >= cu_q[b+1]-cu_q[b] for every b
 *   max_lq, max_lk  host upper bounds of lq_b and lk_b (they size grids and the
 *                padded pooled-key buffer; a longer sequence is not detected and is
 *                processed only up to the bounds)
 *   total_q      host copy of cu_seqlens_q[batch]
 *   k_pooled     output bf16 [batch][max_lk/r][d_idx]: sequence b's complete blocks
 *                in its slot (the rest of the slot is left as it was)
 *   sel          int32 [total_q][K/r]: block ids LOCAL to each row's sequence,
 *                ascending, -1 padded, as stage 3 writes them for one sequence
 * The selection runs in chunks of row_chunk local rows of every sequence at once
 * (the workspace holds batch x row_chunk score rows). pe (or NULL) encodes each
 * sequence's pooled keys at positions counted from the sequence's first token. The attention launches one
 * resident generation of rows at a time over the packed rows, sequences mixed.
 */
size_t qsa_prefill_varlen_workspace_bytes(int batch, int64_t max_lq, int64_t max_lk, int r,
                                          int budget_tokens, int64_t row_chunk);
qsa_status qsa_prefill_varlen_select(int batch, const int32_t* cu_seqlens_q,
                                     const int32_t* cu_seqlens_k, int64_t max_lq,
                                     int64_t max_lk, int h_idx, int d_idx, int r,
                                     int budget_tokens, const void* q_idx, const float* w,
                                     const void* k_idx, void* k_pooled, int32_t* sel,
                                     int64_t row_chunk, void* workspace, size_t workspace_bytes,
                                     const qsa_pooled_pe* pe, void* stream);
qsa_status qsa_sparse_attn_varlen_fwd(int batch, const int32_t* cu_seqlens_q,
                                      const int32_t* cu_seqlens_k, int64_t total_q,
                                      int64_t max_lk, int hq, int hkv, int d, int r, int n_sel,
                                      const void* q, const void* k, const void* v,
                                      const int32_t* sel, float softmax_scale, void* out,
                                      float* lse, void* stream);
qsa_status qsa_prefill_varlen_forward(int batch, const int32_t* cu_seqlens_q,
                                      const int32_t* cu_seqlens_k, int64_t total_q,
                                      int64_t max_lq, int64_t max_lk, int hq, int hkv, int d,
                                      int h_idx, int d_idx, int r, int budget_tokens,
                                      const void* q, const void* k, const void* v,
                                      const void* q_idx, const float* w, const void* k_idx,
                                      void* k_pooled, float softmax_scale, int32_t* sel,
                                      void* out, float* lse, int64_t row_chunk,
                                      void* workspace, size_t workspace_bytes,
                                      const qsa_pooled_pe* pe, void* stream);

/*
 * Whole decode step for `batch` sequences: scores against the pooled-key cache,
 * top-k, split attention and combine. Inputs as in stages 2-4'; q_idx
 * [batch][h_idx][d_idx], w [batch][h_idx], k_pooled [batch][lmax/r][d_idx]
 * (sequence s at + s*k_pooled_batch_stride). sel [batch][K/r] is an output.
 */
size_t qsa_decode_workspace_bytes(int batch, int hq, int d, int64_t lmax, int r,
                                  int budget_tokens);
qsa_status qsa_decode_forward(int batch, int hq, int hkv, int d, int h_idx, int d_idx, int r,
                              int budget_tokens, const void* q, const void* q_idx,
                              const float* w, const void* k_pooled,
                              int64_t k_pooled_batch_stride, const void* k_cache,
                              const void* v_cache, int64_t cache_batch_stride, int64_t lmax,
                              const int32_t* seq_lens, float softmax_scale, int32_t* sel,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * qsa_decode_forward for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation and
 * arguments without the workspace, which comes from a static device scratch of
 * QSA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until the
 * process ends. The call allocates nothing. A step whose workspace
 * (qsa_decode_workspace_bytes) exceeds the scratch returns QSA_ERR_WORKSPACE before
 * anything is enqueued (at 1M-token caches, 24 heads, d = 256, K = 2048: up to 22
 * sequences).
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (on
 * different streams or threads without ordering) race; calls ordered on one stream
 * are safe. The caller still owns q, the caches, sel, out and lse.
 */
#define QSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
qsa_status qsa_decode_forward_noalloc(int batch, int hq, int hkv, int d, int h_idx, int d_idx,
                                      int r, int budget_tokens, const void* q,
                                      const void* q_idx, const float* w, const void* k_pooled,
                                      int64_t k_pooled_batch_stride, const void* k_cache,
                                      const void* v_cache, int64_t cache_batch_stride,
                                      int64_t lmax, const int32_t* seq_lens,
                                      float softmax_scale, int32_t* sel, void* out, float* lse,
                                      void* stream);

/*
 * Decode from a PAGED K/V cache (serving engines keep the cache in fixed-size pages
 * [MR5]): the same computation as qsa_sparse_attn_decode / qsa_decode_forward, with
 * the K/V rows of token j of sequence s at pool slot
 *   block_table[s * table_stride + j / page_size] * page_size + j % page_size.
 *   k_pool, v_pool  bf16 [num_pages * page_size][hkv][d]
 *   page_size       tokens per page, a multiple of r (a block never straddles pages)
 *   block_table     device int32 [batch][table_stride], table_stride >=
 *                   ceil(lmax / page_size); entries outside [0, num_pages) are clamped
 *                   into it (wrong but in-bounds reads: the caller keeps them valid)
 * The pooled-key cache keeps its per-sequence layout ([batch][lmax/r][d_idx] with
 * k_pooled_batch_stride). Each kept block's page is looked up once, when the decode
 * attention reads its block ids; every other argument, the workspace and the errors
 * are those of the contiguous calls, plus QSA_ERR_UNSUPPORTED for a page size that is
 * not a multiple of r.
 */
qsa_status qsa_sparse_attn_decode_paged(int batch, int hq, int hkv, int d, int r, int n_sel,
                                        const void* q, const void* k_pool, const void* v_pool,
                                        int64_t num_pages, int page_size,
                                        const int32_t* block_table, int64_t table_stride,
                                        int64_t lmax, const int32_t* seq_lens,
                                        const int32_t* sel, float softmax_scale, void* out,
                                        float* lse, void* workspace, size_t workspace_bytes,
                                        void* stream);
qsa_status qsa_decode_forward_paged(int batch, int hq, int hkv, int d, int h_idx, int d_idx,
                                    int r, int budget_tokens, const void* q, const void* q_idx,
                                    const float* w, const void* k_pooled,
                                    int64_t k_pooled_batch_stride, const void* k_pool,
                                    const void* v_pool, int64_t num_pages, int page_size,
                                    const int32_t* block_table, int64_t table_stride,
                                    int64_t lmax, const int32_t* seq_lens, float softmax_scale,
                                    int32_t* sel, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */

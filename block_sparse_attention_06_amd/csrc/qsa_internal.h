// Host-side internals of libqsa: launchers (no argument checking; the C ABI layer
// validates before calling them) and the shared tuning constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Packed variable-length sequences (THD): sequence b owns the query rows
// cu_q[b] .. cu_q[b+1]-1 and the key tokens cu_k[b] .. cu_k[b+1]-1 of the packed
// tensors, its queries being its last cu_q[b+1]-cu_q[b] tokens. A score or top-k
// launch takes the local query rows row0 .. row0+lq-1 of every sequence.
struct Varlen {
  const int32_t* cu_q;  // device [batch + 1]; null: not packed
  const int32_t* cu_k;  // device [batch + 1]
  int64_t row0;
};

// The rows of sequence bi in a launch of lq local rows: how many exist, the packed
// index of the launch's first row, and that row's position among the sequence's keys.
struct SeqRows {
  int64_t n, first, pos;
};
__device__ __forceinline__ SeqRows varlen_rows(const Varlen& v, int bi, int64_t lq) {
  const int64_t q0 = v.cu_q[bi], q1 = v.cu_q[bi + 1];
  const int64_t lk = (int64_t)v.cu_k[bi + 1] - v.cu_k[bi];
  const int64_t left = q1 - q0 - v.row0;
  return SeqRows{left < 0 ? 0 : (left < lq ? left : lq), q0 + v.row0, lk - (q1 - q0) + v.row0};
}

// ---- stage 1 ----
// Positional encoding of the pooled keys: RoPE on the leading rope_dim columns (0: none)
// at the block's position (first_block + b) * r.
struct PooledPe {
  int rope_dim;
  double theta;
  int64_t first_block;
};
hipError_t launch_pool_keys(const uint16_t* k_idx, int64_t k_stride, int64_t n_blocks, int d_idx,
                            int r, uint16_t* k_pooled, int64_t p_stride, const PooledPe& pe,
                            hipStream_t stream);
// Packed sequences (keys cu_k[b] .. cu_k[b+1]-1 of k_idx [.][d_idx]) into the padded
// k_pooled [batch][max_nb][d_idx]; blocks past a sequence's complete blocks are untouched.
// Block positions count from each sequence's first token (pe.first_block unused).
hipError_t launch_pool_keys_varlen(const uint16_t* k_idx, const int32_t* cu_k, int batch,
                                   int64_t max_nb, int d_idx, int r, uint16_t* k_pooled,
                                   const PooledPe& pe, hipStream_t stream);

// Two-level top-k: per segment of kTopkWaveSeg candidates, the kTopkWaveKeep best as
// (score, id) pairs (id -1: empty) and the worst kept one when the segment had more.
// kTopkWaveSeg is a multiple of 256 up to 1024 (a wave's lanes hold kTopkWaveSeg / 64
// each); kTopkWaveKeep is a multiple of 4 up to 16.
constexpr int kTopkWaveSeg = 1024;
constexpr int kTopkWaveKeep = 16;
static_assert(kTopkWaveSeg % 256 == 0 && kTopkWaveSeg <= 1024, "segment size");
static_assert(kTopkWaveKeep % 4 == 0 && kTopkWaveKeep <= 16, "kept per segment");
struct TopkCandidates {
  float* cand_val;   // [rows][n_seg][kTopkWaveKeep]
  int32_t* cand_idx;
  float* bnd_val;    // [rows][n_seg]
  int32_t* bnd_idx;  // -1: the segment kept all its candidates
  int n_seg;
};

// ---- stage 2 ----
struct ScoreArgs {
  const uint16_t* q_idx;
  int64_t q_bs;
  const float* w;
  int64_t w_bs;
  const uint16_t* kp;
  int64_t kp_bs;
  int64_t nblk;
  int64_t lq;
  int h_idx;
  int d_idx;
  int r;
  int64_t q_pos0;
  const int32_t* seq_lens;
  float* scores;
  int64_t ld;
  int64_t s_bs;
  int batch;
  TopkCandidates cand;  // optional (few rows per sequence): also emit segment candidates
  Varlen vl;            // packed sequences: q_idx / w rows packed, kp and scores per sequence
  // optional [lq]: only the 64-row tiles holding a row whose flag is set are scored (the
  // exact fallback of the fused selection); always the GEMM kernel
  const int32_t* row_flags;
};
hipError_t launch_index_scores(const ScoreArgs& a, hipStream_t stream);

// ---- stages 2 + 3 fused (prefill): scores go to short per-row lists, not to memory ----
// Per row of a chunk: a threshold from a strided sample of its blocks' scores, then
// every score at or above it appended (ascending block id) to the row's list; the m
// best are selected from the list. Rows whose list came out shorter than m or longer
// than the capacity are flagged and selected exactly from materialised scores.
constexpr int kFusedListCap = 2048;  // list entries a row may hold in all (select in registers)
struct FusedSelArgs {
  const uint16_t* q_idx;  // the chunk's row 0: [lq][h_idx][d_idx]
  const float* w;         // [lq][h_idx]
  const uint16_t* kp;     // pooled keys [nblk][d_idx]
  int64_t nblk;
  int64_t lq;             // rows of the chunk
  int64_t q_pos0;         // position of the chunk's row 0
  int h_idx;
  int d_idx;
  int r;
  int n_sel;
  uint2* lists;           // [lq][n_split][16][lane_cap] entries (fp32 score bits, block id)
  int32_t* counts;        // [lq][n_split][16]
  int32_t* flags;         // [lq]: 1 where the fallback selects
  uint4* s_top;           // [lq][n_split][16][2]: a lane's 8 best sampled keys of a piece's share
  int32_t* s_nv;          // [lq][n_split][16]: its sampled candidates
  int n_split;            // key-range pieces of a row tile (one workgroup each)
  int lane_cap;           // entries a (row, piece, lane) list holds
  int cap;                // entries a row's lists may hold in all (<= kFusedListCap)
  int target;             // list entries a row aims at
  int sample_k;           // the threshold is about the sample_k-th best sampled score
  float* scores;          // fallback: [lq][ld]
  int64_t ld;
  int32_t* sel;           // the chunk's selection rows [lq][n_sel]
};
// Pieces per row tile for a chunk of lq rows (enough workgroups to fill the device).
int fused_n_split(int64_t lq);
hipError_t launch_select_fused(const FusedSelArgs& f, hipStream_t stream);

// ---- stage 3 ----
struct TopkArgs {
  const float* scores;
  int64_t ld;
  int64_t s_bs;
  int64_t lq;
  int64_t nblk;
  int64_t q_pos0;
  const int32_t* seq_lens;
  int r;
  int n_sel;
  int32_t* sel;
  int batch;
  Varlen vl;  // packed sequences: sel rows packed, scores per sequence (chunk-local rows)
};
size_t topk_workspace_bytes(const TopkArgs& a);
bool topk_supported(const TopkArgs& a);
hipError_t launch_topk_blocks(const TopkArgs& a, void* ws, hipStream_t stream);
// Candidate layout inside a top-k workspace (when topk_workspace_bytes(a) > 0), and
// the merge launch alone (for a caller that wrote the candidates itself).
TopkCandidates topk_candidates(const TopkArgs& a, void* ws);
hipError_t launch_topk_merge(const TopkArgs& a, void* ws, hipStream_t stream);

// ---- stage 4 / 4' ----
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* sel;
  uint16_t* out;
  float* lse;
  int64_t lq;       // prefill: query rows; decode: batch
  int64_t lk;       // prefill: keys; decode: cache capacity per sequence
  int64_t q_pos0;   // prefill only
  const int32_t* seq_lens;  // decode only
  int64_t cache_bs;         // decode only: elements between sequences of the caches
  int hq;
  int hkv;
  int d;
  int n_sel;
  float scale_log2;  // softmax scale * log2(e)
  // decode split-KV partials
  float* part_o;     // [batch][hq][n_split][d]
  float* part_ml;    // [batch][hq][n_split][2]
  int n_split;
  int steps_per_split;
  // prefill: the launch takes rows row_begin .. row_begin + lq - 1; with cu_q / cu_k
  // (device [batch + 1]) the rows and keys are packed sequences, each row's position
  // counted within its own sequence
  int64_t row_begin;
  int kv_group;  // prefill: the KV group every wave of the launch takes; -1: (row, group) pairs
  const int32_t* cu_q;
  const int32_t* cu_k;
  int batch_vl;
  // prefill: key count of the longest sequence, which chooses the launch order (one KV
  // group at a time or both together); 0: lk, or for packed rows their average count
  int64_t keys_hint;
  // decode from a paged cache: k / v are pools of num_pages pages of page_blocks
  // 4-token blocks; page p of sequence s is block_table[s * table_stride + p]
  const int32_t* block_table;
  int64_t table_stride;
  int page_blocks;
  int num_pages;
};
hipError_t launch_sparse_attn_fwd(const AttnArgs& a, hipStream_t stream);
// Workgroups of `kernel` (block_threads threads) the current device holds at once; 0
// when the runtime cannot say.
int resident_workgroups(const void* kernel, int block_threads);
// Multi-row tile (four neighbouring rows of one KV group per workgroup, the union of
// their kept blocks staged in LDS): kept lists of at most kTileMaxSel entries; the
// union is used where a sample of row 0's blocks finds at least min_shared of 64 in
// row 1's list (0: always, 65: never).
constexpr int kTileMaxSel = 512;
hipError_t launch_sparse_attn_fwd_tiled(const AttnArgs& a, int min_shared, hipStream_t stream);
int64_t sparse_attn_tiled_rows_per_launch(int d);
// Rows per launch of launch_sparse_attn_fwd on the current device; -1 if unknown.
int64_t sparse_attn_fwd_rows_per_launch(int hkv, int d);
// Kernel launches of one launch_sparse_attn_fwd call over lq rows whose longest
// sequence has `keys` keys (the same rule as the launcher); 0 if lq <= 0.
int64_t sparse_attn_fwd_launches(int64_t lq, int64_t keys, int hkv, int d);
hipError_t launch_sparse_attn_decode(const AttnArgs& a, hipStream_t stream);

// ---- stage 4 backward ----
struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* sel;
  const uint16_t* out;   // forward output (bf16), for D = dO . O
  const float* lse;      // forward lse (natural log)
  const uint16_t* dout;  // output gradient (bf16)
  float* dq;             // [lq][hq][d]
  float* dk;             // [lk][hkv][d]
  float* dv;
  float* dbuf;                // workspace: D [lq][hq]
  const int32_t* pair_rows;   // workspace: rows of the (block, row) pairs sorted by block
  int32_t* start;             // workspace: [n_kb + 1] first pair of each key block
  int64_t lq;
  int64_t lk;
  int64_t q_pos0;
  int64_t n_kb;  // key blocks (the last may be partial): ceil(lk / 4)
  int hq;
  int hkv;
  int d;
  int n_sel;
  float scale;
  float scale_log2;
};
// Byte offsets of the backward's workspace parts.
struct BwdLayout {
  size_t dbuf, keys0, keys1, rows0, rows1, start, temp, temp_bytes, total;
};
BwdLayout bwd_layout(int64_t lq, int64_t lk, int hq, int n_sel, int r);
hipError_t launch_sparse_attn_bwd(BwdArgs a, char* ws, size_t ws_bytes, hipStream_t stream);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);

// ---- indexer warm-up (KL distillation) ----
constexpr int kKlMaxGroups = 4;  // KV groups the dense KL passes hold in one wave
struct KlArgs {
  const uint16_t* q;  // [lq][hq][d]
  const uint16_t* k;  // [lk][hkv][d]
  float* lse;         // [lq][hq], dense causal
  float* target;      // [lq][ld], unnormalised pooled probabilities of the scored blocks
  int64_t lq;
  int64_t lk;
  int64_t q_pos0;
  int64_t nblk;
  int64_t ld;
  int hq;
  int hkv;
  int d;
  int r;
  float scale_log2;
};
struct KlLossArgs {
  const float* scores;  // [lq][ld]
  const float* target;  // [lq][ld]
  float* loss;          // [lq]
  float* dscores;       // [lq][ld]
  int64_t lq;
  int64_t q_pos0;
  int64_t nblk;
  int64_t ld;
  int r;
};
struct IdxBwdArgs {
  const uint16_t* q_idx;  // [lq][h_idx][d_idx]
  const float* w;         // [lq][h_idx]
  const uint16_t* kp;     // [nblk][d_idx]
  const float* dscores;   // [lq][ld]
  float* dq_idx;          // [lq][h_idx][d_idx]
  float* dw;              // [lq][h_idx]
  float* dk_pooled;       // [nblk][d_idx]
  float* dk_idx;          // [n_tokens][d_idx] or null
  int64_t lq;
  int64_t q_pos0;
  int64_t nblk;
  int64_t ld;
  int64_t n_tokens;
  int h_idx;
  int d_idx;
  int r;
};
hipError_t launch_kl_target(const KlArgs& a, hipStream_t stream);
hipError_t launch_kl_loss(const KlLossArgs& a, hipStream_t stream);
hipError_t launch_index_scores_bwd(const IdxBwdArgs& a, hipStream_t stream);

// Decode split heuristic for a given n_sel: 4-block steps per wave (1, 2 or 4) and
// workgroups of 4 waves (= partials) per (sequence, head).
int decode_steps_per_split(int n_sel);
int decode_num_splits(int n_sel);

}  // namespace qsa

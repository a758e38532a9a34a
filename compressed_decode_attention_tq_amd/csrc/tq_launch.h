// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include "tq_common.h"

namespace tq {

// Split-context geometry of one decode call.  Every split covers `split_len` tokens
// (a multiple of kSplitAlign) of one (batch, kv head); the number of splits is chosen
// so the grid has enough blocks for the chip.  The same function sizes the workspace.
constexpr int kSplitAlign = 64;
constexpr int kSparseWeights = 8192;  // floats of the Sparse-V pass's per-split weight table

struct SplitPlan {
  int n_splits;
  int split_len;
};

SplitPlan plan_splits(int batch, int n_kv_heads, int ctx_len, int group);
// Splits of the single-launch dense path: about one workgroup per CU, whole 64-token tiles.
SplitPlan plan_fused(int batch, int n_kv_heads, int ctx_len);
// Sparse V's fused first pass: splits of a whole number (<= kMaxChunksPerSplit) of the
// second pass's splits `p`, about as long as the dense plan's.
SplitPlan plan_fused_sparse(int batch, int n_kv_heads, int ctx_len, const SplitPlan &p);
constexpr int kMaxChunksPerSplit = 64;
constexpr int kMaxQueryPositions = 4096;  // query positions of one multi-query call
constexpr int kSmallAppendMax = 8;        // appends of up to this many tokens take one wave per plane
constexpr int kMultiAppendMax = 8;        // new tokens the multi-query launch writes itself

// Workspace layout (byte offsets, 256-byte aligned sections).
struct WorkspaceLayout {
  size_t counters;    // unsigned [batch][n_kv_heads]   zero between calls
  size_t fpart_ml;    // float2 [batch][n_q_heads][fused splits]
  size_t fpart_o;     // float  [batch][n_q_heads][fused splits][128]
  size_t part_ml;     // float2 [batch][n_q_heads][n_splits]      (m, l) per split
  size_t part_o;      // float  [batch][n_q_heads][n_splits][128] rotated-domain sums
  size_t cand_count;  // int    [batch][n_kv_heads][n_splits]      Sparse-V candidates
  size_t cand;        // float  [batch][n_kv_heads][n_splits][split_len][1 + g]
  size_t vpart_ml;    // Sparse V, masked value pass: float2 [batch][n_q_heads][value-pass splits]
  size_t vpart_o;     //   and float [batch][n_q_heads][value-pass splits][128]
  size_t tile_max;    // Sparse V: float [batch][n_q_heads][ceil(ctx_len / 64)] per-tile maxima
  size_t total;
};

WorkspaceLayout workspace_layout(int batch, int n_q_heads, int n_kv_heads, int ctx_len,
                                 bool sparse);
// Multi-query attention (n_q query positions): the single-launch kernel's counters and
// partials only.
struct MultiQueryShape {
  int vgroups, vg_size;
  bool prefill;  // vgroups >= 8: row groups by wave (see DecodeArgs::prefill)
};
constexpr int kPrefillMinGroups = 8;
MultiQueryShape multi_query_shape(int group, int n_q);
WorkspaceLayout workspace_layout_multi(int batch, int n_q_heads, int n_kv_heads, int n_q, int ctx_len);

struct DecodeArgs {
  CacheView k, v;
  const void *q;
  int q_dtype;
  int batch, n_q_heads, n_kv_heads, group;
  const int32_t *seq_lens;
  int ctx_len;
  float scale;
  float ln_tau;  // log(tau), only read when sparse
  int sparse;
  SplitPlan plan;
  float *out, *lse, *scores;
  float2 *part_ml;
  float *part_o;
  int *cand_count;
  float *cand;
  // single-launch dense path: one partial per (batch, query head, split of fplan) and an
  // arrival counter per (batch, kv head) that the last workgroup clears
  SplitPlan fplan;
  float2 *fpart_ml;
  float *fpart_o;
  unsigned *counters;
  // Sparse V: the (m, l) partials (natural log) the LSE is merged from, per (batch, query
  // head): lse_splits of them.  The per-wave first pass writes part_ml (plan splits), the
  // fused first pass fpart_ml (fplan splits).
  const float2 *lse_ml;
  int lse_splits;
  // Query rows of the single-launch kernel: n_q query positions per sequence (1 for decode)
  // give n_q * group rows per kv head, taken vg_size at a time by `vgroups` work items.
  int n_q, vgroups, vg_size;
  // several query positions with at least 8 row groups per kv head (a prefill chunk): a
  // workgroup's 8 waves take 8 row groups over the same split
  int prefill;
  // Append in the same launch (single-query dense decode): the new token of each sequence,
  // [batch][1][n_kv_heads][d] of x_dtype, is quantized into position T - 1 first.
  const void *xk, *xv;
  int x_dtype;
  // Paged caches (block_table != nullptr): k and v view the page pools, with capacity =
  // page_tokens so that plane(page, h) is one page of one kv head; position t of sequence b
  // lies in pool page block_table[b * max_pages + t / page_tokens].
  const int32_t *block_table;
  int max_pages, n_pages;
  // Sparse V, masked value pass (the dense fused kernel after the key pass): its own
  // partials; a.lse_ml / a.lse_splits are the key pass's (m, l) per split
  float2 *vpart_ml;
  float *vpart_o;
  // Sparse V: the key pass writes the largest scaled score (log2 units) of every (batch, query
  // head, 64-token tile) to tile_max[(b * n_q_heads + h) * tile_stride + t / 64]; the value pass
  // visits only the tiles whose maximum reaches some head's threshold
  float *tile_max;
  int tile_stride;
  // QJL keys (qjl_m > 0): beside the key codes, the sign sketch of each key's residual,
  // [batch][n_kv_heads][capacity][qjl_m / 8] bytes, its fp16 norms [batch][n_kv_heads][capacity],
  // and the sketch matrix S [qjl_m][d] fp32
  const uint8_t *qjl_bits;
  const uint16_t *qjl_rnorm;
  const float *qjl_proj;
  int qjl_m;
};

// QJL key quantization: the key cache k (ROWS) gets the codes and norms, bits / res_norms the
// sign sketch of each token's residual and its fp16 norm, from S = proj [128][d] fp32.
struct QjlQuantArgs {
  CacheView k;
  uint8_t *bits;
  uint16_t *res_norms;
  const float *proj;
  const void *x;
  int x_dtype;
  int start_pos, n_tokens;
};
hipError_t launch_qjl_quantize(const QjlQuantArgs &a, int batch, hipStream_t stream);
// QJL keys and plain values of 1..8 tokens in one launch: a.k (with the sketch) as
// launch_qjl_quantize, the value cache vc (groups of 8) from xv as launch_append_small.
hipError_t launch_qjl_quantize_kv_small(const QjlQuantArgs &a, const CacheView &vc, const void *xv, int batch,
                                       hipStream_t stream);
// QJL decode on matrix cores (3-bit codes, 2-bit values, groups up to 8, no Sparse V): the fused
// kernel with the query's sketch and the sign-sketch products.
bool decode_fused_qjl_supported(const DecodeArgs &a);
hipError_t launch_decode_fused_qjl(const DecodeArgs &a, hipStream_t stream);
// QJL decode with Sparse V on matrix cores: key_pass as for the key-only fused pass (no
// candidate records), value_pass the masked value pass over the key pass's partials.
bool decode_fused_qjl_sparse_supported(const DecodeArgs &a);
hipError_t launch_decode_fused_qjl_sparse(const DecodeArgs &key_pass, const DecodeArgs &value_pass,
                                          hipStream_t stream);
// The generic split kernel, the Sparse-V second pass (if a.sparse) and the split merge: any code
// width, group <= 16, and the only path that takes QJL keys.
hipError_t launch_decode_generic(const DecodeArgs &a, hipStream_t stream);

hipError_t launch_quantize(const CacheView &c, int batch, const void *x, int x_dtype,
                           int start_pos, int n_tokens, hipStream_t stream);
hipError_t launch_quantize_kv(const CacheView &kc, const CacheView &vc, int batch, const void *xk,
                              const void *xv, int x_dtype, int start_pos, int n_tokens,
                              hipStream_t stream);
// Appends of 1..kSmallAppendMax tokens to a key cache (rows) and a value cache (groups of 8):
// one block per (batch, kv head, key or value) plane, one wave per token.
hipError_t launch_append_small(const CacheView &kc, const CacheView &vc, int batch, const void *xk,
                               const void *xv, int x_dtype, int start_pos, int n_tokens, hipStream_t stream);
// The same for one cache (x is [batch][n_tokens][n_kv_heads][d]): its layout picks the path.
hipError_t launch_append_small_one(const CacheView &c, int batch, const void *x, int x_dtype, int start_pos,
                                   int n_tokens, hipStream_t stream);
// Appends to paged caches (views of the page pools, capacity = page_tokens): token j of
// sequence b at position start_pos[b] + j; one block per aligned 8-token window of one
// (sequence, kv head, key or value), one wave per token.
hipError_t launch_append_paged(const CacheView &kc, const CacheView &vc, const int32_t *block_table,
                               int max_pages, int n_pages, int batch, const void *xk, const void *xv,
                               int x_dtype, const int32_t *start_pos, int n_tokens, hipStream_t stream);
// Longest split of the paged decode: 64 tiles per wave, so that one lane per tile holds the
// wave's page offsets.  In prefill mode every wave walks every tile of its split: 64 tiles.
constexpr int kPagedMaxSplit = 8 * 64 * 64;
constexpr int kPagedPrefillMaxSplit = 64 * 64;
SplitPlan plan_fused_paged(int batch, int n_kv_heads, int ctx_len);
// Splits of Sparse V's value pass: the dense plan with at most 64 tiles per wave (8 * 64 * 64
// tokens per split), so that one lane per tile decides which tiles a wave needs.
constexpr int kVmaskMaxSplit = 8 * 64 * 64;
SplitPlan plan_fused_vmask(int batch, int n_kv_heads, int ctx_len);
WorkspaceLayout workspace_layout_paged(int batch, int n_q_heads, int n_kv_heads, int ctx_len);
hipError_t launch_decode_fused_paged(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_fused_paged_sparse(const DecodeArgs &key_pass, const DecodeArgs &value_pass,
                                            hipStream_t stream);
// Workspace of the paged calls with several query positions or Sparse V (tau > 0).
WorkspaceLayout workspace_layout_paged_ext(int batch, int n_q_heads, int n_kv_heads, int n_q, int ctx_len, bool sparse);
SplitPlan plan_multi(int batch, int n_kv_heads, const MultiQueryShape &m, int ctx_len);
constexpr int kSearchBlock = 1024;
constexpr int kSearchMaxK = 64;
// Inner-product search candidates in caller scratch: cand [n_q][blocks][k] rank entries
// (order key << 32 | ~index), bnd [n_q][blocks] the keys of each block's k-th best and best,
// blocks = ceil(n / kSearchBlock).
struct SearchState {
  uint64_t *cand;
  uint2 *bnd;
};
// Inner-product search: scores of n_q queries against n database vectors (plane (0, 0) of
// db, 3- or 4-bit rows), each block's k best, then the k best per query.
hipError_t launch_ip_search(const CacheView &db, const void *q, int q_dtype, int n_q, int n, int k, int32_t *out_idx,
                            float *out_score, const SearchState &st, hipStream_t stream);
hipError_t launch_dequantize(const CacheView &c, int batch, void *out, int out_dtype,
                             int start_pos, int n_tokens, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
// Sparse V's two matrix-core passes (key pass, masked value pass); with a.xk set the key pass
// first writes the decode step's new token.  hipErrorNotSupported, with nothing launched,
// where that path does not apply (other widths, groups above 8).
hipError_t launch_sparse_two_pass(const DecodeArgs &a, hipStream_t stream);
int compute_units();
bool decode_mfma_supported(const DecodeArgs &a);
bool decode_fused_supported(const DecodeArgs &a);
// The single-launch kernel covers these widths and shapes (the workspace aside).
bool decode_fused_shape_ok(const DecodeArgs &a);
bool decode_fused_sparse_supported(const DecodeArgs &a);
hipError_t launch_decode_fused_sparse(const DecodeArgs &a, hipStream_t stream);
// Sparse V's masked value pass: the dense single-launch kernel over the dense plan (a.fplan,
// partials a.fpart_ml / a.fpart_o) with the key pass's partials in a.lse_ml.
hipError_t launch_decode_fused_vmask(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_fused(const DecodeArgs &a, int n_cu, hipStream_t stream);
// Validation and argument set-up shared by tq_decode_attn_append and its allocation-free
// variant: fills `a` (everything but the workspace pointers) and the workspace layout `w`;
// returns a tq_status.
int setup_decode_append(const tq_cache *k, const tq_cache *v, const void *xk, const void *xv, int x_dtype,
                        const void *q, int q_dtype, int n_q_heads, const int32_t *seq_lens, int ctx_len,
                        float scale, float *out, float *lse, DecodeArgs &a, WorkspaceLayout &w);
hipError_t launch_decode_mfma(const DecodeArgs &a, int n_cu, hipStream_t stream);

}  // namespace tq

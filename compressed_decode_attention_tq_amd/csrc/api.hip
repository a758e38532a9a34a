// C-ABI entry points: argument validation (before any HIP call), split planning,
// workspace layout and kernel launches.  See include/tq.h for the contract.
#include <cmath>
#include <cstdint>

#include "tq_launch.h"

namespace tq {
namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool valid_bits(int bits) { return bits == 2 || bits == 3 || bits == 4 || bits == 8; }
bool valid_dtype(int dt) { return dt == TQ_F32 || dt == TQ_BF16 || dt == TQ_F16; }

// Largest capacity accepted: keeps every plane offset far inside 64-bit and every token
// index inside int32 arithmetic in the kernels.
constexpr int kMaxCapacity = 1 << 26;

int check_cache(const tq_cache *c) {
  if (c == nullptr) return TQ_ERR_INVALID_ARG;
  if (c->codes == nullptr || c->norms == nullptr || c->centroids == nullptr ||
      c->boundaries == nullptr || c->signs == nullptr)
    return TQ_ERR_INVALID_ARG;
  if (!aligned(c->codes, 16) || !aligned(c->norms, 16) || !aligned(c->centroids, 4) ||
      !aligned(c->boundaries, 4) || !aligned(c->signs, 16))
    return TQ_ERR_INVALID_ARG;
  if (c->batch < 1 || c->n_kv_heads < 1 || c->capacity < 1) return TQ_ERR_INVALID_ARG;
  if (c->layout != TQ_LAYOUT_ROWS && c->layout != TQ_LAYOUT_GROUP8) return TQ_ERR_INVALID_ARG;
  if (c->d != kD) return TQ_ERR_UNSUPPORTED;
  if (!valid_bits(c->bits)) return TQ_ERR_UNSUPPORTED;
  if (c->capacity % kChunk != 0 || c->capacity > kMaxCapacity) return TQ_ERR_UNSUPPORTED;
  if (!(c->table_scale == 0.f || (c->table_scale >= 1.f && c->table_scale <= 2.f))) return TQ_ERR_INVALID_ARG;
  return TQ_OK;
}

CacheView view_of(const tq_cache *c) {
  CacheView v;
  v.codes = c->codes;
  v.norms = c->norms;
  v.centroids = c->centroids;
  v.boundaries = c->boundaries;
  v.signs = c->signs;
  v.bits = c->bits;
  v.layout = c->layout;
  v.n_kv_heads = c->n_kv_heads;
  v.capacity = c->capacity;
  v.table_scale = c->table_scale > 0.f ? c->table_scale : 1.f;
  return v;
}

int hip_status(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_ERR_HIP; }

}  // namespace

SplitPlan plan_splits(int batch, int n_kv_heads, int ctx_len, int group) {
  const long units = (long)batch * n_kv_heads;
  const long target_blocks = 1024;
  // a split's softmax weights [split_len][group] fit the Sparse-V pass's LDS
  const long padded = group <= 4 ? 4 : group <= 8 ? 8 : 16;
  const long max_len = (kSparseWeights / padded) / kSplitAlign * kSplitAlign;
  long s_target = (target_blocks + units - 1) / units;
  if (s_target < 1) s_target = 1;
  long len = (ctx_len + s_target - 1) / s_target;
  len = (len + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
  if (len > max_len) len = max_len;
  if (len < kSplitAlign) len = kSplitAlign;
  long n = (ctx_len + len - 1) / len;
  if (n < 1) n = 1;
  return SplitPlan{(int)n, (int)len};
}

SplitPlan plan_fused(int batch, int n_kv_heads, int ctx_len) {
  const long units = (long)batch * n_kv_heads;
  const long target_groups = 256;       // about one workgroup per CU
  const long max_len = 1L << 20;        // keeps in-split byte offsets within 32 bits
  const long min_len = 8 * kSplitAlign;  // one tile for each of the 8 waves of a workgroup
  long s_target = (target_groups + units - 1) / units;
  if (s_target < 1) s_target = 1;
  long len = (ctx_len + s_target - 1) / s_target;
  len = (len + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
  if (len < min_len) len = min_len;
  if (len > max_len) len = max_len;
  long n = (ctx_len + len - 1) / len;
  if (n < 1) n = 1;
  return SplitPlan{(int)n, (int)len};
}

SplitPlan plan_fused_sparse(int batch, int n_kv_heads, int ctx_len, const SplitPlan &p) {
  const SplitPlan d = plan_fused(batch, n_kv_heads, ctx_len);
  long k = (d.split_len + p.split_len / 2) / p.split_len;
  if (k < 1) k = 1;
  if (k > kMaxChunksPerSplit) k = kMaxChunksPerSplit;
  const long len = k * p.split_len;
  long n = (ctx_len + len - 1) / len;
  if (n < 1) n = 1;
  return SplitPlan{(int)n, (int)len};
}

WorkspaceLayout workspace_layout(int batch, int n_q_heads, int n_kv_heads, int ctx_len,
                                 bool sparse) {
  const SplitPlan p = plan_splits(batch, n_kv_heads, ctx_len, n_q_heads / n_kv_heads);
  const SplitPlan fp = sparse ? plan_fused_sparse(batch, n_kv_heads, ctx_len, p)
                              : plan_fused(batch, n_kv_heads, ctx_len);
  const size_t heads = (size_t)batch * n_q_heads * p.n_splits;
  const size_t fheads = (size_t)batch * n_q_heads * fp.n_splits;
  WorkspaceLayout w{};
  size_t off = 0;
  w.counters = off;  // first, so no other section of any layout ever overlaps it
  off = align_up(off + (size_t)batch * n_kv_heads * sizeof(unsigned), 256);
  w.fpart_ml = off;
  off = align_up(off + fheads * sizeof(float2), 256);
  w.fpart_o = off;
  off = align_up(off + fheads * kD * sizeof(float), 256);
  w.part_ml = off;
  off = align_up(off + heads * sizeof(float2), 256);
  w.part_o = off;
  off = align_up(off + heads * kD * sizeof(float), 256);
  w.cand_count = off;
  w.cand = off;
  if (sparse) {
    const size_t units = (size_t)batch * n_kv_heads * p.n_splits;
    const int g = n_q_heads / n_kv_heads;
    off = align_up(off + units * sizeof(int), 256);
    w.cand = off;
    off = align_up(off + units * (size_t)p.split_len * (1 + g) * sizeof(float), 256);
    const SplitPlan dp = plan_fused_vmask(batch, n_kv_heads, ctx_len);  // value pass: <= 64 tiles per split
    const size_t vheads = (size_t)batch * n_q_heads * dp.n_splits;
    w.vpart_ml = off;
    off = align_up(off + vheads * sizeof(float2), 256);
    w.vpart_o = off;
    off = align_up(off + vheads * kD * sizeof(float), 256);
    w.tile_max = off;
    off = align_up(off + (size_t)batch * n_q_heads * ((ctx_len + 63) / 64) * sizeof(float), 256);
  }
  w.total = off;
  return w;
}

MultiQueryShape multi_query_shape(int group, int n_q) {
  const long rows = (long)group * n_q;
  const int vgroups = (int)((rows + 7) / 8);
  return MultiQueryShape{vgroups, (int)((rows + vgroups - 1) / vgroups), vgroups >= kPrefillMinGroups};
}

// Splits of a multi-query call: one work item per (batch, kv head, row group, split), or with
// prefill one per (batch, kv head, 8 row groups, split).
SplitPlan plan_multi(int batch, int n_kv_heads, const MultiQueryShape &m, int ctx_len) {
  const int items = m.prefill ? (m.vgroups + 7) / 8 : m.vgroups;
  return plan_fused(batch, n_kv_heads * items, ctx_len);
}

WorkspaceLayout workspace_layout_multi(int batch, int n_q_heads, int n_kv_heads, int n_q, int ctx_len) {
  const MultiQueryShape m = multi_query_shape(n_q_heads / n_kv_heads, n_q);
  const SplitPlan fp = plan_multi(batch, n_kv_heads, m, ctx_len);
  const size_t rows = (size_t)batch * n_q * n_q_heads * fp.n_splits;
  WorkspaceLayout w{};
  size_t off = 0;
  w.counters = off;
  off = align_up(off + (size_t)batch * n_kv_heads * m.vgroups * sizeof(unsigned), 256);
  w.fpart_ml = off;
  off = align_up(off + rows * sizeof(float2), 256);
  w.fpart_o = off;
  off = align_up(off + rows * kD * sizeof(float), 256);
  w.part_ml = w.part_o = w.cand_count = w.cand = off;
  w.total = off;
  return w;
}

// Splits of a paged multi-query call: those of the contiguous call, capped so that a wave's
// page offsets fit its lanes (one tile per lane; in prefill mode every wave walks every tile).
SplitPlan plan_paged_multi(int batch, int n_kv_heads, const MultiQueryShape &m, int ctx_len) {
  SplitPlan fp = plan_multi(batch, n_kv_heads, m, ctx_len);
  const int cap = m.prefill ? kPagedPrefillMaxSplit : kPagedMaxSplit;
  if (fp.split_len > cap) fp = SplitPlan{(ctx_len + cap - 1) / cap, cap};
  return fp;
}

SplitPlan plan_fused_paged(int batch, int n_kv_heads, int ctx_len) {
  SplitPlan p = plan_fused(batch, n_kv_heads, ctx_len);
  if (p.split_len > kPagedMaxSplit) {
    p.split_len = kPagedMaxSplit;
    p.n_splits = (ctx_len + kPagedMaxSplit - 1) / kPagedMaxSplit;
  }
  return p;
}

SplitPlan plan_fused_vmask(int batch, int n_kv_heads, int ctx_len) {
  SplitPlan p = plan_fused(batch, n_kv_heads, ctx_len);
  if (p.split_len > kVmaskMaxSplit) {
    p.split_len = kVmaskMaxSplit;
    p.n_splits = (ctx_len + kVmaskMaxSplit - 1) / kVmaskMaxSplit;
  }
  return p;
}

WorkspaceLayout workspace_layout_paged(int batch, int n_q_heads, int n_kv_heads, int ctx_len) {
  const SplitPlan fp = plan_fused_paged(batch, n_kv_heads, ctx_len);
  const size_t rows = (size_t)batch * n_q_heads * fp.n_splits;
  WorkspaceLayout w{};
  size_t off = 0;
  w.counters = off;
  off = align_up(off + (size_t)batch * n_kv_heads * sizeof(unsigned), 256);
  w.fpart_ml = off;
  off = align_up(off + rows * sizeof(float2), 256);
  w.fpart_o = off;
  off = align_up(off + rows * kD * sizeof(float), 256);
  w.part_ml = w.part_o = w.cand_count = w.cand = off;
  w.total = off;
  return w;
}

WorkspaceLayout workspace_layout_paged_ext(int batch, int n_q_heads, int n_kv_heads, int n_q, int ctx_len,
                                          bool sparse) {
  WorkspaceLayout w{};
  size_t off = 0;
  w.counters = off;
  if (!sparse) {  // several query positions (a long chunk in prefill mode, as without pages)
    const MultiQueryShape m = multi_query_shape(n_q_heads / n_kv_heads, n_q);
    const SplitPlan fp = plan_paged_multi(batch, n_kv_heads, m, ctx_len);
    const size_t rows = (size_t)batch * n_q * n_q_heads * fp.n_splits;
    off = align_up(off + (size_t)batch * n_kv_heads * m.vgroups * sizeof(unsigned), 256);
    w.fpart_ml = off;
    off = align_up(off + rows * sizeof(float2), 256);
    w.fpart_o = off;
    off = align_up(off + rows * kD * sizeof(float), 256);
    w.part_ml = w.part_o = w.cand_count = w.cand = w.vpart_ml = w.vpart_o = w.tile_max = off;
  } else {  // Sparse V: the key pass's (m, l) partials, the value pass's partials, the tile maxima
    const SplitPlan kp = plan_fused_paged(batch, n_kv_heads, ctx_len);
    const SplitPlan vp = plan_fused_vmask(batch, n_kv_heads, ctx_len);
    off = align_up(off + (size_t)batch * n_kv_heads * sizeof(unsigned), 256);
    w.fpart_ml = off;
    off = align_up(off + (size_t)batch * n_q_heads * kp.n_splits * sizeof(float2), 256);
    w.fpart_o = w.part_ml = w.part_o = w.cand_count = w.cand = off;
    w.vpart_ml = off;
    off = align_up(off + (size_t)batch * n_q_heads * vp.n_splits * sizeof(float2), 256);
    w.vpart_o = off;
    off = align_up(off + (size_t)batch * n_q_heads * vp.n_splits * kD * sizeof(float), 256);
    w.tile_max = off;
    off = align_up(off + (size_t)batch * n_q_heads * ((ctx_len + 63) / 64) * sizeof(float), 256);
  }
  w.total = off;
  return w;
}

struct SearchLayout {
  size_t cand, bnd, total;
};

SearchLayout search_layout(int n_q, int n, int k) {
  const size_t blocks = (size_t)n_q * ((n + kSearchBlock - 1) / kSearchBlock);
  SearchLayout w{};
  size_t off = 0;
  w.cand = off;
  off = align_up(off + blocks * k * sizeof(uint64_t), 256);
  w.bnd = off;
  off = align_up(off + blocks * sizeof(uint2), 256);
  w.total = off;
  return w;
}

bool search_shape_ok(int n_q, int n, int k) {
  return n_q >= 1 && n_q <= 65535 * 8 && n >= 1 && k >= 1 && k <= kSearchMaxK;
}

int check_paged(const tq_paged_cache *c) {
  if (c == nullptr) return TQ_ERR_INVALID_ARG;
  if (c->codes == nullptr || c->norms == nullptr || c->block_table == nullptr || c->centroids == nullptr ||
      c->boundaries == nullptr || c->signs == nullptr)
    return TQ_ERR_INVALID_ARG;
  if (!aligned(c->codes, 16) || !aligned(c->norms, 16) || !aligned(c->block_table, 4) ||
      !aligned(c->centroids, 4) || !aligned(c->boundaries, 4) || !aligned(c->signs, 16))
    return TQ_ERR_INVALID_ARG;
  if (c->batch < 1 || c->n_kv_heads < 1 || c->page_tokens < 1 || c->n_pages < 1 || c->max_pages < 1)
    return TQ_ERR_INVALID_ARG;
  if (c->layout != TQ_LAYOUT_ROWS && c->layout != TQ_LAYOUT_GROUP8) return TQ_ERR_INVALID_ARG;
  if (c->d != kD) return TQ_ERR_UNSUPPORTED;
  if (!valid_bits(c->bits)) return TQ_ERR_UNSUPPORTED;
  if (c->page_tokens % kChunk != 0 || c->page_tokens > kMaxCapacity) return TQ_ERR_UNSUPPORTED;
  if (!(c->table_scale == 0.f || (c->table_scale >= 1.f && c->table_scale <= 2.f))) return TQ_ERR_INVALID_ARG;
  // 32-bit offsets in the kernels: pool code bytes below 3 GiB, positions below 2^30
  const double pool = (double)c->n_pages * c->n_kv_heads * c->page_tokens * kD * c->bits / 8;
  if (pool >= 3.0 * (1u << 30) || (double)c->max_pages * c->page_tokens >= (double)(1 << 30))
    return TQ_ERR_UNSUPPORTED;
  return TQ_OK;
}

// a view of the pool in which plane(page, h) is one page of one kv head
CacheView view_of_pool(const tq_paged_cache *c) {
  CacheView v;
  v.codes = c->codes;
  v.norms = c->norms;
  v.centroids = c->centroids;
  v.boundaries = c->boundaries;
  v.signs = c->signs;
  v.bits = c->bits;
  v.layout = c->layout;
  v.n_kv_heads = c->n_kv_heads;
  v.capacity = c->page_tokens;
  v.table_scale = c->table_scale > 0.f ? c->table_scale : 1.f;
  return v;
}

int check_paged_pair(const tq_paged_cache *k, const tq_paged_cache *v) {
  int st = check_paged(k);
  if (st != TQ_OK) return st;
  st = check_paged(v);
  if (st != TQ_OK) return st;
  if (k->batch != v->batch || k->n_kv_heads != v->n_kv_heads || k->page_tokens != v->page_tokens ||
      k->n_pages != v->n_pages || k->max_pages != v->max_pages || k->block_table != v->block_table)
    return TQ_ERR_INVALID_ARG;
  if (k->layout != TQ_LAYOUT_ROWS || v->layout != TQ_LAYOUT_GROUP8) return TQ_ERR_INVALID_ARG;
  return TQ_OK;
}

int check_sketch(const tq_qjl_sketch *s) {
  if (s == nullptr || s->bits == nullptr || s->res_norms == nullptr || s->proj == nullptr) return TQ_ERR_INVALID_ARG;
  if (!aligned(s->bits, 16) || !aligned(s->res_norms, 2) || !aligned(s->proj, 16)) return TQ_ERR_INVALID_ARG;
  if (s->m != kD) return TQ_ERR_UNSUPPORTED;
  return TQ_OK;
}

int setup_decode(const tq_cache *k, const tq_cache *v, const void *q, int q_dtype, int n_q_heads,
                 const int32_t *seq_lens, int ctx_len, float scale, float sparse_v_tau, float *out, float *lse,
                 float *scores, void *workspace, size_t workspace_bytes, DecodeArgs &a) {
  int st = check_cache(k);
  if (st != TQ_OK) return st;
  st = check_cache(v);
  if (st != TQ_OK) return st;
  if (k->batch != v->batch || k->n_kv_heads != v->n_kv_heads || k->capacity != v->capacity ||
      k->signs != v->signs)
    return TQ_ERR_INVALID_ARG;
  if (k->layout != TQ_LAYOUT_ROWS || v->layout != TQ_LAYOUT_GROUP8) return TQ_ERR_UNSUPPORTED;
  if (q == nullptr || !aligned(q, 16) || !valid_dtype(q_dtype)) return TQ_ERR_INVALID_ARG;
  if (out == nullptr || !aligned(out, 16)) return TQ_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return TQ_ERR_INVALID_ARG;
  if (scores != nullptr && !aligned(scores, 4)) return TQ_ERR_INVALID_ARG;
  if (seq_lens != nullptr && !aligned(seq_lens, 4)) return TQ_ERR_INVALID_ARG;
  if (n_q_heads < 1 || n_q_heads % k->n_kv_heads != 0) return TQ_ERR_INVALID_ARG;
  const int group = n_q_heads / k->n_kv_heads;
  if (group > 16) return TQ_ERR_UNSUPPORTED;
  if (ctx_len < 0) return TQ_ERR_INVALID_ARG;
  if (ctx_len > k->capacity) return TQ_ERR_CAPACITY;
  if (!std::isfinite(scale)) return TQ_ERR_INVALID_ARG;
  if (!(sparse_v_tau >= 0.f && sparse_v_tau < 1.f)) return TQ_ERR_INVALID_ARG;
  const bool sparse = sparse_v_tau > 0.f;
  const WorkspaceLayout w = workspace_layout(k->batch, n_q_heads, k->n_kv_heads, ctx_len, sparse);
  if (workspace == nullptr || !aligned(workspace, 256)) return TQ_ERR_INVALID_ARG;
  if (workspace_bytes < w.total) return TQ_ERR_WORKSPACE;

  a = DecodeArgs{};
  a.k = view_of(k);
  a.v = view_of(v);
  a.q = q;
  a.q_dtype = q_dtype;
  a.batch = k->batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = k->n_kv_heads;
  a.group = group;
  a.seq_lens = seq_lens;
  a.ctx_len = ctx_len;
  a.scale = scale;
  a.ln_tau = sparse ? std::log(sparse_v_tau) : 0.f;
  a.sparse = sparse ? 1 : 0;
  a.n_q = 1;
  a.vgroups = 1;
  a.vg_size = group;
  a.plan = plan_splits(k->batch, k->n_kv_heads, ctx_len, group);
  a.fplan = sparse ? plan_fused_sparse(k->batch, k->n_kv_heads, ctx_len, a.plan)
                   : plan_fused(k->batch, k->n_kv_heads, ctx_len);
  a.out = out;
  a.lse = lse;
  a.scores = scores;
  char *ws = static_cast<char *>(workspace);
  a.part_ml = reinterpret_cast<float2 *>(ws + w.part_ml);
  a.part_o = reinterpret_cast<float *>(ws + w.part_o);
  a.cand_count = reinterpret_cast<int *>(ws + w.cand_count);
  a.cand = reinterpret_cast<float *>(ws + w.cand);
  a.counters = reinterpret_cast<unsigned *>(ws + w.counters);
  a.fpart_ml = reinterpret_cast<float2 *>(ws + w.fpart_ml);
  a.fpart_o = reinterpret_cast<float *>(ws + w.fpart_o);
  if (a.sparse) {
    a.vpart_ml = reinterpret_cast<float2 *>(ws + w.vpart_ml);
    a.vpart_o = reinterpret_cast<float *>(ws + w.vpart_o);
    a.tile_max = reinterpret_cast<float *>(ws + w.tile_max);
    a.tile_stride = (ctx_len + 63) / 64;
  }
  return TQ_OK;
}

int setup_decode_append(const tq_cache *k, const tq_cache *v, const void *xk, const void *xv, int x_dtype,
                        const void *q, int q_dtype, int n_q_heads, const int32_t *seq_lens, int ctx_len,
                        float scale, float *out, float *lse, DecodeArgs &a, WorkspaceLayout &w) {
  int st = check_cache(k);
  if (st != TQ_OK) return st;
  st = check_cache(v);
  if (st != TQ_OK) return st;
  if (k->batch != v->batch || k->n_kv_heads != v->n_kv_heads || k->capacity != v->capacity ||
      k->signs != v->signs)
    return TQ_ERR_INVALID_ARG;
  if (k->layout != TQ_LAYOUT_ROWS || v->layout != TQ_LAYOUT_GROUP8) return TQ_ERR_UNSUPPORTED;
  if (xk == nullptr || xv == nullptr || !aligned(xk, 16) || !aligned(xv, 16) || !valid_dtype(x_dtype))
    return TQ_ERR_INVALID_ARG;
  if (q == nullptr || !aligned(q, 16) || !valid_dtype(q_dtype)) return TQ_ERR_INVALID_ARG;
  if (out == nullptr || !aligned(out, 16)) return TQ_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return TQ_ERR_INVALID_ARG;
  if (seq_lens != nullptr && !aligned(seq_lens, 4)) return TQ_ERR_INVALID_ARG;
  if (n_q_heads < 1 || n_q_heads % k->n_kv_heads != 0) return TQ_ERR_INVALID_ARG;
  const int group = n_q_heads / k->n_kv_heads;
  if (group > 16) return TQ_ERR_UNSUPPORTED;
  if (ctx_len < 0) return TQ_ERR_INVALID_ARG;
  if (ctx_len > k->capacity) return TQ_ERR_CAPACITY;
  if (!std::isfinite(scale)) return TQ_ERR_INVALID_ARG;
  w = workspace_layout(k->batch, n_q_heads, k->n_kv_heads, ctx_len, false);
  a = DecodeArgs{};
  a.k = view_of(k);
  a.v = view_of(v);
  a.q = q;
  a.q_dtype = q_dtype;
  a.batch = k->batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = k->n_kv_heads;
  a.group = group;
  a.seq_lens = seq_lens;
  a.ctx_len = ctx_len;
  a.scale = scale;
  a.n_q = 1;
  a.vgroups = 1;
  a.vg_size = group;
  a.plan = plan_splits(k->batch, k->n_kv_heads, ctx_len, group);
  a.fplan = plan_fused(k->batch, k->n_kv_heads, ctx_len);
  a.out = out;
  a.lse = lse;
  return TQ_OK;
}

}  // namespace tq

using namespace tq;

extern "C" {

const char *tq_status_string(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_CAPACITY: return "token range exceeds cache capacity";
    case TQ_ERR_WORKSPACE: return "workspace too small";
    case TQ_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

size_t tq_code_bytes(int d, int bits, int batch, int n_kv_heads, int capacity) {
  if (d < 1 || batch < 1 || n_kv_heads < 1 || capacity < 1 || bits < 1 || bits > 8) return 0;
  return (size_t)batch * n_kv_heads * capacity * (size_t)d * bits / 8;
}

size_t tq_decode_attn_multi_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int n_q,
                                            int ctx_len) {
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < n_kv_heads || n_q_heads % n_kv_heads != 0 ||
      n_q < 1 || n_q > kMaxQueryPositions || ctx_len < 0)
    return 0;
  return workspace_layout_multi(batch, n_q_heads, n_kv_heads, n_q, ctx_len).total;
}

size_t tq_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int ctx_len,
                                 float sparse_v_tau) {
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < n_kv_heads || n_q_heads % n_kv_heads != 0 ||
      ctx_len < 0 || !(sparse_v_tau >= 0.f && sparse_v_tau < 1.f))
    return 0;
  return workspace_layout(batch, n_q_heads, n_kv_heads, ctx_len, sparse_v_tau > 0.f).total;
}

int tq_quantize_append(const tq_cache *c, const void *x, int x_dtype, int start_pos,
                       int n_tokens, void *hip_stream) {
  int st = check_cache(c);
  if (st != TQ_OK) return st;
  if (x == nullptr || !aligned(x, 16) || !valid_dtype(x_dtype)) return TQ_ERR_INVALID_ARG;
  if (start_pos < 0 || n_tokens < 0) return TQ_ERR_INVALID_ARG;
  if ((long)start_pos + n_tokens > c->capacity) return TQ_ERR_CAPACITY;
  if (n_tokens == 0) return TQ_OK;
  if (n_tokens <= kSmallAppendMax)  // decode steps and short drafts: one wave per token
    return hip_status(launch_append_small_one(view_of(c), c->batch, x, x_dtype, start_pos, n_tokens,
                                              static_cast<hipStream_t>(hip_stream)));
  return hip_status(launch_quantize(view_of(c), c->batch, x, x_dtype, start_pos, n_tokens,
                                    static_cast<hipStream_t>(hip_stream)));
}

int tq_quantize_append_kv(const tq_cache *k, const tq_cache *v, const void *xk, const void *xv,
                          int x_dtype, int start_pos, int n_tokens, void *hip_stream) {
  int st = check_cache(k);
  if (st != TQ_OK) return st;
  st = check_cache(v);
  if (st != TQ_OK) return st;
  if (k->layout != TQ_LAYOUT_ROWS || v->layout != TQ_LAYOUT_GROUP8) return TQ_ERR_INVALID_ARG;
  if (k->batch != v->batch || k->n_kv_heads != v->n_kv_heads || k->capacity != v->capacity)
    return TQ_ERR_INVALID_ARG;
  if (xk == nullptr || xv == nullptr || !aligned(xk, 16) || !aligned(xv, 16) || !valid_dtype(x_dtype))
    return TQ_ERR_INVALID_ARG;
  if (start_pos < 0 || n_tokens < 0) return TQ_ERR_INVALID_ARG;
  if ((long)start_pos + n_tokens > k->capacity) return TQ_ERR_CAPACITY;
  if (n_tokens == 0) return TQ_OK;
  if (n_tokens <= kSmallAppendMax)  // decode steps and short drafts: one wave per plane
    return hip_status(launch_append_small(view_of(k), view_of(v), k->batch, xk, xv, x_dtype, start_pos,
                                          n_tokens, static_cast<hipStream_t>(hip_stream)));
  return hip_status(launch_quantize_kv(view_of(k), view_of(v), k->batch, xk, xv, x_dtype, start_pos,
                                       n_tokens, static_cast<hipStream_t>(hip_stream)));
}

int tq_dequantize(const tq_cache *c, int start_pos, int n_tokens, void *out, int out_dtype,
                  void *hip_stream) {
  int st = check_cache(c);
  if (st != TQ_OK) return st;
  if (out == nullptr || !aligned(out, 16) || !valid_dtype(out_dtype)) return TQ_ERR_INVALID_ARG;
  if (start_pos < 0 || n_tokens < 0) return TQ_ERR_INVALID_ARG;
  if ((long)start_pos + n_tokens > c->capacity) return TQ_ERR_CAPACITY;
  if (n_tokens == 0) return TQ_OK;
  return hip_status(launch_dequantize(view_of(c), c->batch, out, out_dtype, start_pos, n_tokens,
                                      static_cast<hipStream_t>(hip_stream)));
}

int tq_decode_attn(const tq_cache *k, const tq_cache *v, const void *q, int q_dtype,
                   int n_q_heads, const int32_t *seq_lens, int ctx_len, float scale,
                   float sparse_v_tau, float *out, float *lse, float *scores, void *workspace,
                   size_t workspace_bytes, void *hip_stream) {
  DecodeArgs a{};
  const int st = setup_decode(k, v, q, q_dtype, n_q_heads, seq_lens, ctx_len, scale, sparse_v_tau, out, lse, scores,
                              workspace, workspace_bytes, a);
  if (st != TQ_OK) return st;
  return hip_status(launch_decode(a, static_cast<hipStream_t>(hip_stream)));
}

int tq_qjl_quantize_append(const tq_cache *k, const tq_qjl_sketch *s, const void *x, int x_dtype, int start_pos,
                           int n_tokens, void *hip_stream) {
  int st = check_cache(k);
  if (st != TQ_OK) return st;
  st = check_sketch(s);
  if (st != TQ_OK) return st;
  if (k->layout != TQ_LAYOUT_ROWS) return TQ_ERR_INVALID_ARG;
  if (x == nullptr || !aligned(x, 16) || !valid_dtype(x_dtype)) return TQ_ERR_INVALID_ARG;
  if (start_pos < 0 || n_tokens < 0) return TQ_ERR_INVALID_ARG;
  if ((long)start_pos + n_tokens > k->capacity) return TQ_ERR_CAPACITY;
  if (n_tokens == 0) return TQ_OK;
  QjlQuantArgs a{};
  a.k = view_of(k);
  a.bits = s->bits;
  a.res_norms = s->res_norms;
  a.proj = s->proj;
  a.x = x;
  a.x_dtype = x_dtype;
  a.start_pos = start_pos;
  a.n_tokens = n_tokens;
  return hip_status(launch_qjl_quantize(a, k->batch, static_cast<hipStream_t>(hip_stream)));
}

int tq_qjl_quantize_append_kv(const tq_cache *k, const tq_qjl_sketch *s, const tq_cache *v, const void *xk,
                              const void *xv, int x_dtype, int start_pos, int n_tokens, void *hip_stream) {
  int st = check_cache(k);
  if (st != TQ_OK) return st;
  st = check_sketch(s);
  if (st != TQ_OK) return st;
  st = check_cache(v);
  if (st != TQ_OK) return st;
  if (k->layout != TQ_LAYOUT_ROWS || v->layout != TQ_LAYOUT_GROUP8) return TQ_ERR_INVALID_ARG;
  if (k->batch != v->batch || k->n_kv_heads != v->n_kv_heads || k->capacity != v->capacity)
    return TQ_ERR_INVALID_ARG;
  if (xk == nullptr || xv == nullptr || !aligned(xk, 16) || !aligned(xv, 16) || !valid_dtype(x_dtype))
    return TQ_ERR_INVALID_ARG;
  if (start_pos < 0 || n_tokens < 0) return TQ_ERR_INVALID_ARG;
  if ((long)start_pos + n_tokens > k->capacity) return TQ_ERR_CAPACITY;
  if (n_tokens == 0) return TQ_OK;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  QjlQuantArgs a{};
  a.k = view_of(k);
  a.bits = s->bits;
  a.res_norms = s->res_norms;
  a.proj = s->proj;
  a.x = xk;
  a.x_dtype = x_dtype;
  a.start_pos = start_pos;
  a.n_tokens = n_tokens;
  if (n_tokens <= kSmallAppendMax && k->batch <= 65535 && k->n_kv_heads <= 65535)  // a decode step: one launch
    return hip_status(launch_qjl_quantize_kv_small(a, view_of(v), xv, k->batch, stream));
  st = hip_status(launch_qjl_quantize(a, k->batch, stream));
  if (st != TQ_OK) return st;
  return hip_status(launch_quantize(view_of(v), v->batch, xv, x_dtype, start_pos, n_tokens, stream));
}

int tq_qjl_decode_attn(const tq_cache *k, const tq_qjl_sketch *ks, const tq_cache *v, const void *q, int q_dtype,
                       int n_q_heads, const int32_t *seq_lens, int ctx_len, float scale, float sparse_v_tau,
                       float *out, float *lse, float *scores, void *workspace, size_t workspace_bytes,
                       void *hip_stream) {
  int st = check_sketch(ks);
  if (st != TQ_OK) return st;
  DecodeArgs a{};
  st = setup_decode(k, v, q, q_dtype, n_q_heads, seq_lens, ctx_len, scale, sparse_v_tau, out, lse, scores, workspace,
                    workspace_bytes, a);
  if (st != TQ_OK) return st;
  a.qjl_bits = ks->bits;
  a.qjl_rnorm = ks->res_norms;
  a.qjl_proj = ks->proj;
  a.qjl_m = ks->m;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  // 3-bit codes, 2-bit values, groups up to 8, no Sparse V: one launch on matrix cores
  if (decode_fused_qjl_supported(a)) return hip_status(launch_decode_fused_qjl(a, stream));
  if (a.sparse) {  // with Sparse V: the key pass for the LSE, then the masked value pass
    DecodeArgs k1 = a;
    k1.cand = nullptr;
    k1.cand_count = nullptr;
    DecodeArgs v2 = a;
    v2.sparse = 0;
    v2.lse_ml = a.fpart_ml;
    v2.lse_splits = a.fplan.n_splits;
    v2.fplan = plan_fused_vmask(a.batch, a.n_kv_heads, a.ctx_len);  // at most 64 tiles per split
    v2.fpart_ml = a.vpart_ml;
    v2.fpart_o = a.vpart_o;
    if (decode_fused_qjl_sparse_supported(k1) && decode_fused_supported(v2))
      return hip_status(launch_decode_fused_qjl_sparse(k1, v2, stream));
  }
  return hip_status(launch_decode_generic(a, stream));
}

int tq_decode_attn_append(const tq_cache *k, const tq_cache *v, const void *xk, const void *xv,
                          int x_dtype, const void *q, int q_dtype, int n_q_heads,
                          const int32_t *seq_lens, int ctx_len, float scale, float *out, float *lse,
                          void *workspace, size_t workspace_bytes, void *hip_stream) {
  DecodeArgs a{};
  WorkspaceLayout w{};
  const int st = setup_decode_append(k, v, xk, xv, x_dtype, q, q_dtype, n_q_heads, seq_lens, ctx_len, scale, out,
                                     lse, a, w);
  if (st != TQ_OK) return st;
  if (workspace == nullptr || !aligned(workspace, 256)) return TQ_ERR_INVALID_ARG;
  if (workspace_bytes < w.total) return TQ_ERR_WORKSPACE;
  char *ws = static_cast<char *>(workspace);
  a.part_ml = reinterpret_cast<float2 *>(ws + w.part_ml);
  a.part_o = reinterpret_cast<float *>(ws + w.part_o);
  a.cand_count = reinterpret_cast<int *>(ws + w.cand_count);
  a.cand = reinterpret_cast<float *>(ws + w.cand);
  a.counters = reinterpret_cast<unsigned *>(ws + w.counters);
  a.fpart_ml = reinterpret_cast<float2 *>(ws + w.fpart_ml);
  a.fpart_o = reinterpret_cast<float *>(ws + w.fpart_o);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (decode_fused_supported(a)) {  // one launch: append, then attend
    a.xk = xk;
    a.xv = xv;
    a.x_dtype = x_dtype;
    return hip_status(launch_decode_fused(a, compute_units(), stream));
  }
  // other code widths: the append kernel, then the decode path (one common position only)
  if (seq_lens != nullptr) return TQ_ERR_UNSUPPORTED;
  if (ctx_len >= 1) {
    const hipError_t e = launch_append_small(a.k, a.v, k->batch, xk, xv, x_dtype, ctx_len - 1, 1, stream);
    if (e != hipSuccess) return TQ_ERR_HIP;
  }
  return hip_status(launch_decode(a, stream));
}

int tq_decode_attn_append_sparse(const tq_cache *k, const tq_cache *v, const void *xk, const void *xv, int x_dtype,
                                 const void *q, int q_dtype, int n_q_heads, const int32_t *seq_lens, int ctx_len,
                                 float scale, float sparse_v_tau, float *out, float *lse, void *workspace,
                                 size_t workspace_bytes, void *hip_stream) {
  if (!(sparse_v_tau >= 0.f && sparse_v_tau < 1.f)) return TQ_ERR_INVALID_ARG;
  if (sparse_v_tau == 0.f)
    return tq_decode_attn_append(k, v, xk, xv, x_dtype, q, q_dtype, n_q_heads, seq_lens, ctx_len, scale, out, lse,
                                 workspace, workspace_bytes, hip_stream);
  DecodeArgs chk{};
  WorkspaceLayout w{};
  int st = setup_decode_append(k, v, xk, xv, x_dtype, q, q_dtype, n_q_heads, seq_lens, ctx_len, scale, out, lse,
                               chk, w);  // the append's checks
  if (st != TQ_OK) return st;
  DecodeArgs a{};
  st = setup_decode(k, v, q, q_dtype, n_q_heads, seq_lens, ctx_len, scale, sparse_v_tau, out, lse, nullptr, workspace,
                    workspace_bytes, a);
  if (st != TQ_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  DecodeArgs k1 = a;  // the key pass writes each sequence's new token at T - 1 first
  k1.xk = xk;
  k1.xv = xv;
  k1.x_dtype = x_dtype;
  hipError_t e = launch_sparse_two_pass(k1, stream);
  if (e != hipErrorNotSupported) return hip_status(e);
  // other code widths or groups: the append kernel, then the decode call (one common position)
  if (seq_lens != nullptr) return TQ_ERR_UNSUPPORTED;
  if (ctx_len >= 1) {
    e = launch_append_small(a.k, a.v, k->batch, xk, xv, x_dtype, ctx_len - 1, 1, stream);
    if (e != hipSuccess) return TQ_ERR_HIP;
  }
  return hip_status(launch_decode(a, stream));
}

// Validation and arguments of a multi-query call (everything but the append inputs).
static int setup_multi(const tq_cache *k, const tq_cache *v, const void *q, int q_dtype, int n_q_heads, int n_q,
                       const int32_t *seq_lens, int ctx_len, float scale, float *out, float *lse, void *workspace,
                       size_t workspace_bytes, DecodeArgs &a) {
  int st = check_cache(k);
  if (st != TQ_OK) return st;
  st = check_cache(v);
  if (st != TQ_OK) return st;
  if (k->batch != v->batch || k->n_kv_heads != v->n_kv_heads || k->capacity != v->capacity ||
      k->signs != v->signs)
    return TQ_ERR_INVALID_ARG;
  if (k->layout != TQ_LAYOUT_ROWS || v->layout != TQ_LAYOUT_GROUP8) return TQ_ERR_UNSUPPORTED;
  if (q == nullptr || !aligned(q, 16) || !valid_dtype(q_dtype)) return TQ_ERR_INVALID_ARG;
  if (out == nullptr || !aligned(out, 16)) return TQ_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return TQ_ERR_INVALID_ARG;
  if (seq_lens != nullptr && !aligned(seq_lens, 4)) return TQ_ERR_INVALID_ARG;
  if (n_q_heads < 1 || n_q_heads % k->n_kv_heads != 0) return TQ_ERR_INVALID_ARG;
  if (n_q < 1 || n_q > kMaxQueryPositions) return TQ_ERR_INVALID_ARG;
  if (ctx_len < 0) return TQ_ERR_INVALID_ARG;
  if (ctx_len > k->capacity) return TQ_ERR_CAPACITY;
  if (!std::isfinite(scale)) return TQ_ERR_INVALID_ARG;
  const int group = n_q_heads / k->n_kv_heads;
  const WorkspaceLayout w = workspace_layout_multi(k->batch, n_q_heads, k->n_kv_heads, n_q, ctx_len);
  if (workspace == nullptr || !aligned(workspace, 256)) return TQ_ERR_INVALID_ARG;
  if (workspace_bytes < w.total) return TQ_ERR_WORKSPACE;

  const MultiQueryShape m = multi_query_shape(group, n_q);
  a = DecodeArgs{};
  a.k = view_of(k);
  a.v = view_of(v);
  a.q = q;
  a.q_dtype = q_dtype;
  a.batch = k->batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = k->n_kv_heads;
  a.group = group;
  a.seq_lens = seq_lens;
  a.ctx_len = ctx_len;
  a.scale = scale;
  a.n_q = n_q;
  a.vgroups = m.vgroups;
  a.vg_size = m.vg_size;
  a.prefill = m.prefill ? 1 : 0;
  a.fplan = plan_multi(k->batch, k->n_kv_heads, m, ctx_len);
  a.out = out;
  a.lse = lse;
  char *ws = static_cast<char *>(workspace);
  a.counters = reinterpret_cast<unsigned *>(ws + w.counters);
  a.fpart_ml = reinterpret_cast<float2 *>(ws + w.fpart_ml);
  a.fpart_o = reinterpret_cast<float *>(ws + w.fpart_o);
  return decode_fused_supported(a) ? TQ_OK : TQ_ERR_UNSUPPORTED;
}


int tq_decode_attn_multi(const tq_cache *k, const tq_cache *v, const void *q, int q_dtype,
                         int n_q_heads, int n_q, const int32_t *seq_lens, int ctx_len, float scale,
                         float *out, float *lse, void *workspace, size_t workspace_bytes,
                         void *hip_stream) {
  DecodeArgs a{};
  const int st = setup_multi(k, v, q, q_dtype, n_q_heads, n_q, seq_lens, ctx_len, scale, out, lse, workspace,
                             workspace_bytes, a);
  if (st != TQ_OK) return st;
  return hip_status(launch_decode_fused(a, compute_units(), static_cast<hipStream_t>(hip_stream)));
}

int tq_decode_attn_multi_append(const tq_cache *k, const tq_cache *v, const void *xk, const void *xv, int x_dtype,
                                const void *q, int q_dtype, int n_q_heads, int n_q, const int32_t *seq_lens,
                                int ctx_len, float scale, float *out, float *lse, void *workspace,
                                size_t workspace_bytes, void *hip_stream) {
  if (xk == nullptr || xv == nullptr || !aligned(xk, 16) || !aligned(xv, 16) || !valid_dtype(x_dtype))
    return TQ_ERR_INVALID_ARG;
  DecodeArgs a{};
  const int st = setup_multi(k, v, q, q_dtype, n_q_heads, n_q, seq_lens, ctx_len, scale, out, lse, workspace,
                             workspace_bytes, a);
  if (st != TQ_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (n_q <= kMultiAppendMax && !a.prefill) {  // one launch: the new tokens written, then attended
    a.xk = xk;
    a.xv = xv;
    a.x_dtype = x_dtype;
    return hip_status(launch_decode_fused(a, compute_units(), stream));
  }
  // a prefill chunk or more than 8 positions: the append kernels, then the attention (one
  // common position for the chunk)
  if (seq_lens != nullptr || ctx_len < n_q) return TQ_ERR_UNSUPPORTED;
  const hipError_t e = n_q <= kSmallAppendMax
                           ? launch_append_small(a.k, a.v, k->batch, xk, xv, x_dtype, ctx_len - n_q, n_q, stream)
                           : launch_quantize_kv(a.k, a.v, k->batch, xk, xv, x_dtype, ctx_len - n_q, n_q, stream);
  if (e != hipSuccess) return TQ_ERR_HIP;
  return hip_status(launch_decode_fused(a, compute_units(), stream));
}

int tq_paged_quantize_append_kv(const tq_paged_cache *k, const tq_paged_cache *v, const void *xk,
                                const void *xv, int x_dtype, const int32_t *start_pos, int n_tokens,
                                void *hip_stream) {
  const int st = check_paged_pair(k, v);
  if (st != TQ_OK) return st;
  if (xk == nullptr || xv == nullptr || !aligned(xk, 16) || !aligned(xv, 16) || !valid_dtype(x_dtype))
    return TQ_ERR_INVALID_ARG;
  if (start_pos == nullptr || !aligned(start_pos, 4) || n_tokens < 0) return TQ_ERR_INVALID_ARG;
  if (n_tokens == 0) return TQ_OK;
  if (n_tokens > (1 << 24)) return TQ_ERR_UNSUPPORTED;
  return hip_status(launch_append_paged(view_of_pool(k), view_of_pool(v), k->block_table, k->max_pages, k->n_pages,
                                        k->batch, xk, xv, x_dtype, start_pos, n_tokens,
                                        static_cast<hipStream_t>(hip_stream)));
}

size_t tq_paged_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int max_ctx_len) {
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < n_kv_heads || n_q_heads % n_kv_heads != 0 || max_ctx_len < 0)
    return 0;
  return workspace_layout_paged(batch, n_q_heads, n_kv_heads, max_ctx_len).total;
}

static int paged_decode(const tq_paged_cache *k, const tq_paged_cache *v, const void *xk, const void *xv,
                        int x_dtype, const void *q, int q_dtype, int n_q_heads, const int32_t *seq_lens,
                        int max_ctx_len, float scale, float *out, float *lse, void *workspace,
                        size_t workspace_bytes, void *hip_stream) {
  const int st = check_paged_pair(k, v);
  if (st != TQ_OK) return st;
  if (k->signs != v->signs) return TQ_ERR_INVALID_ARG;
  if (q == nullptr || !aligned(q, 16) || !valid_dtype(q_dtype)) return TQ_ERR_INVALID_ARG;
  if (out == nullptr || !aligned(out, 16)) return TQ_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return TQ_ERR_INVALID_ARG;
  if (seq_lens == nullptr || !aligned(seq_lens, 4)) return TQ_ERR_INVALID_ARG;
  if (n_q_heads < 1 || n_q_heads % k->n_kv_heads != 0) return TQ_ERR_INVALID_ARG;
  const int group = n_q_heads / k->n_kv_heads;
  if (max_ctx_len < 0 || !std::isfinite(scale)) return TQ_ERR_INVALID_ARG;
  if ((long)max_ctx_len > (long)k->max_pages * k->page_tokens) return TQ_ERR_CAPACITY;
  if (group > 8 || (k->bits != 3 && k->bits != 4) || v->bits != 2) return TQ_ERR_UNSUPPORTED;
  const WorkspaceLayout w = workspace_layout_paged(k->batch, n_q_heads, k->n_kv_heads, max_ctx_len);
  if (workspace == nullptr || !aligned(workspace, 256)) return TQ_ERR_INVALID_ARG;
  if (workspace_bytes < w.total) return TQ_ERR_WORKSPACE;

  DecodeArgs a{};
  a.k = view_of_pool(k);
  a.v = view_of_pool(v);
  a.q = q;
  a.q_dtype = q_dtype;
  a.batch = k->batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = k->n_kv_heads;
  a.group = group;
  a.seq_lens = seq_lens;
  a.ctx_len = max_ctx_len;
  a.scale = scale;
  a.n_q = 1;
  a.vgroups = 1;
  a.vg_size = group;
  a.fplan = plan_fused_paged(k->batch, k->n_kv_heads, max_ctx_len);
  a.plan = a.fplan;
  a.out = out;
  a.lse = lse;
  char *ws = static_cast<char *>(workspace);
  a.counters = reinterpret_cast<unsigned *>(ws + w.counters);
  a.fpart_ml = reinterpret_cast<float2 *>(ws + w.fpart_ml);
  a.fpart_o = reinterpret_cast<float *>(ws + w.fpart_o);
  a.block_table = k->block_table;
  a.max_pages = k->max_pages;
  a.n_pages = k->n_pages;
  a.xk = xk;
  a.xv = xv;
  a.x_dtype = x_dtype;
  return hip_status(launch_decode_fused_paged(a, static_cast<hipStream_t>(hip_stream)));
}

int tq_paged_decode_attn(const tq_paged_cache *k, const tq_paged_cache *v, const void *q, int q_dtype,
                         int n_q_heads, const int32_t *seq_lens, int max_ctx_len, float scale, float *out,
                         float *lse, void *workspace, size_t workspace_bytes, void *hip_stream) {
  return paged_decode(k, v, nullptr, nullptr, TQ_BF16, q, q_dtype, n_q_heads, seq_lens, max_ctx_len, scale, out,
                      lse, workspace, workspace_bytes, hip_stream);
}

int tq_paged_decode_attn_append(const tq_paged_cache *k, const tq_paged_cache *v, const void *xk, const void *xv,
                                int x_dtype, const void *q, int q_dtype, int n_q_heads, const int32_t *seq_lens,
                                int max_ctx_len, float scale, float *out, float *lse, void *workspace,
                                size_t workspace_bytes, void *hip_stream) {
  if (xk == nullptr || xv == nullptr || !aligned(xk, 16) || !aligned(xv, 16) || !valid_dtype(x_dtype))
    return TQ_ERR_INVALID_ARG;
  return paged_decode(k, v, xk, xv, x_dtype, q, q_dtype, n_q_heads, seq_lens, max_ctx_len, scale, out, lse,
                      workspace, workspace_bytes, hip_stream);
}

size_t tq_paged_decode_ext_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int n_q, int max_ctx_len,
                                           float sparse_v_tau) {
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < n_kv_heads || n_q_heads % n_kv_heads != 0 || max_ctx_len < 0 ||
      n_q < 1 || n_q > kMaxQueryPositions || !(sparse_v_tau >= 0.f && sparse_v_tau < 1.f) ||
      (sparse_v_tau > 0.f && n_q != 1))
    return 0;
  return workspace_layout_paged_ext(batch, n_q_heads, n_kv_heads, n_q, max_ctx_len, sparse_v_tau > 0.f).total;
}

int tq_paged_decode_attn_ext(const tq_paged_cache *k, const tq_paged_cache *v, const void *q, int q_dtype,
                             int n_q_heads, int n_q, const int32_t *seq_lens, int max_ctx_len, float scale,
                             float sparse_v_tau, float *out, float *lse, void *workspace, size_t workspace_bytes,
                             void *hip_stream) {
  const int st = check_paged_pair(k, v);
  if (st != TQ_OK) return st;
  if (k->signs != v->signs) return TQ_ERR_INVALID_ARG;
  if (q == nullptr || !aligned(q, 16) || !valid_dtype(q_dtype)) return TQ_ERR_INVALID_ARG;
  if (out == nullptr || !aligned(out, 16)) return TQ_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return TQ_ERR_INVALID_ARG;
  if (seq_lens == nullptr || !aligned(seq_lens, 4)) return TQ_ERR_INVALID_ARG;
  if (n_q_heads < 1 || n_q_heads % k->n_kv_heads != 0) return TQ_ERR_INVALID_ARG;
  if (n_q < 1 || n_q > kMaxQueryPositions) return TQ_ERR_INVALID_ARG;
  if (max_ctx_len < 0 || !std::isfinite(scale)) return TQ_ERR_INVALID_ARG;
  if (!(sparse_v_tau >= 0.f && sparse_v_tau < 1.f)) return TQ_ERR_INVALID_ARG;
  if ((long)max_ctx_len > (long)k->max_pages * k->page_tokens) return TQ_ERR_CAPACITY;
  const int group = n_q_heads / k->n_kv_heads;
  const bool sparse = sparse_v_tau > 0.f;
  if (group > 8 || (k->bits != 3 && k->bits != 4) || v->bits != 2 || (sparse && n_q != 1)) return TQ_ERR_UNSUPPORTED;
  const WorkspaceLayout w = workspace_layout_paged_ext(k->batch, n_q_heads, k->n_kv_heads, n_q, max_ctx_len, sparse);
  if (workspace == nullptr || !aligned(workspace, 256)) return TQ_ERR_INVALID_ARG;
  if (workspace_bytes < w.total) return TQ_ERR_WORKSPACE;

  DecodeArgs a{};
  a.k = view_of_pool(k);
  a.v = view_of_pool(v);
  a.q = q;
  a.q_dtype = q_dtype;
  a.batch = k->batch;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = k->n_kv_heads;
  a.group = group;
  a.seq_lens = seq_lens;
  a.ctx_len = max_ctx_len;
  a.scale = scale;
  a.out = out;
  a.lse = lse;
  char *ws = static_cast<char *>(workspace);
  a.counters = reinterpret_cast<unsigned *>(ws + w.counters);
  a.fpart_ml = reinterpret_cast<float2 *>(ws + w.fpart_ml);
  a.fpart_o = reinterpret_cast<float *>(ws + w.fpart_o);
  a.block_table = k->block_table;
  a.max_pages = k->max_pages;
  a.n_pages = k->n_pages;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (!sparse) {
    const MultiQueryShape m = multi_query_shape(group, n_q);
    a.n_q = n_q;
    a.vgroups = m.vgroups;
    a.vg_size = m.vg_size;
    a.prefill = m.prefill ? 1 : 0;
    a.fplan = plan_paged_multi(k->batch, k->n_kv_heads, m, max_ctx_len);
    a.plan = a.fplan;
    return hip_status(launch_decode_fused_paged(a, stream));
  }
  // Sparse V: key pass (LSE partials and tile maxima), then the masked value pass
  a.n_q = 1;
  a.vgroups = 1;
  a.vg_size = group;
  a.sparse = 1;
  a.ln_tau = std::log(sparse_v_tau);
  a.fplan = plan_fused_paged(k->batch, k->n_kv_heads, max_ctx_len);
  a.plan = a.fplan;
  a.tile_max = reinterpret_cast<float *>(ws + w.tile_max);
  a.tile_stride = (max_ctx_len + 63) / 64;
  DecodeArgs vp = a;
  vp.sparse = 0;
  vp.lse_ml = a.fpart_ml;
  vp.lse_splits = a.fplan.n_splits;
  vp.fplan = plan_fused_vmask(k->batch, k->n_kv_heads, max_ctx_len);
  vp.plan = vp.fplan;
  vp.fpart_ml = reinterpret_cast<float2 *>(ws + w.vpart_ml);
  vp.fpart_o = reinterpret_cast<float *>(ws + w.vpart_o);
  return hip_status(launch_decode_fused_paged_sparse(a, vp, stream));
}

size_t tq_ip_search_workspace_bytes(int n_queries, int n_vectors, int top_k) {
  if (!search_shape_ok(n_queries, n_vectors, top_k)) return 0;
  return search_layout(n_queries, n_vectors, top_k).total;
}

int tq_ip_search(const tq_cache *db, const void *q, int q_dtype, int n_queries, int n_vectors, int top_k,
                 int32_t *out_idx, float *out_score, void *workspace, size_t workspace_bytes, void *hip_stream) {
  const int st = check_cache(db);
  if (st != TQ_OK) return st;
  if (q == nullptr || !aligned(q, 16) || !valid_dtype(q_dtype)) return TQ_ERR_INVALID_ARG;
  if (out_idx == nullptr || out_score == nullptr || !aligned(out_idx, 4) || !aligned(out_score, 4))
    return TQ_ERR_INVALID_ARG;
  if (n_queries < 1 || n_vectors < 1 || top_k < 1) return TQ_ERR_INVALID_ARG;
  if (db->batch != 1 || db->n_kv_heads != 1 || db->layout != TQ_LAYOUT_ROWS || (db->bits != 3 && db->bits != 4))
    return TQ_ERR_UNSUPPORTED;
  if (n_vectors > db->capacity) return TQ_ERR_CAPACITY;
  if (!search_shape_ok(n_queries, n_vectors, top_k)) return TQ_ERR_UNSUPPORTED;
  const SearchLayout w = search_layout(n_queries, n_vectors, top_k);
  if (workspace == nullptr || !aligned(workspace, 256)) return TQ_ERR_INVALID_ARG;
  if (workspace_bytes < w.total) return TQ_ERR_WORKSPACE;
  char *ws = static_cast<char *>(workspace);
  const SearchState state{reinterpret_cast<uint64_t *>(ws + w.cand), reinterpret_cast<uint2 *>(ws + w.bnd)};
  return hip_status(launch_ip_search(view_of(db), q, q_dtype, n_queries, n_vectors, top_k, out_idx, out_score, state,
                                     static_cast<hipStream_t>(hip_stream)));
}

}  // extern "C"

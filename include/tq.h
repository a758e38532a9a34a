/*
 * tq.h - C ABI of the TurboQuant compressed-KV library for AMD Instinct MI355X (gfx950).
 *
 * Two halves of one data-parallel hot path:
 *   - quantize: every K or V head vector x (d = 128) is rotated by a random-sign
 *     Walsh-Hadamard transform R = H diag(s) / sqrt(d), its L2 norm is split off and
 *     stored as fp16, and each coordinate of the unit direction u = R x / ||x|| is
 *     mapped to the nearest entry of a data-independent Lloyd-Max codebook of
 *     2^bits levels; the codes are bit-packed.
 *   - decode attention: one query per (batch, query head) is scored directly
 *     against the packed keys in the rotated domain,
 *         s_t = scale * ||k_t|| * (R q) . c_K[idx_t],
 *     followed by a softmax, optional Sparse-V row skipping, accumulation of
 *     p_t * ||v_t|| * c_V[idx_v_t] in the rotated domain and one inverse rotation.
 *
 * Source pages (cited by title and section):
 *   [inferrs]  "inferrs & TurboQuant：本地 LLM 推理的内存革命" - §核心技术 (Walsh-Hadamard
 *              rotation before quantization), table §压缩格式对比 (2/3/4-bit formats),
 *              §三个反直觉的关键发现 (K/V asymmetry, boundary layers), §Sparse V (skip the
 *              decode of V positions with low attention weight).
 *   [tq-80]    "TurboQuant：让大模型本地推理内存占用降低80%的KV缓存压缩技术" - §核心创新
 *              (random orthogonal rotation, Beta-distributed coordinates, precomputed
 *              Lloyd-Max codebooks, norm kept as fp16), §tqai项目 (bits_k / bits_v),
 *              §配置策略与质量权衡 (K4/V2, K3/V2, K4/V3).
 *   [tq-plus]  "TurboQuant+：跨平台KV缓存压缩技术助力本地LLM高效推理" - §KV缓存的作用与开销
 *              (cache size = 2 * layers * heads * head_dim * length * bytes).
 *   [tq-fwht]  "TurboQuant：用Rust核心与FWHT预处理实现LLM推理的4-bit KV缓存量化" - §2 FWHT
 *              (orthogonal, exactly invertible transform before 4-bit quantization).
 *   [google]   "Google 最新極限壓縮算法，砸碎大模型本地部署的內存墻，8 倍提升！" - the list of
 *              mlx-vlm kernels (score against quantized keys, pack / unpack low-bit codes,
 *              multi-head weighted sum in the rotated domain) and the 4-bit-key speed-up.
 *
 * Conventions shared by every call:
 *   - Status: 0 = TQ_OK, negative = error (enum tq_status).  Nothing throws across
 *     the ABI.  All argument validation happens before any HIP call, so invalid
 *     arguments are reported without touching the GPU.
 *   - Memory: every buffer is allocated and owned by the caller.  Pointers named
 *     "device" must be device memory of the current HIP device.  The library keeps
 *     no global state and allocates nothing.
 *   - Asynchrony: device work is enqueued on `hip_stream` (a hipStream_t, NULL =
 *     the null stream) and the call returns without waiting.  Only launch errors
 *     are returned (TQ_ERR_HIP); faults surface at the caller's next sync.
 *   - Head dim d must be 128.  Code widths: bits in {2, 3, 4, 8}.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum tq_status {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1, /* null or misaligned pointer, negative size, bad enum, NaN */
  TQ_ERR_UNSUPPORTED = -2, /* valid in principle but not implemented (d != 128, bits, group) */
  TQ_ERR_CAPACITY = -3,    /* token range or context longer than the cache capacity */
  TQ_ERR_WORKSPACE = -4,   /* workspace smaller than tq_decode_workspace_bytes() */
  TQ_ERR_HIP = -5          /* a HIP launch failed */
};

enum tq_dtype { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 };

/* Packed-code layouts inside one (batch, kv head) plane of `capacity` tokens.
 * Bit k of the code of (token t, rotated coordinate i) sits at bit offset
 *   TQ_LAYOUT_ROWS:   t*d*bits + i*bits + k
 *   TQ_LAYOUT_GROUP8: (t/8)*d*8*bits + (i*8 + t%8)*bits + k
 * of the plane, byte = offset >> 3, bit within byte = offset & 7 (LSB first).
 * ROWS keeps one vector's codes in one d*bits/8-byte row (how the keys are read);
 * GROUP8 puts the codes of 8 consecutive tokens for one coordinate next to each
 * other (how the values are read when they are summed over tokens).  Both use
 * exactly d*bits/8 bytes per vector.  Decode attention needs K in ROWS and V in
 * GROUP8; quantize and dequantize accept either. */
enum tq_layout { TQ_LAYOUT_ROWS = 0, TQ_LAYOUT_GROUP8 = 1 };

/* One K or V cache of one layer.  Every pointer is device memory owned by the caller.
 *   codes       [batch][n_kv_heads][capacity * d * bits / 8] bytes, 16-byte aligned
 *   norms       [batch][n_kv_heads][capacity] IEEE fp16 bit patterns, 16-byte aligned
 *   centroids   [1 << bits] fp32, ascending (from tq_make_codebook_table)
 *   boundaries  [(1 << bits) - 1] fp32 midpoints (from tq_make_codebook_table); the
 *               kernels rely on the symmetry that table has: boundaries[L-2-j] =
 *               -boundaries[j] and boundaries[L/2-1] = 0 (L = 1 << bits)
 *   signs       [d] int8, each +1 or -1, 16-byte aligned: the diagonal of the rotation
 *               (shared by the K and V caches of a layer)
 *   table_scale 0 (none), or a factor s in [1, 2] that the matrix-core decode kernels apply
 *               to the value centroids of their fp16 operand table and take off the output
 *               again; tq_value_table_scale() gives one for which a 4-level codebook is held
 *               almost exactly in fp16 (about 1e-6 relative instead of 2^-12).  Only a value
 *               cache's is read.  Results do not depend on it beyond that rounding.
 * capacity must be a positive multiple of 64. */
typedef struct tq_cache {
  int32_t d;
  int32_t bits;
  int32_t layout;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t capacity;
  uint8_t *codes;
  uint16_t *norms;
  const float *centroids;
  const float *boundaries;
  const int8_t *signs;
  float table_scale;
} tq_cache;

/* The QJL sign sketch that accompanies a key cache in the residual variant ([google] §第二步：
 * QJL —— 1 bit 清理殘差: one bit per sketch row of a Johnson-Lindenstrauss projection of the
 * first stage's error removes the bias of inner products, i.e. of attention scores).  For the
 * key at (b, h, t) with codes idx, stored norm n16 and r = R x - n16 c[idx] (rotated domain):
 *   bits       device [batch][n_kv_heads][capacity][m / 8] bytes, 16-byte aligned; bit j (LSB
 *              first) of a row is 1 iff (S r)_j >= 0
 *   res_norms  device [batch][n_kv_heads][capacity] fp16 bit patterns of ||r||, 2-byte aligned
 *   proj       device [m][d] fp32: the Gaussian matrix S, i.i.d. N(0, 1) entries drawn by the
 *              caller (the library has no random generator), 16-byte aligned
 *   m          sketch rows; m must equal d (128): one bit per coordinate
 * The key cache itself (tq_cache, ROWS layout) holds the first stage's codes and norms; with
 * bits = b - 1 the key costs b bits per coordinate plus two fp16 norms. */
typedef struct tq_qjl_sketch {
  int32_t m;
  uint8_t *bits;
  uint16_t *res_norms;
  const float *proj;
} tq_qjl_sketch;

/* Lloyd-Max codebook for the marginal density of one coordinate of a random unit
 * vector in R^d, f(x) proportional to (1 - x^2)^((d-3)/2) on [-1, 1] ([tq-80] §核心创新:
 * rotated coordinates are Beta distributed; the codebook is data-independent and
 * precomputed).  Host-only, no GPU: computed in fp64 (Lloyd iterations refined by
 * Newton steps on the Lloyd fixed point), symmetrised, rounded to fp32.
 *   centroids   host out [1 << bits], ascending
 *   boundaries  host out [(1 << bits) - 1], midpoints of adjacent centroids
 * Errors: TQ_ERR_INVALID_ARG (null pointer, d < 4), TQ_ERR_UNSUPPORTED (bits outside 1..8). */
int tq_make_codebook_table(int d, int bits, float *centroids, float *boundaries);

/* Host only: the table_scale for a cache with these centroids (host memory, n_levels of
 * them).  For a symmetric 4-level codebook {-b, -a, a, b}: with p/q the best convergent of the
 * continued fraction of b/a whose p is below 2048, s = q 2^j / a in [1, 2), so that s a = q 2^j
 * and s b = p 2^j up to that convergent's error are both fp16 values.  1 for any other
 * codebook (no scale).  Never fails. */
float tq_value_table_scale(const float *centroids, int n_levels);

/* Quantize n_tokens new tokens of every (batch, kv head) into cache positions
 * [start_pos, start_pos + n_tokens) ([tq-80] §核心创新; [inferrs] §核心技术):
 *   n = ||x||_2 (fp32), norm stored as fp16 (round to nearest even),
 *   u = R x / n (u = 0 for a zero vector), code = #{ j : boundaries[j] < u_i },
 *   codes packed in the cache's layout.
 *   x      device in [batch][n_tokens][n_kv_heads][d] of x_dtype (TQ_F32/TQ_BF16/TQ_F16),
 *          16-byte aligned
 * Positions outside the range are left untouched (a GROUP8 cache is read-modified-
 * written at the edges of the range).  Calls that overlap on one cache race.
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY
 * (start_pos < 0 or start_pos + n_tokens > capacity), TQ_ERR_HIP. */
int tq_quantize_append(const tq_cache *c, const void *x, int x_dtype, int start_pos,
                       int n_tokens, void *hip_stream);

/* tq_quantize_append on a key cache and a value cache of one layer in a single launch
 * (same operation and references as tq_quantize_append, applied to both).
 *   k          cache in TQ_LAYOUT_ROWS;  v  cache in TQ_LAYOUT_GROUP8; they must agree on
 *              batch, n_kv_heads and capacity (bits, codebooks and signs may differ)
 *   xk, xv     device in [batch][n_tokens][n_kv_heads][d] of x_dtype, 16-byte aligned
 * Results are bit-identical to two tq_quantize_append calls.  Calls that overlap on one
 * cache race.
 * Errors: TQ_ERR_INVALID_ARG (also for other layouts or mismatched shapes),
 * TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_HIP. */
int tq_quantize_append_kv(const tq_cache *k, const tq_cache *v, const void *xk, const void *xv,
                          int x_dtype, int start_pos, int n_tokens, void *hip_stream);

/* Decode attention against the packed cache, one query per (batch, query head).
 * Query head h reads kv head h / (n_q_heads / n_kv_heads).  For each (b, h) with
 * T = seq_lens ? clamp(seq_lens[b], 0, ctx_len) : ctx_len tokens:
 *   s_t  = scale * ||k_t||_fp16 * (R q) . c_K[idx_t]                    ([google] score kernel)
 *   LSE  = log sum_t exp(s_t),  p_t = exp(s_t - LSE)
 *   o    = R^T sum_t keep_t p_t ||v_t||_fp16 c_V[idx_v_t]                 ([google] weighted
 *                                                                        rotated sum; [tq-fwht] §2)
 * with keep_t = 1 when sparse_v_tau == 0 and keep_t = (p_t >= sparse_v_tau) otherwise
 * ([inferrs] §Sparse V; no renormalisation, o = 0 when every row is dropped).
 *   k, v       caches of one layer; k in TQ_LAYOUT_ROWS, v in TQ_LAYOUT_GROUP8; they must
 *              agree on d, batch, n_kv_heads, capacity and signs (bits may differ)
 *   q          device in [batch][n_q_heads][d] of q_dtype, 16-byte aligned
 *   n_q_heads  a multiple of n_kv_heads with n_q_heads / n_kv_heads <= 16
 *   seq_lens   device int32 [batch] or NULL
 *   ctx_len    0 <= ctx_len <= capacity
 *   scale      finite softmax scale (1/sqrt(d) in the usual case)
 *   sparse_v_tau  0 (dense) or a threshold in (0, 1)
 *   out        device out [batch][n_q_heads][d] fp32, 16-byte aligned
 *   lse        device out [batch][n_q_heads] fp32 or NULL (-inf when T = 0)
 *   scores     device out [batch][n_q_heads][ctx_len] fp32 or NULL (s_t; -inf past T)
 *   workspace  device scratch of at least tq_decode_workspace_bytes(...) bytes,
 *              256-byte aligned, owned by the caller.  Zero-fill it once before the first
 *              call that uses it: it holds per-(batch, kv head) arrival counters that every
 *              completed call leaves at zero again.  Calls that share one workspace must not
 *              overlap in time (same stream, or ordered by events).
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
int tq_decode_attn(const tq_cache *k, const tq_cache *v, const void *q, int q_dtype,
                   int n_q_heads, const int32_t *seq_lens, int ctx_len, float scale,
                   float sparse_v_tau, float *out, float *lse, float *scores, void *workspace,
                   size_t workspace_bytes, void *hip_stream);

/* QJL residual variant, quantize: as tq_quantize_append into the key cache k (ROWS layout), and
 * for each token the sign sketch of its residual and the residual's norm into s ([google]
 * §第二步：QJL; [tq-80] §技术背景与学术渊源):
 *   r = R x - n16 c[idx] (rotated domain, n16 the stored fp16 norm), ||r|| -> fp16 (nearest
 *   even), bit j = ((S r)_j >= 0) with (S r)_j summed in fp32.
 * A sign bit equals the one computed in exact arithmetic except where |(S r)_j| is within
 * about 1e-5 ||S_j|| ||r|| of zero (fp32 rounding).  Positions outside the range are kept.
 * Errors: TQ_ERR_INVALID_ARG (also for a GROUP8 key cache), TQ_ERR_UNSUPPORTED (m != d),
 * TQ_ERR_CAPACITY, TQ_ERR_HIP. */
int tq_qjl_quantize_append(const tq_cache *k, const tq_qjl_sketch *s, const void *x, int x_dtype,
                           int start_pos, int n_tokens, void *hip_stream);

/* QJL residual variant, keys and values of one step: tq_qjl_quantize_append(k, s, xk, ...) and
 * tq_quantize_append(v, xv, ...) over the same positions, with the same results, in one launch
 * for up to 8 tokens (a decode step; two launches for longer ranges).
 *   k, s       the key cache (ROWS) and its sketch, as for tq_qjl_quantize_append
 *   v          the value cache (GROUP8), same batch, n_kv_heads and capacity as k
 *   xk, xv     device in [batch][n_tokens][n_kv_heads][d] of x_dtype, 16-byte aligned
 * Errors: TQ_ERR_INVALID_ARG (also for other layouts or mismatched caches), TQ_ERR_UNSUPPORTED,
 * TQ_ERR_CAPACITY, TQ_ERR_HIP. */
int tq_qjl_quantize_append_kv(const tq_cache *k, const tq_qjl_sketch *s, const tq_cache *v, const void *xk,
                              const void *xv, int x_dtype, int start_pos, int n_tokens, void *hip_stream);

/* QJL residual variant, decode attention: tq_decode_attn with every score corrected by the key's
 * sign sketch ([google] _prod_score_kernel: the score against the codes plus the QJL term),
 *   s_t = scale ( ||k_t||_fp16 (R q) . c_K[idx_t]
 *                 + sqrt(pi/2) / m ||r_t||_fp16 (S R q) . (2 bits_t - 1) ),
 * an unbiased estimate of scale q . k_t over the draw of S, followed by the same softmax,
 * Sparse V, value sum and inverse rotation.  Arguments as tq_decode_attn plus ks, the sketch of
 * the keys in k; the workspace is tq_decode_workspace_bytes(...).  Keys of 3 bits, values of 2
 * bits and groups up to 8 run on matrix cores (the query's sketch S R q and the sign products
 * as fp16 matrix operands, the signs exact as +/-1): one launch, or with Sparse V the key pass
 * and the masked value pass; any other widths and groups up to 16 take the fp32 vector
 * kernels.
 * Errors: as tq_decode_attn, and TQ_ERR_INVALID_ARG / TQ_ERR_UNSUPPORTED for the sketch. */
int tq_qjl_decode_attn(const tq_cache *k, const tq_qjl_sketch *ks, const tq_cache *v, const void *q,
                       int q_dtype, int n_q_heads, const int32_t *seq_lens, int ctx_len, float scale,
                       float sparse_v_tau, float *out, float *lse, float *scores, void *workspace,
                       size_t workspace_bytes, void *hip_stream);

/* Workspace bytes tq_decode_attn needs for this problem (0 for invalid arguments). */
size_t tq_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int ctx_len,
                                 float sparse_v_tau);

/* Append and attend in one call: for every sequence b with T = seq_lens ? clamp(seq_lens[b], 0,
 * ctx_len) : ctx_len >= 1, quantize its new key xk[b] and value xv[b] into position T - 1 of
 * the caches (as tq_quantize_append_kv with start_pos = T - 1, n_tokens = 1), then dense
 * decode attention exactly as tq_decode_attn with sparse_v_tau = 0 and no scores.  One launch
 * for keys of 3/4 bits, values of 2 bits and n_q_heads / n_kv_heads <= 8 (the wave that
 * reads position T - 1 writes the token first); otherwise the append kernel and then the
 * decode call, which needs seq_lens == NULL (TQ_ERR_UNSUPPORTED otherwise).
 *   xk, xv     device in [batch][1][n_kv_heads][d] of x_dtype, 16-byte aligned
 *   the other arguments as for tq_decode_attn; workspace of tq_decode_workspace_bytes(..., 0)
 * A decode step needs this one launch instead of two.  The new token's codes follow the
 * same rule as the append kernels (equal to the oracle's except within 1e-6 of a boundary).
 * The arithmetic is that of the append path for up to 8 tokens; the chunked path for longer
 * appends evaluates the fp32 rotation in another order, so a code within that band can
 * differ from it.
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
int tq_decode_attn_append(const tq_cache *k, const tq_cache *v, const void *xk, const void *xv,
                          int x_dtype, const void *q, int q_dtype, int n_q_heads,
                          const int32_t *seq_lens, int ctx_len, float scale, float *out, float *lse,
                          void *workspace, size_t workspace_bytes, void *hip_stream);

/* Append and attend with Sparse V ([inferrs] §Sparse V): as tq_decode_attn_append, then decode
 * attention exactly as tq_decode_attn at sparse_v_tau (no scores).  sparse_v_tau = 0 is
 * tq_decode_attn_append.  For tau in (0, 1) with keys of 3/4 bits, values of 2 bits and
 * n_q_heads / n_kv_heads <= 8, the new token goes in with Sparse V's first pass (the wave that
 * reads position T - 1 writes the key and value first), so the step is the key pass and the
 * masked value pass, two launches; otherwise the append kernel and the decode call, which
 * needs seq_lens == NULL (TQ_ERR_UNSUPPORTED otherwise).
 *   sparse_v_tau  0 or a threshold in (0, 1)
 *   workspace     tq_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, ctx_len, sparse_v_tau)
 *   the other arguments as for tq_decode_attn_append
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
int tq_decode_attn_append_sparse(const tq_cache *k, const tq_cache *v, const void *xk, const void *xv, int x_dtype,
                                 const void *q, int q_dtype, int n_q_heads, const int32_t *seq_lens, int ctx_len,
                                 float scale, float sparse_v_tau, float *out, float *lse, void *workspace,
                                 size_t workspace_bytes, void *hip_stream);

/* tq_decode_attn_append for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same one-launch decode
 * step with the same arguments and results, except that there is no workspace argument.  Its
 * scratch (arrival counters and per-split partials) is a static device array of the library,
 * 8 MiB per GPU, kept until the process ends; the first call on a GPU clears its counter
 * region with a kernel on hip_stream and every completed call leaves it at zero.  The call
 * allocates nothing.
 *   Limits: keys of 3 or 4 bits, values of 2 bits, n_q_heads / n_kv_heads <= 8 (the one-launch
 *   path; TQ_ERR_UNSUPPORTED otherwise); batch * n_kv_heads <= 16384 and
 *   batch * n_q_heads * splits * 520 bytes of partials within the rest of the 8 MiB
 *   (TQ_ERR_WORKSPACE otherwise; splits is about 256 / (batch * n_kv_heads), at least 1).
 *   Every call on one GPU uses the same scratch: calls that overlap in time on one GPU race,
 *   so order them (one stream, or events).
 * Errors: as tq_decode_attn_append, and TQ_ERR_HIP if the scratch cannot be located. */
int tq_decode_attn_append_noalloc(const tq_cache *k, const tq_cache *v, const void *xk, const void *xv,
                                  int x_dtype, const void *q, int q_dtype, int n_q_heads,
                                  const int32_t *seq_lens, int ctx_len, float scale, float *out, float *lse,
                                  void *hip_stream);

/* Attention of n_q new query positions per sequence against the packed cache, which already
 * holds them (speculative verification of draft tokens, chunked prefill): the same scores,
 * softmax and rotated-domain value sum as tq_decode_attn ([google] score kernel; [inferrs]
 * on prefill speed), causal over positions.  With T = seq_lens ? clamp(seq_lens[b], 0,
 * ctx_len) : ctx_len cached tokens, query i (0 <= i < n_q) of sequence b sits at position
 * T - n_q + i and attends to positions 0 .. T - n_q + i; a query with no such position gets
 * o = 0 and LSE = -inf.  Dense only (no Sparse V), no score output.
 *   k, v       as for tq_decode_attn; keys of 3 or 4 bits and values of 2 bits
 *              (TQ_ERR_UNSUPPORTED otherwise)
 *   q          device in [batch][n_q][n_q_heads][d] of q_dtype, 16-byte aligned
 *   n_q        1 <= n_q <= 4096 (n_q = 1 is tq_decode_attn with sparse_v_tau = 0)
 *   out        device out [batch][n_q][n_q_heads][d] fp32, 16-byte aligned
 *   lse        device out [batch][n_q][n_q_heads] fp32 or NULL
 *   workspace  device scratch of at least tq_decode_attn_multi_workspace_bytes(...) bytes,
 *              256-byte aligned, zero-filled once before first use (arrival counters that
 *              every completed call returns to zero); calls sharing it must not overlap.
 * The n_q * (n_q_heads / n_kv_heads) query rows of a kv head are processed up to 8 at a
 * time, each group of rows reading the kv head's cache once.
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
int tq_decode_attn_multi(const tq_cache *k, const tq_cache *v, const void *q, int q_dtype,
                         int n_q_heads, int n_q, const int32_t *seq_lens, int ctx_len, float scale,
                         float *out, float *lse, void *workspace, size_t workspace_bytes,
                         void *hip_stream);

/* Append and attend for several positions (speculative verification: the draft's tokens): the n_q
 * new keys and values of each sequence, xk, xv [batch][n_q][n_kv_heads][d] of x_dtype, are
 * quantized into positions T_b - n_q .. T_b - 1 (those >= 0; T_b as for tq_decode_attn_multi),
 * then tq_decode_attn_multi runs over the result.  Up to 8 positions (outside the prefill mode)
 * take one launch: in every work item whose split holds new tokens, they are quantized side by
 * side (token j by wave j mod the item's wave count), key rows and norms stored whole and each
 * token's value fields replaced by compare-and-swap, all before the item reads its tiles; the
 * codes follow the same rule as the append kernels.  Longer chunks take the append kernels and
 * then the attention, which needs seq_lens == NULL and n_q <= ctx_len (TQ_ERR_UNSUPPORTED
 * otherwise).  The caches are written in place: calls that overlap on the same caches race.
 *   the other arguments as for tq_decode_attn_multi (workspace of
 *   tq_decode_attn_multi_workspace_bytes)
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
int tq_decode_attn_multi_append(const tq_cache *k, const tq_cache *v, const void *xk, const void *xv, int x_dtype,
                                const void *q, int q_dtype, int n_q_heads, int n_q, const int32_t *seq_lens,
                                int ctx_len, float scale, float *out, float *lse, void *workspace,
                                size_t workspace_bytes, void *hip_stream);

/* Workspace bytes tq_decode_attn_multi needs for this problem (0 for invalid arguments). */
size_t tq_decode_attn_multi_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int n_q,
                                            int ctx_len);

/* A paged K or V cache of one layer, the block-table layout of serving engines: the tokens
 * of every sequence live in fixed-size pages of one shared pool, position t of sequence b
 * in pool page block_table[b][t / page_tokens] at slot t % page_tokens.  A page holds
 * page_tokens consecutive positions of every kv head; within one (page, kv head) the codes
 * follow `layout` exactly as a tq_cache plane of capacity page_tokens does.
 *   codes        [n_pages][n_kv_heads][page_tokens * d * bits / 8] bytes, 16-byte aligned
 *   norms        [n_pages][n_kv_heads][page_tokens] fp16 bit patterns, 16-byte aligned
 *   block_table  device int32 [batch][max_pages], 4-byte aligned; an entry outside
 *                [0, n_pages) means "no page": those positions are not part of the sequence
 *                ([inferrs] §二: tokens live only in allocated pages).  Appends skip them and
 *                decode leaves them out of the softmax (no score, no value; nothing is read
 *                outside the pool); a sequence with no position on a page gets o = 0 and
 *                LSE = -inf
 *   centroids, boundaries, signs, table_scale as for tq_cache.
 * page_tokens: a positive multiple of 64.  The pool's code bytes must stay below 3 GiB
 * (32-bit offsets inside the decode kernel).  The K and V caches of a layer share one
 * block table. */
typedef struct tq_paged_cache {
  int32_t d;
  int32_t bits;
  int32_t layout;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t page_tokens;
  int32_t n_pages;
  int32_t max_pages;
  uint8_t *codes;
  uint16_t *norms;
  const int32_t *block_table;
  const float *centroids;
  const float *boundaries;
  const int8_t *signs;
  float table_scale;
} tq_paged_cache;

/* Quantize n_tokens new tokens of every sequence into a paged key cache (ROWS) and value
 * cache (GROUP8): token j of sequence b goes to position start_pos[b] + j, with the same
 * steps and codes rule as tq_quantize_append ([tq-80] §核心创新; [inferrs] §核心技术).
 * Positions below 0, at or past max_pages * page_tokens, or on a "no page" entry are
 * skipped.  Other positions are left untouched (a value group of 8 tokens is
 * read-modified-written).  Calls that overlap on one pool race, and so do sequences whose
 * tables share a page at the same positions.
 *   xk, xv     device in [batch][n_tokens][n_kv_heads][d] of x_dtype, 16-byte aligned
 *   start_pos  device int32 [batch], 4-byte aligned
 * Errors: TQ_ERR_INVALID_ARG (also for mismatched caches or layouts), TQ_ERR_UNSUPPORTED,
 * TQ_ERR_HIP. */
int tq_paged_quantize_append_kv(const tq_paged_cache *k, const tq_paged_cache *v, const void *xk,
                                const void *xv, int x_dtype, const int32_t *start_pos, int n_tokens,
                                void *hip_stream);

/* Dense decode attention over paged caches: as tq_decode_attn with sparse_v_tau = 0 and no
 * scores, sequence b attending over positions 0 .. T_b - 1, T_b = clamp(seq_lens[b], 0,
 * max_ctx_len), its pages found through the block table.  Keys of 3 or 4 bits (ROWS),
 * values of 2 bits (GROUP8), n_q_heads / n_kv_heads <= 8; otherwise TQ_ERR_UNSUPPORTED.
 * Positions on a "no page" entry below T_b are left out of the softmax (see
 * tq_paged_cache).  Same kernel and arithmetic as the contiguous call: a sequence whose
 * positions 0 .. T_b - 1 all lie on pages gets the output the contiguous call gives for
 * equal codes, bit for bit.
 *   seq_lens     device int32 [batch] (required)
 *   max_ctx_len  upper bound of the lengths, <= max_pages * page_tokens (TQ_ERR_CAPACITY)
 *   out, lse     as for tq_decode_attn
 *   workspace    device scratch of tq_paged_decode_workspace_bytes(...) bytes, 256-byte
 *                aligned, zero-filled once before first use (arrival counters, left at zero
 *                by every completed call); calls sharing it must not overlap in time.
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
int tq_paged_decode_attn(const tq_paged_cache *k, const tq_paged_cache *v, const void *q, int q_dtype,
                         int n_q_heads, const int32_t *seq_lens, int max_ctx_len, float scale, float *out,
                         float *lse, void *workspace, size_t workspace_bytes, void *hip_stream);

/* A paged decode step in one call: the new key and value of every sequence b with
 * T_b = clamp(seq_lens[b], 0, max_ctx_len) >= 1 are quantized into position T_b - 1 (as
 * tq_paged_quantize_append_kv with start_pos = T_b - 1, n_tokens = 1, skipped where the
 * table has no page), then tq_paged_decode_attn runs over positions 0 .. T_b - 1.  One
 * launch: the wave that reads position T_b - 1 writes it first (as tq_decode_attn_append).
 *   xk, xv  device in [batch][1][n_kv_heads][d] of x_dtype, 16-byte aligned
 *   the other arguments as for tq_paged_decode_attn.
 * Errors: as tq_paged_decode_attn. */
int tq_paged_decode_attn_append(const tq_paged_cache *k, const tq_paged_cache *v, const void *xk, const void *xv,
                                int x_dtype, const void *q, int q_dtype, int n_q_heads, const int32_t *seq_lens,
                                int max_ctx_len, float scale, float *out, float *lse, void *workspace,
                                size_t workspace_bytes, void *hip_stream);

/* Paged caches, several query positions or Sparse V: tq_paged_decode_attn extended as
 *   n_q > 1 (sparse_v_tau = 0): the attention of tq_decode_attn_multi ([google] score kernel;
 *     [inferrs] on prefill speed) over paged caches: with T_b = clamp(seq_lens[b], 0,
 *     max_ctx_len), query i of sequence b sits at position T_b - n_q + i and attends causally;
 *     q [batch][n_q][n_q_heads][d], out [batch][n_q][n_q_heads][d], lse [batch][n_q][n_q_heads];
 *   n_q = 1, sparse_v_tau in (0, 1): the Sparse V rule of tq_decode_attn ([inferrs] §Sparse V;
 *     keep_t = exp(s_t - LSE) >= tau, no renormalisation) over paged caches;
 *   n_q = 1, sparse_v_tau = 0: tq_paged_decode_attn.
 * Positions on a "no page" entry leave the softmax (see tq_paged_cache).  Keys of 3 or 4 bits,
 * values of 2 bits, n_q_heads / n_kv_heads <= 8, 1 <= n_q <= 4096; Sparse V with n_q = 1 only
 * (TQ_ERR_UNSUPPORTED otherwise).  A chunk of 8 or more groups of 8 query rows per kv head
 * runs in prefill mode, as without pages: the 8 waves of a workgroup take 8 row groups and
 * walk the same tiles, in splits of at most 4096 tokens (one page offset per lane).  Equal
 * codes give the outputs of the contiguous calls, bit for bit, for sequences without holes
 * wherever both calls split the context alike (always up to 4096 tokens).
 *   workspace  tq_paged_decode_ext_workspace_bytes(...) bytes, 256-byte aligned, zero-filled once
 *              before first use (arrival counters every completed call leaves at zero); calls
 *              sharing it must not overlap in time.
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
int tq_paged_decode_attn_ext(const tq_paged_cache *k, const tq_paged_cache *v, const void *q, int q_dtype,
                             int n_q_heads, int n_q, const int32_t *seq_lens, int max_ctx_len, float scale,
                             float sparse_v_tau, float *out, float *lse, void *workspace, size_t workspace_bytes,
                             void *hip_stream);

/* Workspace bytes tq_paged_decode_attn_ext needs (0 for invalid arguments). */
size_t tq_paged_decode_ext_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int n_q, int max_ctx_len,
                                           float sparse_v_tau);

/* Approximate inner-product nearest-neighbour search with the same quantizer ([tq-80]
 * §技术背景与学术渊源): the database is plane (batch 0, kv head 0) of `db` (batch = 1,
 * n_kv_heads = 1, ROWS layout, 3- or 4-bit codes, vectors 0 .. n_vectors - 1 quantized by
 * tq_quantize_append).  For query j the score of vector t is the inner product with its
 * dequantized vector, s = q_j . x_hat_t = n16_t (R q_j) . c[idx_t]; the result is the top_k
 * indices of largest score, descending, equal scores by ascending index, with their scores
 * (fp32, as the decode kernels compute them: within 1e-3 relative of the exact value).
 *   q          device in [n_queries][d] of q_dtype
 *   out_idx    device out int32 [n_queries][top_k] (-1 past n_vectors)
 *   out_score  device out fp32 [n_queries][top_k] (-inf past n_vectors)
 *   workspace  device scratch of tq_ip_search_workspace_bytes(...) bytes, 256-byte aligned
 *              (per-block candidates; no initial contents needed).  A workspace sized for
 *              (n_queries, n_vectors, top_k) serves any smaller call.
 * Two launches on hip_stream: each workgroup scores 1024 vectors for up to 8 queries and keeps
 * each query's k best; then one workgroup per query ranks the candidates that reach the
 * largest block k-th best.
 * 1 <= top_k <= 64, else TQ_ERR_UNSUPPORTED.
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
int tq_ip_search(const tq_cache *db, const void *q, int q_dtype, int n_queries, int n_vectors, int top_k,
                 int32_t *out_idx, float *out_score, void *workspace, size_t workspace_bytes, void *hip_stream);

/* Workspace bytes tq_ip_search needs (0 for invalid arguments). */
size_t tq_ip_search_workspace_bytes(int n_queries, int n_vectors, int top_k);

/* Workspace bytes tq_paged_decode_attn needs (0 for invalid arguments). */
size_t tq_paged_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int max_ctx_len);

/* Reconstruct x_hat = ||x||_fp16 * R^T c[idx] for cache positions
 * [start_pos, start_pos + n_tokens) ([google] unpack kernel; [tq-fwht] §2 invertibility).
 *   out  device out [batch][n_tokens][n_kv_heads][d] of out_dtype, 16-byte aligned
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_HIP. */
int tq_dequantize(const tq_cache *c, int start_pos, int n_tokens, void *out, int out_dtype,
                  void *hip_stream);

/* Bytes of the packed-code buffer of a cache: batch * n_kv_heads * capacity * d * bits / 8
 * ([tq-plus] §KV缓存的作用与开销 with d*bits/8 bytes per vector); 0 for invalid arguments. */
size_t tq_code_bytes(int d, int bits, int batch, int n_kv_heads, int capacity);

/* Static description of a status code. */
const char *tq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */

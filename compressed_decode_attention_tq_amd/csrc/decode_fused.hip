// Decode attention on matrix cores (gfx950 v_mfma_f32_16x16x32_f16) for keys of 3 or 4 bits
// (TQ_LAYOUT_ROWS) and a query group of up to 8 heads per kv head: dense attention over
// 2-bit values (TQ_LAYOUT_GROUP8) in one launch, or the key-only first pass of Sparse V.
//
// What is computed follows [google] "Google 最新極限壓縮算法…" (scores taken directly
// against the quantized keys as ||k|| (Rq).c[idx], values summed in the rotated domain and
// rotated back once) and, for the gate, [inferrs] "inferrs & TurboQuant：本地 LLM 推理的内存革命"
// §Sparse V.  The schedule is this file's own:
//
//   * Work unit: one workgroup (8 waves, all 160 KB of LDS, so one resident per CU) owns one
//     contiguous split of one (batch, kv head) context; the plan makes about one split per
//     CU.  The waves take the split's 64-token tiles in turn.  Long splits take wider
//     workgroups: 12 waves for groups of up to 4 heads (2 KB wave buffers, 153 KB of LDS),
//     and in the key-only pass 16 (4 heads) or 12 (8 heads).
//   * The query group is rotated once per split: wave h applies the signs and the
//     Walsh-Hadamard butterflies to head h (two coordinates per lane, lane exchanges for the
//     upper six stages) and leaves R q in LDS for all waves.
//   * Codes become fp16 matrix operands through lookup tables in LDS, replicated 32 times
//     so the 32 lanes of one LDS pass never share a bank; every thread builds its part of
//     the tables from the centroids it holds in registers.  A key byte (two 4-bit codes, or
//     a 6-bit pair of 3-bit codes) gives {hi(c_a), hi(c_b), lo(c_a), lo(c_b)}: each centroid
//     split into its fp16 value and the fp16 remainder.  A value byte (four 2-bit codes of
//     one coordinate, four consecutive tokens) gives four fp16 centroids.
//   * Scores keep about 22 significant bits: query row 2h holds the fp16 part of head h,
//     row 2h+1 its remainder, each value repeated to meet the {hi, hi, lo, lo} key operand,
//     so one product sums (q_hi + q_lo).(c_hi + c_lo) over 16 coordinates; the two rows of a
//     head land in the same lane and are added there.
//   * Softmax in base 2 (log2 e is folded into the query) with a stale reference: the
//     reference of a head only moves when a tile would push p * ||v|| past the fp16 range,
//     so the value accumulator is rarely rescaled.  The value product takes P' = p * ||v||
//     split the same way into a fp16 row and a remainder row.
//   * End of split: the waves combine (m, l, O) through LDS; the workgroup writes one
//     partial per query head and bumps a per-(batch, kv head) arrival counter.  The last
//     workgroup to arrive merges the partials, applies the inverse rotation and writes the
//     output and log-sum-exp, then clears the counter for the next call.
//   * Several query positions (speculative verification, a prefill chunk): the query rows
//     are (position, head) pairs, up to 8 per work item, and each row sees the cache up to
//     its own position (a mask in the tiles that reach past the first query's position).
//   * Sparse V first pass (SPARSE): no value loads or products.  Each wave keeps an exact
//     running maximum per head and writes the largest score of each of its tiles per head;
//     the split's (m, l) become the partials the masked value pass (VMASK) merges into each
//     head's final LSE, and that pass visits only the tiles whose maximum reaches some head's
//     threshold.  (With RECORDS, the key pass also writes every token whose score reaches its
//     wave's running maximum + log2(tau) as a candidate record for the vector second pass.)
//   * QJL keys (QJL, 3-bit codes): every score adds the sign-sketch term, the query's sketch
//     against fp16 +/-1 sign operands on matrix cores; dense decode, or Sparse V's key pass
//     and masked value pass.
#include "tq_common.h"
#include "tq_launch.h"
#include "lanes.h"

#include <type_traits>

namespace tq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 64;
constexpr float kInvSqrtD = 0.08838834764831845f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kAMax = 30000.f;   // largest p * ||v|| kept in an fp16 operand
constexpr float kNvFloor = 1e-20f;  // ||v|| used for the range test of an all-zero value
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the key and value code loads: nt (streaming).  Each code byte is read once
// per launch, so the caches get the streaming policy for it; measured 1.5-2.5% faster on
// every decode workload against the default policy, same box.
constexpr int kStreamLoad = 2;

// LDS map (bytes):
//   [0, 64K)      K table: entry e at e*256 + copy*8 (copy < 32); 3-bit keys use entries < 64
//                 only, [0, 16K), and QJL keys put the sign table in [16K, 48K): entry e (a
//                 byte of sign bits) at 16K + e*128 + copy*16 (copy < 8), eight fp16 +/-1
//   [64K, 128K)   V table: entry e at 64K + e*256 + copy*8
//   [128K, 160K)  one 4 KB buffer per wave:
//                   [0, 2K)  scores of the tile, [32 token pairs][2 head halves][2][NH/2]
//                            fp32, 16-byte units XOR-swizzled
//                   [2K, 4K) P' [16 rows][64 tokens] fp16, 16-byte units XOR-swizzled
//                 and, between tiles, the rotated query group (rows of 128 fp32) and the
//                 end-of-split combine.
constexpr int kLdsBytes = 160 * 1024;
constexpr uint32_t kVBase = 64 * 1024;
constexpr uint32_t kWBase = 128 * 1024;
constexpr uint32_t kPBase = 2048;
constexpr uint32_t kSgnBase = 16 * 1024;

__device__ __forceinline__ uint2 lds_u64(const uint8_t *lds, uint32_t addr) {
  return *reinterpret_cast<const uint2 *>(lds + addr);
}
__device__ __forceinline__ uint16_t h16(float x) { return __half_as_ushort(__float2half_rn(x)); }
__device__ __forceinline__ float f16(uint16_t h) { return __half2float(__ushort_as_half(h)); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}

// Score staging: 16-byte unit `u` (0 .. 2*NH/4 - 1 per token pair) of token pair `pr`.
template <int NH>
__device__ __forceinline__ uint32_t score_unit(int pr, int u) {
  if (NH == 4) return (uint32_t)pr * 32u + ((uint32_t)(u ^ ((pr >> 3) & 1)) << 4);
  return (uint32_t)pr * 64u + ((uint32_t)(u ^ ((pr >> 2) & 3)) << 4);
}
// P' staging: 16-byte unit `unit` (tokens 8*unit .. 8*unit+7) of row `row`.
template <uint32_t PB = kPBase>
__device__ __forceinline__ uint32_t pst_off(int row, int unit) {
  return PB + (uint32_t)row * 128u + ((uint32_t)(unit ^ ((row >> 1) & 7)) << 4);
}

// Code tables, built from the centroids each thread holds in registers.  Thread (w, copy),
// w = threadIdx.x / 32, writes copy `copy` of entries e = 16k + w, k = 0..15:
//   K entry e: fp16 {c_K[a], c_K[b]} then their fp16 remainders, a = e & (2^BK - 1) and
//              b the next BK bits of e (two codes of one key byte);
//   V entry e: the fp16 centroids of the four 2-bit codes of value byte e.
template <int BK, bool VTAB>
__device__ __forceinline__ void build_tables(uint8_t *lds, const float (&kcs)[1 << BK], const float (&vcs)[4]) {
  constexpr int NK = 1 << BK;
  uint32_t khl[NK];  // {fp16 value, fp16 remainder}
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const uint16_t h = h16(kcs[i]);
    khl[i] = (uint32_t)h | ((uint32_t)h16(kcs[i] - f16(h)) << 16);
  }
  uint32_t vh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) vh[i] = h16(vcs[i]);
  if (threadIdx.x >= kThreads) return;  // (12-wave workgroups: the first 8 waves build them)
  const int w = threadIdx.x >> 5, copy = threadIdx.x & 31;
  // (3-bit keys: the second code of entry 16k + w is 2k or 2k + 1 by bit 3 of w; a bitwise
  // select, so that the compiler does not turn it into a scratch-memory array index)
  const uint32_t odd = 0u - (uint32_t)((w >> 3) & 1);
  uint32_t c0 = 0u, vlo0 = 0u, vlo1 = 0u;
#pragma unroll
  for (int i = 0; i < NK; ++i) c0 = (w & (NK - 1)) == i ? khl[i] : c0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    vlo0 = (w & 3) == i ? vh[i] : vlo0;
    vlo1 = ((w >> 2) & 3) == i ? vh[i] : vlo1;
  }
  const uint32_t vlo = vlo0 | (vlo1 << 16);
  uint8_t *row = lds + w * 256 + copy * 8;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if (BK == 4 || k < 4) {  // a 3-bit key field has 6 bits: entries < 64
      uint32_t c1;
      if (BK == 4) c1 = khl[k];
      else c1 = (khl[(2 * k + 1) & 7] & odd) | (khl[(2 * k) & 7] & ~odd);
      uint2 kv;
      kv.x = (c0 & 0xffffu) | (c1 << 16);
      kv.y = (c0 >> 16) | (c1 & 0xffff0000u);
      *reinterpret_cast<uint2 *>(row + k * 4096) = kv;
    }
    if (VTAB) *reinterpret_cast<uint2 *>(row + kVBase + k * 4096) = make_uint2(vlo, vh[k & 3] | (vh[(k >> 2) & 3] << 16));
  }
}

// QJL sign table: entry e holds fp16 (2 bit_k - 1) for bits k = 0..7 of e (bit set: +1), eight
// copies so that the 8 lanes of one 128-byte LDS pass read distinct banks.
__device__ __forceinline__ void build_sign_table(uint8_t *lds) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = threadIdx.x + kThreads * i, e = idx >> 3, copy = idx & 7;
    uint32_t wd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      wd[j] = ((e >> (2 * j)) & 1 ? 0x3C00u : 0xBC00u) | ((e >> (2 * j + 1)) & 1 ? 0x3C000000u : 0xBC000000u);
    *reinterpret_cast<uint4 *>(lds + kSgnBase + e * 128 + copy * 16) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }
}

// Partials cross workgroups (and the per-XCD L2 caches) as agent-scope relaxed atomics: the
// stores write through to the coherent level and the loads bypass stale L2 lines, so no
// cache-wide writeback or invalidate is needed around the arrival counter.
__device__ __forceinline__ void store_coherent(float2 *p, float2 v) {
  __hip_atomic_store(reinterpret_cast<uint64_t *>(p), __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_coherent(const float2 *p) {
  return __builtin_bit_cast(float2, __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ float exp2_or_zero(float x, float ref) {
  return (x == -INFINITY || ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x - ref);
}

// Quantize the token at position t of (batch b, kv head kvh) into the key cache (key) or the
// value cache: one wave, two coordinates per lane.  The same steps as the quantize kernels
// ([tq-80] §核心创新: norm, rotation, Lloyd-Max code; [inferrs] §核心技术: Walsh-Hadamard
// rotation): n = ||x|| (fp32, stored as fp16), u = H (s . x) / (sqrt(d) n) with the butterflies
// across the wave, code = number of boundaries below u, then the bits of this token in the
// cache's layout (3/4-bit key rows, 2-bit value groups of 8 tokens, whose other tokens are
// kept).  Two phases, so that the loads are in flight while the wave does other setup work:
// new_token_load reads the input (and the value word the token shares), new_token_store
// computes and writes the codes (the caller waits for the stores before reading them back).
struct NewToken {
  uint32_t x0, x1;  // raw input bits: two fp32 words, or one word of two 16-bit values
  uint32_t vword;   // value cache: the group word that lane's coordinates go into
};

// b: the sequence; j: the token among the sequence's nt new tokens (input [batch][nt][kv heads][d]);
// pb, pt: the plane (sequence, or pool page) and the position in it
__device__ __forceinline__ NewToken new_token_load(const DecodeArgs &a, bool key, int b, int kvh, int pb, int pt,
                                                   int lane, int j = 0, int nt = 1) {
  const void *x = key ? a.xk : a.xv;
  const size_t xi = (((size_t)b * nt + j) * a.n_kv_heads + kvh) * kD + 2 * lane;
  NewToken n{0u, 0u, 0u};
  if (a.x_dtype == TQ_F32) {
    const uint2 w = *reinterpret_cast<const uint2 *>(reinterpret_cast<const float *>(x) + xi);
    n.x0 = w.x;
    n.x1 = w.y;
  } else {
    n.x0 = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(x) + xi);
  }
  if (!key) n.vword = reinterpret_cast<const uint32_t *>(a.v.plane(pb, kvh) + (size_t)(pt >> 3) * 256)[lane];
  return n;
}

// vatomic (values, several new tokens of one group from different waves): the token's two
// 2-bit fields of the group word are replaced with compare-and-swap, which keeps the other
// tokens' fields (disjoint, possibly written meanwhile) instead of storing the word loaded
// before.  Each swap writes the word with the token's fields already final: the work items of
// other row groups append the same tokens into the same words while this one may read them, so
// a field must never pass through a cleared state (an and-then-or pair would expose one).
template <int BK>
__device__ void new_token_store(const DecodeArgs &a, bool key, const NewToken &in, int pb, int kvh, int t, int lane,
                                uint8_t *scratch, bool vatomic = false) {
  const CacheView &c = key ? a.k : a.v;
  float x0, x1;
  if (a.x_dtype == TQ_F32) {
    x0 = __uint_as_float(in.x0);
    x1 = __uint_as_float(in.x1);
  } else if (a.x_dtype == TQ_BF16) {
    x0 = __uint_as_float(in.x0 << 16);
    x1 = __uint_as_float(in.x0 & 0xffff0000u);
  } else {
    x0 = f16((uint16_t)(in.x0 & 0xffffu));
    x1 = f16((uint16_t)(in.x0 >> 16));
  }
  const float ss = x0 * x0 + x1 * x1;
  const float n = sqrtf(wave_reduce<false>(ss));
  const float y0 = c.signs[2 * lane] < 0 ? -x0 : x0, y1 = c.signs[2 * lane + 1] < 0 ? -x1 : x1;
  float u0 = y0 + y1, u1 = y0 - y1;
  wave_fwht_upper(u0, u1, lane);
  const float inv = n > 0.f ? 1.0f / (n * 11.313708498984761f) : 0.f;
  u0 *= inv;
  u1 *= inv;
  const int nb = key ? (1 << BK) - 1 : 3;
  uint32_t c0 = 0u, c1 = 0u;
  for (int j = 0; j < nb; ++j) {
    const float tj = c.boundaries[j];
    c0 += u0 > tj ? 1u : 0u;
    c1 += u1 > tj ? 1u : 0u;
  }
  if (lane == 0) c.norm_plane(pb, kvh)[t] = float_to_half_bits(n);
  uint8_t *plane = c.plane(pb, kvh);
  if (key) {
    if (BK == 4) {
      plane[(size_t)t * 64 + lane] = (uint8_t)(c0 | (c1 << 4));
    } else {  // the 384-bit row, lane l's two codes at bit 6 l
      uint32_t *words = reinterpret_cast<uint32_t *>(scratch);
      if (lane < 12) words[lane] = 0u;
      __builtin_amdgcn_wave_barrier();
      __asm__ volatile("" ::: "memory");
      const uint32_t f = c0 | (c1 << 3);
      const int bit = 6 * lane, wi = bit >> 5, sh = bit & 31;
      atomicOr(&words[wi], f << sh);
      if (sh > 26) atomicOr(&words[wi + 1], f >> (32 - sh));
      __builtin_amdgcn_wave_barrier();
      __asm__ volatile("" ::: "memory");
      if (lane < 12) reinterpret_cast<uint32_t *>(plane + (size_t)t * 48)[lane] = words[lane];
    }
  } else {
    // value group of 8 tokens: coordinate i of token p at bit 2 (8 i + p); lane l's
    // coordinates 2l and 2l+1 make up 32-bit word l of the group
    const int p = t & 7, s0 = 8 * (p >> 2) + 2 * (p & 3), s1 = s0 + 16;
    const uint32_t mask = (3u << s0) | (3u << s1), bits = (c0 << s0) | (c1 << s1);
    uint32_t *word = reinterpret_cast<uint32_t *>(plane + (size_t)(t >> 3) * 256) + lane;
    if (vatomic) {
      // each failed swap means another writer's swap succeeded, and every writer swaps once:
      // the loop ends after at most as many rounds as there are writers of the word
      uint32_t old = in.vword;
      for (;;) {
        const uint32_t seen = atomicCAS(word, old, (old & ~mask) | bits);
        if (seen == old) break;
        old = seen;
      }
    } else {
      *word = (in.vword & ~mask) | bits;
    }
  }
}

// MULTI: several query positions (a.n_q > 1 or several row groups); a template flag so that
// single-query decode keeps none of its bookkeeping live across the tile loop.
// APPEND: the new token of each sequence is quantized into the caches first (a.xk, a.xv).
// PAGED: the caches are page pools found through a.block_table; each tile lies inside one
// page (pages are whole multiples of 64 tokens), so a tile's loads differ from the
// contiguous case only by its base offset.
// VMASK: Sparse V's value pass after the key pass.  The final LSE of every head is merged from
// the key pass's partials (a.lse_ml) at set-up, so the pass needs no running softmax: p =
// exp(s - LSE) is the final weight, and a row with p < tau adds nothing (no renormalisation).
// A wave visits only the tiles whose largest score (a.tile_max, written by the key pass)
// reaches some head's threshold LSE + ln tau: it loads keys and values of those tiles alone.
// Partials are then already normalised: the merge sums them and writes the key pass's LSE.
// RECORDS (with SPARSE): the key pass also writes candidate records for the record-based second
// pass; without, it writes only the (m, l) partials and the per-tile maxima the masked value
// pass reads.
// The key pass without records needs only the key table and the score staging: its LDS is the
// 64 KB table plus 2 KB per wave (80 KB with 8 waves).  (Two such workgroups per CU, 4 waves per
// SIMD at 128 VGPRs forced, made the pass slower: 22 -> 28 us on the 131072-token workload, with
// spills; one workgroup of 16 or 12 waves at the VGPRs the pass needs anyway made it faster.)
// PREFILL (with MULTI): several query positions with many row groups per kv head (a prefill
// chunk).  The 8 waves of a workgroup take 8 row groups, not 8 slices of the tiles: every wave
// walks all tiles of the split for its own rows, so the workgroup reads each tile of keys and
// values from memory once for up to 64 query rows (the other waves find it in L2).  Each wave
// keeps its own softmax, writes its own partials and merges its row group's splits when it is
// the last to arrive; there is no combine across waves.
template <int BK, int NH, bool SPARSE, bool MULTI, bool APPEND, bool PAGED, bool VMASK = false, bool RECORDS = true,
          bool PREFILL = false, bool QJL = false, int W = kWaves>
__device__ __forceinline__ void decode_fused_body(const DecodeArgs &a) {
  static_assert(NH == 4 || NH == 8, "NH heads of two rows each must fit 16 rows");
  static_assert(!PREFILL || (MULTI && !SPARSE && !APPEND && !VMASK), "prefill: dense multi-query only");
  static_assert(!(MULTI && APPEND) || (!SPARSE && !PAGED), "several new tokens: dense, contiguous caches");
  static_assert(!PAGED || !((SPARSE && RECORDS) || (MULTI && APPEND)),
                "paged caches: decode, its append, several query positions (prefill chunks too), Sparse V's two passes");
  static_assert(!VMASK || !(SPARSE || MULTI || APPEND), "masked value pass: single-query decode");
  static_assert(!QJL || (BK == 3 && !(MULTI || APPEND || PAGED || PREFILL || (SPARSE && RECORDS))),
                "QJL keys: 3-bit codes, single-query decode, dense or Sparse V's two passes");
  constexpr bool KEYS_ONLY = SPARSE && !RECORDS;
  // More waves per workgroup for single-query decode, paged or not, with long splits:
  //   W = 12 (three per SIMD), groups of up to 4 heads, values too: 2 KB wave buffers (scores
  //     [0, 1K), P' rows 0..7 [1K, 2K)) and a shared zero block for P' rows 8..15, behind the
  //     tables;
  //   the key-only first pass of Sparse V (2 KB wave buffers already): W = 16 for groups of
  //     up to 4 heads, W = 12 for up to 8.
  static_assert(W == kWaves ||
                    (!(MULTI || VMASK || PREFILL || QJL) &&
                     ((W == 12 && NH == 4 && !SPARSE) || (KEYS_ONLY && ((W == 16 && NH == 4) || (W == 12 && NH == 8))))),
                "wider workgroups: single-query decode with long splits");
  constexpr uint32_t PB = W == 12 ? 1024u : kPBase;   // P' staging inside a wave buffer
  constexpr uint32_t kZeroBase = kWBase + 12 * 2048;  // (W = 12) 1 KB of zeros
  constexpr int NH2 = NH / 2;      // heads per softmax lane
  constexpr int KROW = 16 * BK;    // key bytes per token
  constexpr uint32_t WBASE = KEYS_ONLY ? kVBase : kWBase;  // per-wave staging buffers
  constexpr uint32_t WSTRIDE = KEYS_ONLY || W == 12 ? 2048u : 4096u;
  __shared__ __attribute__((aligned(16))) uint8_t lds[KEYS_ONLY ? kVBase + W * 2048
                                                      : W == 12 ? kZeroBase + 1024 : kLdsBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar offsets
  const int g = a.group, S = a.fplan.n_splits, L = a.fplan.split_len;
  const int n_q = MULTI ? a.n_q : 1, VG = MULTI ? a.vgroups : 1, vgs = MULTI ? a.vg_size : g;
  const int m_row = lane & 15, quarter = lane >> 4;
  const int pr = lane & 31, half_id = lane >> 5;  // softmax mapping: tokens 2pr, 2pr+1
  const uint32_t kc8 = (uint32_t)(lane & 31) << 3;
  const uint32_t vc8 = ((uint32_t)(lane & 31) << 3) | kVBase;
  uint8_t *wbuf = lds + WBASE + wave * WSTRIDE;
  float *qrot = reinterpret_cast<float *>(lds + WBASE);  // [NH][128] between tiles

  if constexpr (W == 12 && !KEYS_ONLY) {  // the zero block that P' rows 8..15 read
    if (wave == 0) *reinterpret_cast<uint4 *>(lds + kZeroBase + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
  } else if (!SPARSE && NH == 4) {  // P' rows 8..15 stay zero for the whole launch
    *reinterpret_cast<uint4 *>(wbuf + kPBase + 1024 + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
  }

  {  // one split of one (batch, kv head) per workgroup
    const int VGB = PREFILL ? (VG + kWaves - 1) / kWaves : VG;  // items per (batch, kv head, split)
    // Work item -> (unit u = (b, kv head, split), row-group item vgb).  With several row-group
    // items per unit they read the same tiles: workgroups are dealt to the 8 XCDs round robin
    // by their index, so the items of one unit get indices congruent to u mod 8 (all on one
    // XCD, whose L2 then serves the repeated reads): item = (vgb * G + u / 8) * 8 + u % 8,
    // G = ceil(units / 8), indices past the last unit idle.
    int u = blockIdx.x, vgb = 0;
    if (VGB > 1) {
      const int units = a.batch * a.n_kv_heads * S, G = (units + 7) / 8;
      const int lo = (int)blockIdx.x & 7, hi = (int)blockIdx.x >> 3;
      vgb = hi / G;
      u = (hi - vgb * G) * 8 + lo;
      if (u >= units || vgb >= VGB) return;  // (uniform: before any barrier or store)
    }
    const int split = u % S;
    const int vgi = PREFILL ? vgb * kWaves + wave : vgb;  // PREFILL: each wave its own row group
    const int kvh = (u / S) % a.n_kv_heads;
    const int b = u / (S * a.n_kv_heads);
    const bool wave_on = !PREFILL || vgi < VG;
    int T = a.ctx_len;
    if (a.seq_lens != nullptr) T = __builtin_amdgcn_readfirstlane(min(max(a.seq_lens[b], 0), a.ctx_len));
    const int t_begin = split * L;
    const int t_end = min(t_begin + L, T);
    const int qh0 = kvh * g;  // first query head of the group
    // Query rows ("heads" of this item): row h is query position f / g, head kvh*g + f % g,
    // f = vgi * vgs + h; it sees cache positions up to T - n_q + f / g.  For decode (n_q = 1,
    // one item per kv head) row h is simply head qh0 + h.
    auto vlive = [&](int h) { return MULTI ? h < vgs && vgi * vgs + h < n_q * g : h < g; };
    auto vrow = [&](int h) -> size_t {  // row of q, out and lse: [batch][n_q][n_q_heads]
      if constexpr (!MULTI) return (size_t)b * a.n_q_heads + qh0 + h;
      const int f = vgi * vgs + h, i = f / g;
      return ((size_t)b * n_q + i) * a.n_q_heads + kvh * g + (f - i * g);
    };

    const int n_tiles = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;
    // Buffers: the split's span of one plane, or (paged) the whole pools, whose size the host
    // keeps below 3 GiB.  tile_tok(tile) is the tile's first position counted in tokens of
    // the buffer; a tile with no page gets an offset past the end, so its loads read zeros
    // without touching memory, and its positions are masked out of the softmax.
    const uint32_t span_tok = PAGED ? (uint32_t)a.n_pages * a.n_kv_heads * a.k.capacity : (uint32_t)n_tiles * kTile;
    const __amdgpu_buffer_rsrc_t krs =
        PAGED ? make_rsrc(a.k.codes, span_tok * KROW) : make_rsrc(a.k.plane(b, kvh) + (size_t)t_begin * KROW, span_tok * KROW);
    const __amdgpu_buffer_rsrc_t vrs =
        PAGED ? make_rsrc(a.v.codes, span_tok * 32) : make_rsrc(a.v.plane(b, kvh) + (size_t)t_begin * 32, span_tok * 32);
    const __amdgpu_buffer_rsrc_t knrs =
        PAGED ? make_rsrc(a.k.norms, span_tok * 2) : make_rsrc(a.k.norm_plane(b, kvh) + t_begin, span_tok * 2);
    const __amdgpu_buffer_rsrc_t vnrs =
        PAGED ? make_rsrc(a.v.norms, span_tok * 2) : make_rsrc(a.v.norm_plane(b, kvh) + t_begin, span_tok * 2);
    // QJL: the split's sign rows (16 bytes per token) and residual norms
    const size_t qjl_row = QJL ? ((size_t)b * a.n_kv_heads + kvh) * a.k.capacity + t_begin : 0;
    const __amdgpu_buffer_rsrc_t sbrs = make_rsrc(QJL ? a.qjl_bits + qjl_row * 16 : nullptr, QJL ? span_tok * 16 : 0);
    const __amdgpu_buffer_rsrc_t rnrs = make_rsrc(QJL ? a.qjl_rnorm + qjl_row : nullptr, QJL ? span_tok * 2 : 0);
    constexpr uint32_t kNoPage = 0xffffffffu;
    // A value-pass split of at most 64 tiles is shared out by need (lane k: tile k, see VMASK
    // below); every other split keeps the round-robin tiles (lane i: tile wave + W i).
    const bool by_need = VMASK && n_tiles <= 64;
    // lane k holds tile k's page offset where a wave may visit any tile of its split (shared
    // by need, or prefill: every wave walks all of at most 64 tiles)
    const bool by_tile = by_need || PREFILL;
    uint32_t page_tok = kNoPage;  // paged: lane i holds tile_tok of its tile in the mapping above
    if constexpr (PAGED) {
      const int tile_i = by_tile ? lane : wave + W * lane;
      if (tile_i < n_tiles) {
        const int P = a.k.capacity, t0 = t_begin + tile_i * kTile, slot = t0 / P;
        const int page = slot < a.max_pages ? a.block_table[(size_t)b * a.max_pages + slot] : -1;
        if (page >= 0 && page < a.n_pages) page_tok = ((uint32_t)page * a.n_kv_heads + kvh) * P + (t0 - slot * P);
      }
    }
    auto tile_tok = [&](int tile) -> uint32_t {
      if constexpr (PAGED)
        return (uint32_t)__builtin_amdgcn_readlane((int)page_tok, by_tile ? tile : (tile - wave) / W);
      else return (uint32_t)tile * kTile;
    };
    auto tile_off = [&](uint32_t tok, uint32_t unit) -> uint32_t {  // bytes; past the end for no page
      return PAGED && tok == kNoPage ? 0xf0000000u : tok * unit;
    };
    const uint32_t k_voff = (uint32_t)m_row * KROW + (uint32_t)quarter * (4 * BK);
    const uint32_t v_voff = (uint32_t)quarter * 256u + (uint32_t)m_row * 16u;
    const uint32_t n_voff = (uint32_t)pr * 4u;

    uint32_t kw[4][4];
    uint32_t nkw = 0;
    // QJL, per sub-tile s: the sign bits 32 quarter .. 32 quarter + 31 of token 16 s + m_row (the
    // lane's B-operand column), and that token's key norm and residual norm
    uint32_t sgw[4] = {0u, 0u, 0u, 0u};
    uint16_t nq16[4] = {0, 0, 0, 0}, rq16[4] = {0, 0, 0, 0};
    auto load_keys = [&](int tile) {
      // the whole offset is in the vector offset: a tile past the split's end lies outside
      // the buffer's range and reads as zeros without touching memory
      const uint32_t tok = tile_tok(tile);
      const uint32_t so = tile_off(tok, KROW);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (BK == 4) {
          const auto w = __builtin_amdgcn_raw_buffer_load_b128(krs, k_voff + so + s * 16 * KROW, 0, kStreamLoad);
          kw[s][0] = w[0]; kw[s][1] = w[1]; kw[s][2] = w[2]; kw[s][3] = w[3];
        } else {
          const auto w = __builtin_amdgcn_raw_buffer_load_b96(krs, k_voff + so + s * 16 * KROW, 0, kStreamLoad);
          kw[s][0] = w[0]; kw[s][1] = w[1]; kw[s][2] = w[2]; kw[s][3] = 0u;
        }
      }
      if constexpr (QJL) {
        const uint32_t t16 = (uint32_t)tile * kTile + (uint32_t)m_row;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          sgw[s] = __builtin_amdgcn_raw_buffer_load_b32(sbrs, (t16 + 16 * s) * 16 + (uint32_t)quarter * 4, 0, 0);
          nq16[s] = __builtin_amdgcn_raw_buffer_load_b16(knrs, (t16 + 16 * s) * 2, 0, 0);
          rq16[s] = __builtin_amdgcn_raw_buffer_load_b16(rnrs, (t16 + 16 * s) * 2, 0, 0);
        }
      } else {
        nkw = __builtin_amdgcn_raw_buffer_load_b32(knrs, n_voff + tile_off(tok, 2), 0, 0);
      }
    };

    // APPEND: in the workgroup whose split holds position T - 1, the wave that reads that
    // position's tile (tiles go to waves round robin) writes the new token's key and value
    // first.  Only that wave ever loads those bytes, so no other wave waits for the stores:
    // the writer waits for its own stores to complete after the first barrier and only then
    // issues its first key tile if that tile holds T - 1; later tiles are loaded later still.
    // Paged: the token goes to its slot of the page the table names; with no page there, it
    // is not written (and its tile reads zeros).
    const bool has_new = APPEND && T >= 1 && T - 1 >= t_begin && T - 1 < t_end;
    const int new_tile = has_new ? (T - 1 - t_begin) / kTile : -1;
    bool appends = has_new && new_tile % W == wave;
    int new_pb = b, new_pt = T - 1;  // plane and position of the new token
    if constexpr (PAGED) {
      if (appends) {
        const int P = a.k.capacity, slot = (T - 1) / P;
        new_pb = __builtin_amdgcn_readfirstlane(a.block_table[(size_t)b * a.max_pages + slot]);
        new_pt = T - 1 - slot * P;
        appends = new_pb >= 0 && new_pb < a.n_pages;
      }
    }
    bool defer_keys = appends && new_tile == wave;
    NewToken ntk{0u, 0u, 0u}, ntv{0u, 0u, 0u};
    if (!MULTI && appends) {
      ntk = new_token_load(a, true, b, kvh, new_pb, new_pt, lane);
      ntv = new_token_load(a, false, b, kvh, new_pb, new_pt, lane);
    }
    // MULTI: the n_q new tokens of the sequence go to positions T - n_q .. T - 1 (those >= 0) of
    // this split; token j goes in through wave j mod W (bit j of `mine`), so the tokens are
    // quantized side by side.  Their value fields are set with compare-and-swap (tokens of one
    // group touch disjoint fields of the same words); every appending wave waits for its writes
    // before the set-up barrier, and a wave whose first tile holds a new token loads it after
    // that barrier.  With several row groups per kv head each item writes the same bytes again,
    // every write already final, so a reader sees the same bytes whichever write it follows.
    constexpr int MT = MULTI && APPEND ? kMultiAppendMax : 1;
    uint32_t mine = 0u;
    NewToken mk[MT], mv[MT];
    if constexpr (MULTI && APPEND) {
      defer_keys = false;
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int p = T - n_q + j;
        mk[j] = mv[j] = NewToken{0u, 0u, 0u};
        if (j < n_q && p >= 0 && p >= t_begin && p < t_end) {
          if ((p - t_begin) / kTile == wave) defer_keys = true;
          if (j % W == wave) {
            mine |= 1u << j;
            mk[j] = new_token_load(a, true, b, kvh, b, p, lane, j, n_q);
            mv[j] = new_token_load(a, false, b, kvh, b, p, lane, j, n_q);
          }
        }
      }
      appends = mine != 0u;
    }

    // the small loads the setup needs go out first, then the wave's first key tile; nothing
    // is used until all of them are in flight (a use would make the wave wait right there)
    float kcs[1 << BK], vcs[4];
#pragma unroll
    for (int i = 0; i < (1 << BK); ++i) kcs[i] = a.k.centroids[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) vcs[i] = a.v.centroids[i];
    // (PREFILL: each wave loads its own rows when it rotates them; a wave past the last row group
    // has no row to read)
    uint32_t qw0 = 0u, qw1 = 0u;
    if constexpr (!PREFILL) {
      const size_t qbase = vrow(vlive(wave) ? wave : 0) * kD + 2 * lane;
      if (a.q_dtype == TQ_F32) {
        const uint2 w = *reinterpret_cast<const uint2 *>(reinterpret_cast<const float *>(a.q) + qbase);
        qw0 = w.x;
        qw1 = w.y;
      } else {
        qw0 = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(a.q) + qbase);
      }
    }
    const uint16_t sgn = *reinterpret_cast<const uint16_t *>(a.k.signs + 2 * lane);
    // QJL: wave w computes sketch rows j = 16 w .. 16 w + 15 of the query group; the lane loads
    // S[j][32 quarter .. 32 quarter + 31], j = 16 w + m_row (its B-operand column)
    float4 srow[8];
    if constexpr (QJL) {
      const float4 *src = reinterpret_cast<const float4 *>(a.qjl_proj + (size_t)(16 * wave + m_row) * kD + 32 * quarter);
#pragma unroll
      for (int m = 0; m < 8; ++m) srow[m] = src[m];
    }
    if (!defer_keys && !VMASK) load_keys(PREFILL ? 0 : wave);
    // VMASK: a split of at most 64 tiles is shared out by need (lane k looks at tile k); a longer
    // one (at most 64 tiles per wave) keeps the round-robin tiles (lane k: tile wave + 8 k), where
    // most tiles are needed anyway.  The maxima of those tiles for every head of the group are
    // loaded now, so that only the comparison waits for the thresholds.
    float tmx[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) tmx[h] = -INFINITY;
    if constexpr (VMASK) {
      const int tile_k = by_need ? lane : wave + kWaves * lane;
      if (tile_k < n_tiles) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
          if (vlive(h)) tmx[h] = a.tile_max[vrow(h) * a.tile_stride + (t_begin >> 6) + tile_k];
      }
    }
    // value centroids scaled by the cache's table scale, chosen so that the fp16 table holds
    // them almost exactly (taken off the output at merge)
    const float vscale = SPARSE ? 1.f : a.v.table_scale;
    float vcs_s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vcs_s[i] = vcs[i] * vscale;
    build_tables<BK, !SPARSE>(lds, kcs, vcs_s);  // read only after the barriers below
    if constexpr (QJL) build_sign_table(lds);
    // 3-bit rows are assembled in the first 48 bytes of the wave's own buffer: during set-up
    // no other wave writes there (the rotated query's rows 1.. start at byte 512 of wave 0's).
    // The key-only pass has 2 KB buffers, where the rotated query of 8 heads covers those of
    // waves 0 and 1: there the rows go behind the 16 KB table of 3-bit keys, a region the pass
    // does not use.
    if (appends) {
      uint8_t *ascr = KEYS_ONLY ? lds + 16 * 1024 + wave * 64 : lds + kWBase + wave * WSTRIDE;
      if constexpr (MULTI && APPEND) {
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          if (!((mine >> j) & 1u)) continue;
          const int p = T - n_q + j;
          new_token_store<BK>(a, true, mk[j], b, kvh, p, lane, ascr);
          new_token_store<BK>(a, false, mv[j], b, kvh, p, lane, ascr, true);
        }
      } else {
        new_token_store<BK>(a, true, ntk, new_pb, kvh, new_pt, lane, ascr);
        new_token_store<BK>(a, false, ntv, new_pb, kvh, new_pt, lane, ascr);
      }
    }
    // Sparse V: candidate count of each second-pass split this split covers (LDS atomics;
    // the value-table region is free in that mode)
    int *chunk_count = reinterpret_cast<int *>(lds + kVBase);
    const int c_first = SPARSE ? t_begin / a.plan.split_len : 0;
    const int n_chunks = SPARSE ? a.fplan.split_len / a.plan.split_len : 0;
    if (SPARSE && RECORDS && (int)threadIdx.x < n_chunks) chunk_count[threadIdx.x] = 0;

    // ---- rotated query group: wave h rotates head h into qrot[h] (PREFILL: every wave rotates
    //      its own rows into its own buffer)
    auto rotate_row = [&](bool live, uint32_t w0, uint32_t w1, float *dst) {
      float x0 = 0.f, x1 = 0.f;
      if (live) {
        if (a.q_dtype == TQ_F32) {
          x0 = __uint_as_float(w0);
          x1 = __uint_as_float(w1);
        } else if (a.q_dtype == TQ_BF16) {
          x0 = __uint_as_float(w0 << 16);
          x1 = __uint_as_float(w0 & 0xffff0000u);
        } else {
          x0 = f16((uint16_t)(w0 & 0xffffu));
          x1 = f16((uint16_t)(w0 >> 16));
        }
        if (sgn & 0x80u) x0 = -x0;
        if (sgn & 0x8000u) x1 = -x1;
      }
      const float y0 = x0 + x1, y1 = x0 - x1;
      x0 = y0;
      x1 = y1;
      wave_fwht_upper(x0, x1, lane);
      const float qs = a.scale * kInvSqrtD * kLog2e;
      *reinterpret_cast<float2 *>(dst + 2 * lane) = make_float2(x0 * qs, x1 * qs);
    };
    if constexpr (PREFILL) {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        uint32_t w0 = 0u, w1 = 0u;
        if (vlive(h)) {
          const size_t qi = vrow(h) * kD + 2 * lane;
          if (a.q_dtype == TQ_F32) {
            const uint2 w = *reinterpret_cast<const uint2 *>(reinterpret_cast<const float *>(a.q) + qi);
            w0 = w.x;
            w1 = w.y;
          } else {
            w0 = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(a.q) + qi);
          }
        }
        rotate_row(vlive(h), w0, w1, reinterpret_cast<float *>(wbuf) + h * kD);
      }
    } else if (wave < NH) {
      rotate_row(vlive(wave), qw0, qw1, qrot + wave * kD);
    }
    // VMASK, set-up only: [0, NH) thresholds on s (log2 units) = (LSE + ln tau) log2 e, [8, 8 + NH)
    // the LSE in log2 units (the fixed softmax reference of the pass)
    float *thr_lds = reinterpret_cast<float *>(lds + kWBase + 4096 + 64);
    float lse_own = -INFINITY;  // VMASK: natural-log LSE of head `wave`
    if constexpr (VMASK) {
      if (wave < NH) {
        float m = -INFINITY, l = 0.f;
        if (vlive(wave)) {
          const float2 *ml = a.lse_ml + vrow(wave) * a.lse_splits;
          if (a.lse_splits <= 64) {  // one partial per lane, loaded once for both reductions
            const float2 v = lane < a.lse_splits ? ml[lane] : make_float2(-INFINITY, 0.f);
            m = wave_reduce<true>(v.x);
            l = wave_reduce<false>(m != -INFINITY && v.x != -INFINITY ? v.y * __expf(v.x - m) : 0.f);
          } else {
            for (int k = lane; k < a.lse_splits; k += 64) m = fmaxf(m, ml[k].x);
            m = wave_reduce<true>(m);
            if (m != -INFINITY)
              for (int k = lane; k < a.lse_splits; k += 64)
                if (ml[k].x != -INFINITY) l += ml[k].y * __expf(ml[k].x - m);
            l = wave_reduce<false>(l);
          }
        }
        lse_own = m == -INFINITY ? -INFINITY : m + __logf(l);
        if (lane == 0) {
          thr_lds[wave] = m == -INFINITY ? INFINITY : (lse_own + a.ln_tau) * kLog2e;
          thr_lds[8 + wave] = lse_own * kLog2e;
        }
      }
    }
    // MULTI: every appending wave's writes are complete before the barrier (vmcnt(0) covers the
    // wave's own stores and atomics); the deferred tile is loaded after it
    if (MULTI && APPEND && appends) __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (appends || defer_keys) {  // (MULTI: the tokens of a deferred tile may come from other waves,
                                  // all written before the barrier above)
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the new token's stores are complete
      if (defer_keys) load_keys(wave);
    }
    float vthr[NH2], vref[NH2];
#pragma unroll
    for (int hh = 0; hh < NH2; ++hh) {
      vthr[hh] = VMASK ? thr_lds[half_id * NH2 + hh] : -INFINITY;
      vref[hh] = VMASK ? thr_lds[8 + half_id * NH2 + hh] : -INFINITY;
    }
    // VMASK: the needed tiles (a score reaches some head's threshold).  By need, the k-th needed
    // tile of the split goes to wave k mod 8, so that a wave gets at most one more than another,
    // and bit k of `need` is tile k; round robin, bit k is tile wave + 8 k.
    uint64_t need = 0;
    if constexpr (VMASK) {
      bool nd = false;
#pragma unroll
      for (int h = 0; h < NH; ++h) nd |= tmx[h] >= thr_lds[h];
      const uint64_t all = __ballot(nd);
      const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(all >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)all, 0u));
      need = by_need ? __ballot(nd && (rank & (kWaves - 1)) == wave) : all;
    }
    auto need_tile = [&](int bit) { return by_need ? bit : wave + kWaves * bit; };
    // operand rows: 2h = fp16 part of head h, 2h+1 = remainder; rows >= 2*NH are zero
    half8 qop[8];
    {
      const int head = m_row >> 1;
      const bool lo_row = (m_row & 1) != 0;
      const bool live = head < NH && vlive(head);
      float v[32];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float *qsrc = PREFILL ? reinterpret_cast<const float *>(wbuf) : qrot;
        float4 f = live ? *reinterpret_cast<const float4 *>(qsrc + head * kD + 32 * quarter + 4 * r)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
        v[4 * r] = f.x; v[4 * r + 1] = f.y; v[4 * r + 2] = f.z; v[4 * r + 3] = f.w;
      }
      _Float16 part[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const _Float16 hi = (_Float16)v[e];
        part[e] = lo_row ? (_Float16)(v[e] - (float)hi) : hi;
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        qop[m][0] = part[4 * m];     qop[m][1] = part[4 * m + 1];
        qop[m][2] = part[4 * m];     qop[m][3] = part[4 * m + 1];
        qop[m][4] = part[4 * m + 2]; qop[m][5] = part[4 * m + 3];
        qop[m][6] = part[4 * m + 2]; qop[m][7] = part[4 * m + 3];
      }
    }
    // QJL: the query sketch pq[h][j] = sqrt(pi/2)/m (S R q~)_j on matrix cores: the query
    // operands above against S^T (each element split into its fp16 value and remainder, in the
    // {hi, hi, lo, lo} order of the key operands), 8 products per wave for its 16 rows of S.
    // Lane (m_row, quarter) gets heads 2 quarter, 2 quarter + 1 of row j; pq goes to wave
    // buffers 2..3, then comes back as the A operands of the sign products, rows as for qop
    // (2h the fp16 part of head h, 2h+1 the remainder); K step kk of the lane's quarter covers
    // signs 32 quarter + 8 kk .. + 7, byte kk of the lane's sign word.
    half8 sop[4];
    if constexpr (QJL) {
      float *pq_lds = reinterpret_cast<float *>(lds + WBASE + 2 * WSTRIDE);  // [NH][128], wave buffers 2..3
      floatx4 pacc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float f[4] = {srow[m].x, srow[m].y, srow[m].z, srow[m].w};
        _Float16 hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hi[e] = (_Float16)f[e];
          lo[e] = (_Float16)(f[e] - (float)hi[e]);
        }
        half8 sb;
        sb[0] = hi[0]; sb[1] = hi[1]; sb[2] = lo[0]; sb[3] = lo[1];
        sb[4] = hi[2]; sb[5] = hi[3]; sb[6] = lo[2]; sb[7] = lo[3];
        pacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qop[m], sb, pacc, 0, 0, 0);
      }
      constexpr float kQjlKappa = 1.2533141373155003f / (float)kD;  // sqrt(pi/2) / m, m = d
      if (2 * quarter < NH) {
        const int j = 16 * wave + m_row;
        pq_lds[(2 * quarter) * kD + j] = kQjlKappa * (pacc[0] + pacc[1]);
        pq_lds[(2 * quarter + 1) * kD + j] = kQjlKappa * (pacc[2] + pacc[3]);
      }
      __syncthreads();
      const int head = m_row >> 1;
      const bool lo_row = (m_row & 1) != 0;
      const bool live = head < NH && vlive(head);
      const float *src = pq_lds + (live ? head : 0) * kD + 32 * quarter;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const float4 f0 = live ? *reinterpret_cast<const float4 *>(src + 8 * kk) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 f1 = live ? *reinterpret_cast<const float4 *>(src + 8 * kk + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float v[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const _Float16 hi = (_Float16)v[e];
          sop[kk][e] = lo_row ? (_Float16)(v[e] - (float)hi) : hi;
        }
      }
    }
    __syncthreads();  // qrot (wave buffers 0..1) and pq (2..3) are free for staging from here

    // last visible position of this lane's rows (they differ only with several query
    // positions; -1 for a row without a query)
    int vlim[NH2];
#pragma unroll
    for (int hh = 0; hh < NH2; ++hh) {
      const int h = half_id * NH2 + hh;
      vlim[hh] = MULTI && vlive(h) ? T - n_q + (vgi * vgs + h) / g : -1;
    }

    // ---- per-lane softmax state: heads half_id*NH2 + hh
    float mr[NH2], lsum[NH2];
#pragma unroll
    for (int hh = 0; hh < NH2; ++hh) { mr[hh] = vref[hh]; lsum[hh] = 0.f; }
    floatx4 oacc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) oacc[n] = floatx4{0.f, 0.f, 0.f, 0.f};


    // one tile; PREFETCH issues the key loads of the wave's next tile.  The last tile is
    // peeled off so that the loads are never conditional inside the loop body: a load
    // issued on one path only would make every later wait cover it as well.
    auto tile_body = [&](int tile, int next_tile, auto prefetch_tag) {
      constexpr bool PREFETCH = decltype(prefetch_tag)::value;
      const int t0 = t_begin + tile * kTile;
      const uint32_t tok = tile_tok(tile);
      uint32_t vw[2][4];
      uint32_t nvw = 0u;
      if constexpr (!SPARSE) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const auto w = __builtin_amdgcn_raw_buffer_load_b128(vrs, v_voff + tile_off(tok, 32) + c * 1024, 0, kStreamLoad);
          vw[c][0] = w[0]; vw[c][1] = w[1]; vw[c][2] = w[2]; vw[c][3] = w[3];
        }
        nvw = __builtin_amdgcn_raw_buffer_load_b32(vnrs, n_voff + tile_off(tok, 2), 0, 0);
      }

      // ---- scores: sub-tile s, 16-coordinate chunk m -> key fields 2m, 2m+1 of the quarter
      auto key_operands = [&](int m, half8 (&dst)[4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          uint2 t2[2];
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const int f = 2 * m + p;
            uint32_t addr;
            if (BK == 4) {
              addr = __builtin_amdgcn_perm(kw[s][f >> 2], kc8, 0x0C0C0000u | ((4u + (f & 3)) << 8));
            } else {
              const int bit = 6 * f;
              uint32_t fld;
              if ((bit & 31) <= 26) fld = (kw[s][bit >> 5] >> (bit & 31)) & 63u;
              else fld = ((kw[s][bit >> 5] >> (bit & 31)) | (kw[s][(bit >> 5) + 1] << (32 - (bit & 31)))) & 63u;
              addr = (fld << 8) | kc8;
            }
            t2[p] = lds_u64(lds, addr);
          }
          __builtin_memcpy(&dst[s], t2, 16);
        }
      };
      floatx4 acc[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[s] = floatx4{0.f, 0.f, 0.f, 0.f};
      half8 bop[2][4];
      key_operands(0, bop[0]);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        // lookups of step m+1 go out before the products of step m; the fences keep the
        // scheduler to this order so LDS latency hides behind four matrix instructions
        if (m + 1 < 8) key_operands(m + 1, bop[(m + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qop[m], bop[m & 1][s], acc[s], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // QJL: the sign-sketch products, acc2 = pq . (2 bits - 1) per row and token, and the two
      // norms of the lane's tokens, taken before the prefetch overwrites them
      floatx4 acc2[4];
      float nqf[4], rqf[4];
      if constexpr (QJL) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          acc2[s] = floatx4{0.f, 0.f, 0.f, 0.f};
          nqf[s] = f16(nq16[s]);
          rqf[s] = f16(rq16[s]);
        }
        const uint32_t c16 = kSgnBase + (uint32_t)(lane & 7) * 16u;
        auto sign_operand = [&](int kk, int s) {
          const uint4 w = *reinterpret_cast<const uint4 *>(lds + c16 + ((sgw[s] >> (8 * kk)) & 0xffu) * 128u);
          half8 bo;
          __builtin_memcpy(&bo, &w, 16);
          return bo;
        };
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          half8 sb[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) sb[s] = sign_operand(kk, s);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int s = 0; s < 4; ++s) acc2[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sop[kk], sb[s], acc2[s], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const uint32_t nk_pair = nkw;
      if (PREFETCH) load_keys(next_tile);

      // lane holds rows 4q..4q+3 (heads 2q, 2q+1; fp16 and remainder rows) of token 16s+m_row
      if (NH == 8 || quarter < 2) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int tok = 16 * s + m_row, p2 = tok >> 1, tb = tok & 1;
          float2 sv = make_float2(acc[s][0] + acc[s][1], acc[s][2] + acc[s][3]);
          if constexpr (QJL)  // ||k|| (R q).c + ||r|| pq.(2 bits - 1), the token's whole score
            sv = make_float2(fmaf(rqf[s], acc2[s][0] + acc2[s][1], nqf[s] * sv.x),
                             fmaf(rqf[s], acc2[s][2] + acc2[s][3], nqf[s] * sv.y));
          uint32_t off;
          if (NH == 4) off = score_unit<4>(p2, quarter) + tb * 8;
          else off = score_unit<8>(p2, 2 * (quarter >> 1) + tb) + (quarter & 1) * 8;
          *reinterpret_cast<float2 *>(wbuf + off) = sv;
        }
      }
      __builtin_amdgcn_wave_barrier();
      __asm__ volatile("" ::: "memory");
      float sc[2][NH2];  // [token bit][head slot]
      if constexpr (NH == 4) {
        const float4 r = *reinterpret_cast<const float4 *>(wbuf + score_unit<4>(pr, half_id));
        sc[0][0] = r.x; sc[0][1] = r.y; sc[1][0] = r.z; sc[1][1] = r.w;
      } else {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const float4 r = *reinterpret_cast<const float4 *>(wbuf + score_unit<8>(pr, 2 * half_id + tb));
          sc[tb][0] = r.x; sc[tb][1] = r.y; sc[tb][2] = r.z; sc[tb][3] = r.w;
        }
      }

      // ---- online softmax (base 2) for tokens t0 + 2pr + tb, heads half_id*NH2 + hh
      float nk[2], nv[2];
      nk[0] = f16((uint16_t)(nk_pair & 0xffffu));
      nk[1] = f16((uint16_t)(nk_pair >> 16));
      nv[0] = fmaxf(f16((uint16_t)(nvw & 0xffffu)), kNvFloor);
      nv[1] = fmaxf(f16((uint16_t)(nvw >> 16)), kNvFloor);
      if constexpr (!QJL) {  // (QJL scores carry their norms already)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int hh = 0; hh < NH2; ++hh) sc[tb][hh] *= nk[tb];
      }
      if (t0 + kTile > t_end) {  // ragged last tile of the split (uniform branch)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          if (t0 + 2 * pr + tb >= t_end) {
#pragma unroll
            for (int hh = 0; hh < NH2; ++hh) sc[tb][hh] = -INFINITY;
          }
      }
      // Rows of later query positions see more of the tile (uniform branch).  A row can then
      // have no visible token here while its reference is still -inf, where the plain
      // exponent below would give exp2(-inf - -inf): such tiles take the reference-move
      // path, whose exponents treat -inf explicitly.
      bool causal_tile = false;
      // Paged: a tile on a table entry of no page is not part of the sequence; its positions
      // leave the softmax (score -inf).  Like a causal tile it may meet a -inf reference, so it
      // takes the reference-move path (uniform branch).
      if (PAGED && tok == kNoPage) {
        causal_tile = true;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int hh = 0; hh < NH2; ++hh) sc[tb][hh] = -INFINITY;
      }
      if (MULTI && t0 + kTile > T - n_q + 1) {
        causal_tile = true;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int hh = 0; hh < NH2; ++hh)
            if (t0 + 2 * pr + tb > vlim[hh]) sc[tb][hh] = -INFINITY;
      }
      if constexpr (SPARSE) {
        // exact running maximum of the wave per head, sum relative to it; a token is a
        // candidate when some head's score reaches that maximum + log2(tau).  The maximum
        // only grows and never exceeds the final LSE, so every row the final weight keeps is
        // among the candidates.  (A bound shared by the workgroup's waves halves the
        // candidates but costs more per tile than the records it saves.)
        const float log2_tau = a.ln_tau * kLog2e;
        bool cand0 = false, cand1 = false;
#pragma unroll
        for (int hh = 0; hh < NH2; ++hh) {
          const float z = half_max(fmaxf(sc[0][hh], sc[1][hh]));
          if (a.tile_max != nullptr && pr == 0 && half_id * NH2 + hh < g)  // the tile's largest score
            a.tile_max[vrow(half_id * NH2 + hh) * a.tile_stride + (t0 >> 6)] = z;
          const float m_new = fmaxf(mr[hh], z);
          lsum[hh] = lsum[hh] * exp2_or_zero(mr[hh], m_new) + exp2_or_zero(sc[0][hh], m_new) +
                     exp2_or_zero(sc[1][hh], m_new);
          mr[hh] = m_new;
          if (RECORDS && half_id * NH2 + hh < g) {
            cand0 |= sc[0][hh] != -INFINITY && sc[0][hh] >= m_new + log2_tau;
            cand1 |= sc[1][hh] != -INFINITY && sc[1][hh] >= m_new + log2_tau;
          }
        }
        // token 2pr + tb is a candidate if either head half flags it; records are
        // {token, g scores (natural log)} at consecutive slots of the tile's second-pass split
        if (!RECORDS || a.cand == nullptr) { cand0 = false; cand1 = false; }  // key pass for the LSE only
        const uint64_t b0 = __ballot(cand0), b1 = __ballot(cand1);
        const uint32_t c0 = (uint32_t)b0 | (uint32_t)(b0 >> 32);
        const uint32_t c1 = (uint32_t)b1 | (uint32_t)(b1 >> 32);
        const int n0 = __popc(c0), n = n0 + __popc(c1);
        if (n > 0) {
          const int chunk = t0 / a.plan.split_len;
          int base = 0;
          if (lane == 0) base = atomicAdd(&chunk_count[chunk - c_first], n);
          base = __builtin_amdgcn_readfirstlane(base);
          float *cbase = a.cand + (((size_t)b * a.n_kv_heads + kvh) * a.plan.n_splits + chunk) *
                                      (size_t)a.plan.split_len * (1 + g);
          const uint32_t below = (1u << pr) - 1u;
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            const uint32_t cm = tb ? c1 : c0;
            if ((cm >> pr) & 1u) {
              const int slot = base + (tb ? n0 : 0) + __popc(cm & below);
              float *rec = cbase + (size_t)slot * (1 + g);
              if (half_id == 0) rec[0] = __int_as_float(t0 + 2 * pr + tb);
#pragma unroll
              for (int hh = 0; hh < NH2; ++hh) {
                const int h = half_id * NH2 + hh;
                if (h < g) rec[1 + h] = sc[tb][hh] * kLn2;
              }
            }
          }
        }
        if (a.scores != nullptr) {
#pragma unroll
          for (int hh = 0; hh < NH2; ++hh) {
            const int h = half_id * NH2 + hh;
            if (h < g) {
              float *row = a.scores + ((size_t)b * a.n_q_heads + qh0 + h) * a.ctx_len;
#pragma unroll
              for (int tb = 0; tb < 2; ++tb)
                if (t0 + 2 * pr + tb < t_end) row[t0 + 2 * pr + tb] = sc[tb][hh] * kLn2;
            }
          }
        }
        return;
      }
      float p[2][NH2];
      float vmax = 0.f;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int hh = 0; hh < NH2; ++hh) {
          p[tb][hh] = __builtin_amdgcn_exp2f(sc[tb][hh] - mr[hh]);
          vmax = fmaxf(vmax, p[tb][hh] * nv[tb]);
        }
      // (VMASK: the reference is the final LSE, so p <= 1 and never moves; P' is clamped to the
      // fp16 range below)
      if (!VMASK && (causal_tile || __any(!(vmax <= kAMax)))) {
        // move each head's reference to the tile's largest s + log2||v||, rescale
        float alpha[NH2];
#pragma unroll
        for (int hh = 0; hh < NH2; ++hh) {
          float z = fmaxf(sc[0][hh] == -INFINITY ? -INFINITY : sc[0][hh] + __log2f(nv[0]),
                          sc[1][hh] == -INFINITY ? -INFINITY : sc[1][hh] + __log2f(nv[1]));
          z = half_max(z);
          const float m_new = fmaxf(mr[hh], z);
          alpha[hh] = exp2_or_zero(mr[hh], m_new);
          mr[hh] = m_new;
          lsum[hh] *= alpha[hh];
          p[0][hh] = exp2_or_zero(sc[0][hh], m_new);
          p[1][hh] = exp2_or_zero(sc[1][hh], m_new);
        }
        // value rows 4q..4q+3 belong to heads 2q, 2q+1
        float al[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h)
          al[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[h % NH2]), (h / NH2) * 32));
        float a0 = al[0], a1 = al[1];
#pragma unroll
        for (int q = 1; q < NH / 2; ++q)
          if (quarter == q) { a0 = al[2 * q]; a1 = al[2 * q + 1]; }
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          oacc[n][0] *= a0; oacc[n][1] *= a0;
          oacc[n][2] *= a1; oacc[n][3] *= a1;
        }
      }
      if constexpr (!VMASK) {
#pragma unroll
        for (int hh = 0; hh < NH2; ++hh) lsum[hh] += p[0][hh] + p[1][hh];
      }

      if (a.scores != nullptr) {
#pragma unroll
        for (int hh = 0; hh < NH2; ++hh) {
          const int h = half_id * NH2 + hh;
          if (h < g) {
            float *row = a.scores + ((size_t)b * a.n_q_heads + qh0 + h) * a.ctx_len;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
              if (t0 + 2 * pr + tb < t_end) row[t0 + 2 * pr + tb] = sc[tb][hh] * kLn2;
          }
        }
      }

      if constexpr (VMASK) {  // no row of the tile reaches its head's threshold: no value work
        bool kept = false;
#pragma unroll
        for (int hh = 0; hh < NH2; ++hh) kept |= sc[0][hh] >= vthr[hh] || sc[1][hh] >= vthr[hh];
        if (!__any(kept)) return;
      }

      // ---- P' = p * ||v||: fp16 row 2h and remainder row 2h+1, token pair per 32-bit write
#pragma unroll
      for (int hh = 0; hh < NH2; ++hh) {
        const int h = half_id * NH2 + hh;
        float v0 = p[0][hh] * nv[0], v1 = p[1][hh] * nv[1];
        if constexpr (VMASK) {  // Sparse V: rows under the final-weight threshold add no value
          v0 = sc[0][hh] >= vthr[hh] ? fminf(v0, 65504.f) : 0.f;
          v1 = sc[1][hh] >= vthr[hh] ? fminf(v1, 65504.f) : 0.f;
        }
        half2v hi, lo;
        hi[0] = (_Float16)v0;
        hi[1] = (_Float16)v1;
        lo[0] = (_Float16)(v0 - (float)hi[0]);
        lo[1] = (_Float16)(v1 - (float)hi[1]);
        const uint32_t sub = (uint32_t)(pr & 3) * 4u;
        *reinterpret_cast<half2v *>(wbuf + pst_off<PB>(2 * h, pr >> 2) + sub) = hi;
        *reinterpret_cast<half2v *>(wbuf + pst_off<PB>(2 * h + 1, pr >> 2) + sub) = lo;
      }
      __builtin_amdgcn_wave_barrier();
      __asm__ volatile("" ::: "memory");

      // ---- O[row][coord] += P'[row][token] V[token][coord]
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint8_t *pa_src = W == 12 && !KEYS_ONLY && m_row >= 8 ? lds + kZeroBase + lane * 16
                                                      : wbuf + pst_off<PB>(m_row, 4 * c + quarter);
        const uint4 pa = *reinterpret_cast<const uint4 *>(pa_src);
        half8 aop;
        __builtin_memcpy(&aop, &pa, 16);
        auto value_operand = [&](int n) {
          const uint32_t w = vw[c][n >> 1];
          const uint32_t sel_lo = 0x0C020000u | ((4u + 2u * (n & 1)) << 8);
          const uint32_t sel_hi = 0x0C020000u | ((5u + 2u * (n & 1)) << 8);
          uint2 t2[2];
          t2[0] = lds_u64(lds, __builtin_amdgcn_perm(w, vc8, sel_lo));
          t2[1] = lds_u64(lds, __builtin_amdgcn_perm(w, vc8, sel_hi));
          half8 bo;
          __builtin_memcpy(&bo, t2, 16);
          return bo;
        };
        half8 vb[2];
        vb[0] = value_operand(0);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          if (n + 1 < 8) vb[(n + 1) & 1] = value_operand(n + 1);
          __builtin_amdgcn_sched_barrier(0);
          oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, vb[n & 1], oacc[n], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_wave_barrier();
      __asm__ volatile("" ::: "memory");
    };
    if constexpr (VMASK) {  // the wave's needed tiles only, the next one's keys prefetched
      uint64_t rem = need;
      if (rem != 0) {
        int tile = need_tile((int)__builtin_ctzll(rem));
        rem &= rem - 1;
        load_keys(tile);
        while (rem != 0) {
          const int next = need_tile((int)__builtin_ctzll(rem));
          rem &= rem - 1;
          tile_body(tile, next, std::true_type{});
          tile = next;
        }
        tile_body(tile, 0, std::false_type{});
      }
    } else if constexpr (PREFILL) {  // every tile of the split, for this wave's rows
      if (wave_on && n_tiles > 0) {
        int tile = 0;
        for (; tile + 1 < n_tiles; ++tile) tile_body(tile, tile + 1, std::true_type{});
        tile_body(tile, 0, std::false_type{});
      }
    } else {
      int tile = wave;
      for (; tile + W < n_tiles; tile += W) tile_body(tile, tile + W, std::true_type{});
      if (tile < n_tiles) tile_body(tile, 0, std::false_type{});
    }

    // Row h's output from its reference M, total l and rotated-domain sums (o0, o1) of the
    // lane's coordinates 2 lane, 2 lane + 1: normalise, inverse rotation, output and LSE.
    auto finish_row = [&](int h, float M, float l, float o0, float o1) {
      if (M != -INFINITY) {
        // (VMASK partials are final weights already); the value table's scale comes off here
        const float norm = VMASK ? 1.f / a.v.table_scale : 1.f / (a.v.table_scale * l);
        o0 *= norm;
        o1 *= norm;
      }
      // inverse rotation: x = s * (H y) / sqrt(128)
      float y0 = o0 + o1, y1 = o0 - o1;
      wave_fwht_upper(y0, y1, lane);
      y0 *= kInvSqrtD;
      y1 *= kInvSqrtD;
      if (sgn & 0x80u) y0 = -y0;  // the sign bytes loaded at set-up
      if (sgn & 0x8000u) y1 = -y1;
      const size_t orow = vrow(h);
      *reinterpret_cast<float2 *>(a.out + orow * kD + 2 * lane) = make_float2(y0, y1);
      if (lane == 0 && a.lse != nullptr)
        a.lse[orow] = VMASK ? lse_own : M == -INFINITY ? -INFINITY : (M + __log2f(l)) * kLn2;
      if (a.scores != nullptr) {
        float *row = a.scores + orow * a.ctx_len;
        for (int t = T + lane; t < a.ctx_len; t += 64) row[t] = -INFINITY;
      }
    };

    // The last workgroup (PREFILL: the last wave) of a (batch, kv head, row group) merges the
    // splits of row h: LSE merge of the partials, inverse rotation, output and LSE.
    auto merge_row = [&](int h) {
      // lane s of a chunk holds partial s's (m, l); every lane then sums its two
      // coordinates over the partials, 16 loads in flight at a time.  With at most 64 partials
      // (one per lane) each (m, l) is loaded once and the first 16 coordinate loads go out
      // with it, before the maximum is known: one memory round trip where the general loop
      // takes three.  Both add the partials in the same order.
      const size_t prow = vrow(h) * S;
      const float2 *pml = a.fpart_ml + prow;
      const float2 *pof = reinterpret_cast<const float2 *>(a.fpart_o + prow * kD) + lane;
      float o0 = 0.f, o1 = 0.f;
      auto load_o = [&](float2 (&o)[16], int base, int n) {
#pragma unroll
        for (int u = 0; u < 16; ++u)
          o[u] = base + u < n ? load_coherent(pof + (size_t)(base + u) * (kD / 2)) : make_float2(0.f, 0.f);
      };
      auto add_o = [&](const float2 (&o)[16], float w, int lane0) {  // partial lane0 + u is lane lane0 + u's
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), lane0 + u));
          o0 += o[u].x * wu;
          o1 += o[u].y * wu;
        }
      };
      float M = -INFINITY, l = 0.f;
      if (S <= 64) {
        const float2 ml = lane < S ? load_coherent(pml + lane) : make_float2(-INFINITY, 0.f);
        float2 o[16];
        load_o(o, 0, S);
        M = wave_reduce<true>(ml.x);
        if (M != -INFINITY) {
          const float w = exp2_or_zero(ml.x, M);
          l = ml.y * w;
          add_o(o, w, 0);
          for (int s = 16; s < S; s += 16) {
            load_o(o, s, S);
            add_o(o, w, s);
          }
        }
      } else {
        for (int s0 = 0; s0 < S; s0 += 64)
          if (s0 + lane < S) M = fmaxf(M, load_coherent(pml + s0 + lane).x);
        M = wave_reduce<true>(M);
        if (M != -INFINITY) {
          for (int s0 = 0; s0 < S; s0 += 64) {
            float w = 0.f;
            if (s0 + lane < S) {
              const float2 ml = load_coherent(pml + s0 + lane);
              w = exp2_or_zero(ml.x, M);
              l += ml.y * w;
            }
            const int n = min(64, S - s0);
            for (int s = 0; s < n; s += 16) {
              float2 o[16];
              load_o(o, s0 + s, s0 + n);
              add_o(o, w, s);
            }
          }
        }
      }
      if (M != -INFINITY) l = wave_reduce<false>(l);
      finish_row(h, M, l, o0, o1);
    };

    if constexpr (PREFILL) {
      // ---- this wave's rows alone: partials (m, l, O) per row, then its own arrival (with a
      //      single split, the rows' outputs directly)
      float ltot[NH2];
#pragma unroll
      for (int hh = 0; hh < NH2; ++hh) ltot[hh] = half_sum(lsum[hh]);
      __builtin_amdgcn_wave_barrier();
      __asm__ volatile("" ::: "memory");
      if (NH == 8 || quarter < 2) {  // O rows [head][128] fp32 (hi and remainder rows summed)
        const int h0 = 2 * quarter;
        float *dst0 = reinterpret_cast<float *>(wbuf) + h0 * kD + 8 * m_row;
        float *dst1 = dst0 + kD;
        *reinterpret_cast<float4 *>(dst0) = make_float4(oacc[0][0] + oacc[0][1], oacc[1][0] + oacc[1][1],
                                                        oacc[2][0] + oacc[2][1], oacc[3][0] + oacc[3][1]);
        *reinterpret_cast<float4 *>(dst0 + 4) = make_float4(oacc[4][0] + oacc[4][1], oacc[5][0] + oacc[5][1],
                                                            oacc[6][0] + oacc[6][1], oacc[7][0] + oacc[7][1]);
        *reinterpret_cast<float4 *>(dst1) = make_float4(oacc[0][2] + oacc[0][3], oacc[1][2] + oacc[1][3],
                                                        oacc[2][2] + oacc[2][3], oacc[3][2] + oacc[3][3]);
        *reinterpret_cast<float4 *>(dst1 + 4) = make_float4(oacc[4][2] + oacc[4][3], oacc[5][2] + oacc[5][3],
                                                            oacc[6][2] + oacc[6][3], oacc[7][2] + oacc[7][3]);
      }
      __builtin_amdgcn_wave_barrier();
      __asm__ volatile("" ::: "memory");
      if (!wave_on) return;
      if (S == 1) {  // the wave saw the whole context: no partials, no arrival, no merge
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          if (!vlive(h)) continue;
          const float mh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr[h % NH2]), (h / NH2) * 32));
          const float lh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ltot[h % NH2]), (h / NH2) * 32));
          const float2 o = *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(wbuf) + h * kD + 2 * lane);
          finish_row(h, mh, lh, o.x, o.y);
        }
        return;
      }
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        if (!vlive(h)) continue;
        const float mh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr[h % NH2]), (h / NH2) * 32));
        const float lh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ltot[h % NH2]), (h / NH2) * 32));
        const size_t prow = vrow(h) * S + split;
        const float2 o = *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(wbuf) + h * kD + 2 * lane);
        store_coherent(reinterpret_cast<float2 *>(a.fpart_o + prow * kD) + lane, o);
        if (lane == 0) store_coherent(a.fpart_ml + prow, make_float2(mh, lh));
      }
      // arrival of this wave's row group; the ordering is the workgroup arrival's below, for one
      // wave (its own vmcnt covers all of its partial stores)
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      unsigned *counter = a.counters + ((size_t)b * a.n_kv_heads + kvh) * VG + vgi;
      unsigned old = 0u;
      if (lane == 0) old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old = __builtin_amdgcn_readfirstlane(old);
      if (old == (unsigned)(S - 1)) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
          if (vlive(h)) merge_row(h);
        if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }

    // ---- combine the waves of the split.  First pass: (m, l) per head, 64 bytes per wave at
    //      the start of the key-table region (free once every wave is past its tiles), so
    //      that the second pass can write the staging buffers while other waves still read
    //      them.
    float ltot[NH2];
#pragma unroll
    for (int hh = 0; hh < NH2; ++hh) ltot[hh] = half_sum(lsum[hh]);
    __syncthreads();  // every wave is done with its staging buffers
    if (pr == 0) {
#pragma unroll
      for (int hh = 0; hh < NH2; ++hh)
        *reinterpret_cast<float2 *>(lds + wave * 64 + (half_id * NH2 + hh) * 8) = make_float2(mr[hh], ltot[hh]);
    }
    __syncthreads();
    // scale of this wave's value rows (heads 2q, 2q+1) and, for the summing phase, the
    // split's reference and sum of head `wave` (thread (wave, lane) sums coords 2l, 2l+1)
    float f0 = 0.f, f1 = 0.f, Mh = -INFINITY, Lh = 0.f;
    {
      const int h0 = NH == 8 ? 2 * quarter : 2 * (quarter & 1);
      float M0 = -INFINITY, M1 = -INFINITY;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float *src = reinterpret_cast<const float *>(lds + w * 64);
        M0 = fmaxf(M0, src[2 * h0]);
        M1 = fmaxf(M1, src[2 * (h0 + 1)]);
        if (wave < NH) Mh = fmaxf(Mh, src[2 * wave]);
      }
      const float *own = reinterpret_cast<const float *>(lds + wave * 64);
      f0 = exp2_or_zero(own[2 * h0], M0);
      f1 = exp2_or_zero(own[2 * (h0 + 1)], M1);
      if (wave < NH) {
#pragma unroll
        for (int w = 0; w < W; ++w) {
          const float *src = reinterpret_cast<const float *>(lds + w * 64);
          Lh += src[2 * wave + 1] * exp2_or_zero(src[2 * wave], Mh);
        }
      }
    }
    if constexpr (SPARSE) {
      // the split's (m, l) per query head in natural-log units, and the candidate counts;
      // the value pass and the merge are separate kernels
      if (wave < NH && vlive(wave) && lane == 0)
        a.fpart_ml[vrow(wave) * S + split] =
            make_float2(Mh == -INFINITY ? -INFINITY : Mh * kLn2, Lh);
      for (int i = threadIdx.x; RECORDS && i < n_chunks && a.cand_count != nullptr; i += blockDim.x)
        if (c_first + i < a.plan.n_splits)
          a.cand_count[((size_t)b * a.n_kv_heads + kvh) * a.plan.n_splits + c_first + i] = chunk_count[i];
      return;
    }
    // Second pass: scaled O rows of this wave, [head][128] fp32 (hi and remainder rows summed)
    if (NH == 8 || quarter < 2) {
      const int h0 = 2 * quarter;
      float *dst0 = reinterpret_cast<float *>(wbuf) + h0 * kD + 8 * m_row;
      float *dst1 = dst0 + kD;
      *reinterpret_cast<float4 *>(dst0) = make_float4((oacc[0][0] + oacc[0][1]) * f0, (oacc[1][0] + oacc[1][1]) * f0,
                                                      (oacc[2][0] + oacc[2][1]) * f0, (oacc[3][0] + oacc[3][1]) * f0);
      *reinterpret_cast<float4 *>(dst0 + 4) = make_float4((oacc[4][0] + oacc[4][1]) * f0, (oacc[5][0] + oacc[5][1]) * f0,
                                                          (oacc[6][0] + oacc[6][1]) * f0, (oacc[7][0] + oacc[7][1]) * f0);
      *reinterpret_cast<float4 *>(dst1) = make_float4((oacc[0][2] + oacc[0][3]) * f1, (oacc[1][2] + oacc[1][3]) * f1,
                                                      (oacc[2][2] + oacc[2][3]) * f1, (oacc[3][2] + oacc[3][3]) * f1);
      *reinterpret_cast<float4 *>(dst1 + 4) = make_float4((oacc[4][2] + oacc[4][3]) * f1, (oacc[5][2] + oacc[5][3]) * f1,
                                                          (oacc[6][2] + oacc[6][3]) * f1, (oacc[7][2] + oacc[7][3]) * f1);
    }
    __syncthreads();
    const bool live_w = wave < NH && vlive(wave);
    const size_t part_row = vrow(live_w ? wave : 0) * S;  // valid for live_w
    if (live_w) {
      float2 o = make_float2(0.f, 0.f);
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float2 x = *reinterpret_cast<const float2 *>(lds + kWBase + w * WSTRIDE + (wave * kD + 2 * lane) * 4);
        o.x += x.x;
        o.y += x.y;
      }
      store_coherent(reinterpret_cast<float2 *>(a.fpart_o + (part_row + split) * kD) + lane, o);
      if (lane == 0) store_coherent(a.fpart_ml + part_row + split, make_float2(Mh, Lh));
    }

    // ---- arrival; the last workgroup of this (batch, kv head) merges its splits.  Ordering,
    //      on the hardware's terms: (1) each partial is an agent-scope atomic store, which
    //      writes through the XCD's L2 to the device-coherent level; (2) each wave waits for
    //      vmcnt(0), which for such a store means the coherent level has acknowledged it (a
    //      wave's vmcnt counts only its own operations, so every wave waits); (3) the barrier
    //      puts all of that before thread 0's counter increment, a device-coherent atomic; (4)
    //      the workgroup that reads the final count then reads the partials with agent-scope
    //      atomic loads, which bypass its L2 and read the coherent level.  So every partial is
    //      at the coherent level before any read of it.  The language-level form, a release
    //      increment and an acquire in the last workgroup, writes back the XCD's L2 in every
    //      workgroup: +3.5 us at 8192 tokens, +10 us on the batched 32768-token workload in a
    //      same-box comparison, so the kernel keeps the hardware ordering.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    int *flag = reinterpret_cast<int *>(lds + kWBase);
    unsigned *counter = a.counters + ((size_t)b * a.n_kv_heads + kvh) * VG + vgi;
    if (threadIdx.x == 0) {
      const unsigned old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *flag = old == (unsigned)(S - 1) ? 1 : 0;
    }
    __syncthreads();
    const bool last = *flag != 0;
    if (last) {
      if (live_w) {
        merge_row(wave);
      }
      if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int BK, int NH, bool SPARSE, bool MULTI, bool APPEND, bool PAGED, bool VMASK, bool RECORDS, bool PREFILL,
          bool QJL, int W>
__global__ __launch_bounds__(64 * W, 1) void decode_fused_kernel(DecodeArgs a) {
  decode_fused_body<BK, NH, SPARSE, MULTI, APPEND, PAGED, VMASK, RECORDS, PREFILL, QJL, W>(a);
}

// Splits of at least this many tokens run single-query decode with wider workgroups (12
// waves for up to 4 heads per kv head; the key-only pass 16 or 12); shorter ones (a wave
// would have few tiles) keep 8.
constexpr int kWideMinSplit = 48 * kTile;

template <int BK, bool SPARSE, bool MULTI, bool APPEND, bool PAGED = false, bool VMASK = false, bool RECORDS = true,
          bool PREFILL = false, bool QJL = false>
hipError_t launch_nh(const DecodeArgs &a, int grid, hipStream_t stream) {
  constexpr bool kKeysOnly = SPARSE && !RECORDS;
  constexpr bool kCanWide = !(MULTI || VMASK || PREFILL || QJL) && (!SPARSE || kKeysOnly);
  const bool wide = kCanWide && a.fplan.split_len >= kWideMinSplit;
  if (a.vg_size <= 4) {
    if constexpr (kCanWide) {
      if (wide) {
        constexpr int W4 = kKeysOnly ? 16 : 12;
        decode_fused_kernel<BK, 4, SPARSE, MULTI, APPEND, PAGED, VMASK, RECORDS, PREFILL, QJL, W4>
            <<<grid, 64 * W4, 0, stream>>>(a);
        return hipGetLastError();
      }
    }
    decode_fused_kernel<BK, 4, SPARSE, MULTI, APPEND, PAGED, VMASK, RECORDS, PREFILL, QJL, kWaves>
        <<<grid, kThreads, 0, stream>>>(a);
  } else {
    if constexpr (kCanWide && kKeysOnly) {
      if (wide) {
        decode_fused_kernel<BK, 8, SPARSE, MULTI, APPEND, PAGED, VMASK, RECORDS, PREFILL, QJL, 12>
            <<<grid, 64 * 12, 0, stream>>>(a);
        return hipGetLastError();
      }
    }
    decode_fused_kernel<BK, 8, SPARSE, MULTI, APPEND, PAGED, VMASK, RECORDS, PREFILL, QJL, kWaves>
        <<<grid, kThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

template <int BK, bool SPARSE>
hipError_t launch_bk(const DecodeArgs &a, int grid, hipStream_t stream) {
  if (!SPARSE && a.prefill) return launch_nh<BK, false, true, false, false, false, true, true>(a, grid, stream);
  if (!SPARSE && (a.n_q > 1 || a.vgroups > 1) && a.xk != nullptr) {
    if (a.n_q > kMultiAppendMax) return hipErrorInvalidValue;
    return launch_nh<BK, false, true, true>(a, grid, stream);  // the n_q new tokens written first
  }
  if (!SPARSE && (a.n_q > 1 || a.vgroups > 1)) return launch_nh<BK, false, true, false>(a, grid, stream);
  if (!SPARSE && a.xk != nullptr) return launch_nh<BK, false, false, true>(a, grid, stream);
  return launch_nh<BK, SPARSE, false, false>(a, grid, stream);
}

}  // namespace

bool decode_fused_shape_ok(const DecodeArgs &a) {
  return !a.sparse && (a.k.bits == 3 || a.k.bits == 4) && a.v.bits == 2 && a.vg_size <= 8 && a.vg_size >= 1 &&
         a.k.layout == TQ_LAYOUT_ROWS && a.v.layout == TQ_LAYOUT_GROUP8 && a.fplan.split_len % kTile == 0;
}

bool decode_fused_supported(const DecodeArgs &a) { return decode_fused_shape_ok(a) && a.counters != nullptr; }

hipError_t launch_decode_fused(const DecodeArgs &a, int n_cu, hipStream_t stream) {
  (void)n_cu;
  // prefill: one workgroup per 8 row groups (one per wave)
  const long vg_items = a.prefill ? (a.vgroups + kWaves - 1) / kWaves : a.vgroups;
  const long units = (long)a.batch * a.n_kv_heads * a.fplan.n_splits;
  // several row-group items per unit: units padded to a multiple of 8 (XCD grouping)
  const long items = vg_items > 1 ? vg_items * ((units + 7) / 8) * 8 : units;
  if (items < 1 || items > 0x7fffffffL) return hipErrorInvalidValue;
  const int grid = (int)items;
  return a.k.bits == 4 ? launch_bk<4, false>(a, grid, stream) : launch_bk<3, false>(a, grid, stream);
}

bool decode_fused_sparse_supported(const DecodeArgs &a) {
  return a.sparse && a.n_q == 1 && a.vgroups == 1 && (a.k.bits == 3 || a.k.bits == 4) && a.group <= 8 &&
         a.k.layout == TQ_LAYOUT_ROWS && a.v.layout == TQ_LAYOUT_GROUP8 &&
         a.plan.split_len % kTile == 0 && a.fplan.split_len % a.plan.split_len == 0 &&
         a.fplan.split_len / a.plan.split_len <= kMaxChunksPerSplit;
}

hipError_t launch_decode_fused_paged(const DecodeArgs &a, hipStream_t stream) {
  if (a.block_table == nullptr || a.seq_lens == nullptr || a.fplan.split_len > kPagedMaxSplit ||
      a.k.capacity % kTile != 0 || a.v.capacity != a.k.capacity || !decode_fused_supported(a) ||
      (a.prefill && a.fplan.split_len > kPagedPrefillMaxSplit))
    return hipErrorInvalidValue;
  if (a.prefill) {  // a chunk of positions: one workgroup per 8 row groups (one per wave)
    if (a.xk != nullptr) return hipErrorInvalidValue;
    const long vg_items = (a.vgroups + kWaves - 1) / kWaves;
    const long units = (long)a.batch * a.n_kv_heads * a.fplan.n_splits;
    const long items = vg_items > 1 ? vg_items * ((units + 7) / 8) * 8 : units;
    if (items < 1 || items > 0x7fffffffL) return hipErrorInvalidValue;
    return a.k.bits == 4 ? launch_nh<4, false, true, false, true, false, true, true>(a, (int)items, stream)
                         : launch_nh<3, false, true, false, true, false, true, true>(a, (int)items, stream);
  }
  if (a.n_q > 1 || a.vgroups > 1) {  // several query positions (one row group per work item)
    if (a.xk != nullptr) return hipErrorInvalidValue;
    const long units = (long)a.batch * a.n_kv_heads * a.fplan.n_splits;
    const long items = a.vgroups > 1 ? (long)a.vgroups * ((units + 7) / 8) * 8 : units;
    if (items < 1 || items > 0x7fffffffL) return hipErrorInvalidValue;
    return a.k.bits == 4 ? launch_nh<4, false, true, false, true>(a, (int)items, stream)
                         : launch_nh<3, false, true, false, true>(a, (int)items, stream);
  }
  const long items = (long)a.batch * a.n_kv_heads * a.fplan.n_splits;
  if (items < 1 || items > 0x7fffffffL) return hipErrorInvalidValue;
  if (a.xk != nullptr)  // append the new token in the same launch
    return a.k.bits == 4 ? launch_nh<4, false, false, true, true>(a, (int)items, stream)
                         : launch_nh<3, false, false, true, true>(a, (int)items, stream);
  return a.k.bits == 4 ? launch_nh<4, false, false, false, true>(a, (int)items, stream)
                       : launch_nh<3, false, false, false, true>(a, (int)items, stream);
}

// Sparse V over paged caches: the key pass without records, then the masked value pass, both
// reading the pages through the block table (splits of at most kPagedMaxSplit tokens).
hipError_t launch_decode_fused_paged_sparse(const DecodeArgs &key_pass, const DecodeArgs &value_pass,
                                            hipStream_t stream) {
  const DecodeArgs &a = key_pass, &v = value_pass;
  if (a.block_table == nullptr || a.seq_lens == nullptr || a.fplan.split_len > kPagedMaxSplit ||
      v.fplan.split_len > kVmaskMaxSplit || a.k.capacity % kTile != 0 || a.v.capacity != a.k.capacity ||
      (a.k.bits != 3 && a.k.bits != 4) || a.v.bits != 2 || a.vg_size > 8 || a.tile_max == nullptr ||
      v.lse_ml == nullptr || v.counters == nullptr)
    return hipErrorInvalidValue;
  const long items_k = (long)a.batch * a.n_kv_heads * a.fplan.n_splits;
  const long items_v = (long)v.batch * v.n_kv_heads * v.fplan.n_splits;
  if (items_k < 1 || items_k > 0x7fffffffL || items_v < 1 || items_v > 0x7fffffffL) return hipErrorInvalidValue;
  hipError_t e = a.k.bits == 4 ? launch_nh<4, true, false, false, true, false, false>(a, (int)items_k, stream)
                               : launch_nh<3, true, false, false, true, false, false>(a, (int)items_k, stream);
  if (e != hipSuccess) return e;
  return v.k.bits == 4 ? launch_nh<4, false, false, false, true, true>(v, (int)items_v, stream)
                       : launch_nh<3, false, false, false, true, true>(v, (int)items_v, stream);
}

bool decode_fused_qjl_supported(const DecodeArgs &a) {
  return decode_fused_supported(a) && a.k.bits == 3 && a.n_q == 1 && a.vgroups == 1 && a.xk == nullptr &&
         a.block_table == nullptr && a.qjl_bits != nullptr && a.qjl_rnorm != nullptr && a.qjl_proj != nullptr &&
         a.qjl_m == kD;
}

bool decode_fused_qjl_sparse_supported(const DecodeArgs &a) {
  return decode_fused_sparse_supported(a) && a.k.bits == 3 && a.v.bits == 2 && a.xk == nullptr &&
         a.block_table == nullptr && a.qjl_bits != nullptr && a.qjl_rnorm != nullptr && a.qjl_proj != nullptr &&
         a.qjl_m == kD && a.cand == nullptr && a.tile_max != nullptr;
}

// Sparse V with QJL keys: the key pass (LSE partials and tile maxima, QJL-corrected scores),
// then the masked value pass, which recomputes the QJL scores of the tiles it needs.
hipError_t launch_decode_fused_qjl_sparse(const DecodeArgs &key_pass, const DecodeArgs &value_pass,
                                          hipStream_t stream) {
  const DecodeArgs &a = key_pass, &v = value_pass;
  if (!decode_fused_qjl_sparse_supported(a) || !decode_fused_supported(v) || v.lse_ml == nullptr ||
      v.lse_splits < 1 || v.tile_max == nullptr || v.fplan.split_len > kVmaskMaxSplit)
    return hipErrorInvalidValue;
  const long items_k = (long)a.batch * a.n_kv_heads * a.fplan.n_splits;
  const long items_v = (long)v.batch * v.n_kv_heads * v.fplan.n_splits;
  if (items_k < 1 || items_k > 0x7fffffffL || items_v < 1 || items_v > 0x7fffffffL) return hipErrorInvalidValue;
  const hipError_t e = launch_nh<3, true, false, false, false, false, false, false, true>(a, (int)items_k, stream);
  if (e != hipSuccess) return e;
  return launch_nh<3, false, false, false, false, true, true, false, true>(v, (int)items_v, stream);
}

hipError_t launch_decode_fused_qjl(const DecodeArgs &a, hipStream_t stream) {
  if (!decode_fused_qjl_supported(a)) return hipErrorInvalidValue;
  const long items = (long)a.batch * a.n_kv_heads * a.fplan.n_splits;
  if (items < 1 || items > 0x7fffffffL) return hipErrorInvalidValue;
  return launch_nh<3, false, false, false, false, false, true, false, true>(a, (int)items, stream);
}

hipError_t launch_decode_fused_vmask(const DecodeArgs &a, hipStream_t stream) {
  // one lane per tile decides which tiles a wave needs: at most 64 tiles per wave
  if (!decode_fused_supported(a) || a.lse_ml == nullptr || a.lse_splits < 1 || a.tile_max == nullptr ||
      a.fplan.split_len > kVmaskMaxSplit)
    return hipErrorInvalidValue;
  const long items = (long)a.batch * a.n_kv_heads * a.fplan.n_splits;
  if (items < 1 || items > 0x7fffffffL) return hipErrorInvalidValue;
  return a.k.bits == 4 ? launch_nh<4, false, false, false, false, true>(a, (int)items, stream)
                       : launch_nh<3, false, false, false, false, true>(a, (int)items, stream);
}

hipError_t launch_decode_fused_sparse(const DecodeArgs &a, hipStream_t stream) {
  const long items = (long)a.batch * a.n_kv_heads * a.fplan.n_splits;
  if (items < 1 || items > 0x7fffffffL) return hipErrorInvalidValue;
  if (a.cand == nullptr && a.xk != nullptr)  // the same, the decode step's new token written first
    return a.k.bits == 4 ? launch_nh<4, true, false, true, false, false, false>(a, (int)items, stream)
                         : launch_nh<3, true, false, true, false, false, false>(a, (int)items, stream);
  if (a.xk != nullptr) return hipErrorInvalidValue;  // (appends go with the key-only pass alone)
  if (a.cand == nullptr)  // the LSE and tile maxima only (before the masked value pass)
    return a.k.bits == 4 ? launch_nh<4, true, false, false, false, false, false>(a, (int)items, stream)
                         : launch_nh<3, true, false, false, false, false, false>(a, (int)items, stream);
  return a.k.bits == 4 ? launch_bk<4, true>(a, (int)items, stream) : launch_bk<3, true>(a, (int)items, stream);
}

}  // namespace tq

"""CPU oracle for TurboQuant KV-cache compression and compressed decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only the tests, the smoke check of the build entry point and the CPU-baseline
leg of the benchmark may use it.  It shares no code with the HIP library.

Everything here is plain and slow on purpose: fp64 throughout, a dense rotation
matrix, brute-force nearest-codeword search, a bit loop for packing and a full
(two-pass) softmax.  Each function names the passage of the source pages it
follows.  Page keys used in citations:

  [inferrs]  "inferrs & TurboQuant：本地 LLM 推理的内存革命"
  [tq-80]    "TurboQuant：让大模型本地推理内存占用降低80%的KV缓存压缩技术"
  [tq-plus]  "TurboQuant+：跨平台KV缓存压缩技术助力本地LLM高效推理"
  [tq-fwht]  "TurboQuant：用Rust核心与FWHT预处理实现LLM推理的4-bit KV缓存量化"
  [google]   "Google 最新極限壓縮算法，砸碎大模型本地部署的內存墻，8 倍提升！"

Readings of points the pages leave open (each is listed in the design notes):
  * rotation R = H diag(s) / sqrt(d), H the Sylvester-ordered Hadamard matrix;
  * codebook = Lloyd-Max quantizer of the density (1 - x^2)^((d-3)/2) on [-1, 1]
    (the marginal of one coordinate of a uniformly random unit vector, which the
    [tq-80] page describes as a Beta law), centroids ascending;
  * code index = number of boundaries strictly below u (ties go to the lower
    index), boundaries are the midpoints of adjacent centroids;
  * u is normalised by the full-precision norm; the stored norm is its fp16
    round-to-nearest-even value; a zero vector gives u = 0;
  * packing is an LSB-first bit stream (see `code_bit_positions`);
  * Sparse V keeps row t for head h iff the final normalised softmax weight
    p_{h,t} >= tau, without renormalisation;
  * inner-product search ranks database vectors by q . x_hat (their dequantized
    vectors), descending, equal scores by ascending index.

Parity status: every function here is pinned by a test in tests/ against
closed forms, a library routine or brute force, except the end-to-end outputs
on the synthetic workloads, which no page prints (parity unpinned beyond the
oracle for those values).
"""
from __future__ import annotations

import functools
import math

import numpy as np

# ---------------------------------------------------------------------------
# Codebook: Lloyd iteration on a known density  ([tq-80] §核心创新, §tqai项目)
# ---------------------------------------------------------------------------

_GL_NODES, _GL_WEIGHTS = np.polynomial.legendre.leggauss(20)


def rotated_coordinate_density(d: int):
    """Unnormalised density of one coordinate of a random unit vector in R^d.

    [tq-80] §核心创新 states that after the random orthogonal rotation the
    coordinates follow a concentrated Beta law.  For a uniform point on the
    sphere S^{d-1} one coordinate x has density proportional to
    (1 - x^2)^((d-3)/2) on [-1, 1] (that is, (x+1)/2 ~ Beta((d-1)/2, (d-1)/2)).
    """
    alpha = (d - 3) / 2.0

    def f(x):
        x = np.asarray(x, dtype=np.float64)
        return np.power(np.clip(1.0 - x * x, 0.0, None), alpha)

    return f


def cell_integrals(f, edges, max_piece=0.01):
    """Mass and first moment of density f over consecutive cells [edges[k], edges[k+1]].

    Plain composite Gauss-Legendre quadrature: every cell is split into pieces of
    width at most `max_piece`, 20 nodes per piece.
    """
    edges = np.asarray(edges, dtype=np.float64)
    a, b = edges[:-1], edges[1:]
    width = b - a
    npieces = np.maximum(1, np.ceil(width / max_piece).astype(np.int64))
    cell_of_piece = np.repeat(np.arange(len(a)), npieces)
    first_piece = np.concatenate(([0], np.cumsum(npieces)[:-1]))
    j = np.arange(cell_of_piece.size) - np.repeat(first_piece, npieces)
    pw = (width / npieces)[cell_of_piece]
    pa = a[cell_of_piece] + j * pw
    mid = pa + 0.5 * pw
    half = 0.5 * pw
    x = mid[:, None] + half[:, None] * _GL_NODES[None, :]
    fx = f(x)
    w = half[:, None] * _GL_WEIGHTS[None, :]
    mass_p = (fx * w).sum(axis=1)
    mom_p = (x * fx * w).sum(axis=1)
    mass = np.add.reduceat(mass_p, first_piece)
    mom = np.add.reduceat(mom_p, first_piece)
    return mass, mom


def lloyd_max(f, lo: float, hi: float, init, tol: float, max_iter: int = 1_000_000,
              max_piece: float = 0.01):
    """Lloyd's algorithm for the scalar quantizer minimising E (x - Q(x))^2 under f.

    Alternates the two Lloyd-Max optimality conditions:
      boundaries t_j = (c_j + c_{j+1}) / 2          (nearest-neighbour cells)
      centroids  c_k = E[x | t_{k-1} < x < t_k]     (centroid condition)
    until the largest centroid move is below `tol`.
    Returns (centroids, boundaries, iterations).
    """
    c = np.array(init, dtype=np.float64)
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([lo], t, [hi]))
        mass, mom = cell_integrals(f, edges, max_piece)
        c_new = mom / mass
        step = float(np.max(np.abs(c_new - c)))
        c = c_new
        if step < tol:
            break
    return c, 0.5 * (c[:-1] + c[1:]), it


def gaussian_quantile_init(d: int, levels: int):
    """Initial centroids: quantiles of N(0, 1/d) at (k + 1/2) / L."""
    from scipy.special import ndtri

    k = np.arange(levels, dtype=np.float64)
    return ndtri((k + 0.5) / levels) / math.sqrt(d)


def make_codebook(d: int, bits: int, init: str = "gauss"):
    """Data-independent Lloyd-Max codebook for b-bit codes at head dim d.

    [tq-80] §核心创新 and §tqai项目: the codebook is derived from the known
    distribution of the rotated coordinates, precomputed, and shared by every
    model.  The result is symmetrised (c_k = -c_{L-1-k}), which is exact for the
    even density and makes the middle boundary exactly 0.
    """
    levels = 1 << bits
    f = rotated_coordinate_density(d)
    if init == "gauss":
        c0 = gaussian_quantile_init(d, levels)
    elif init == "uniform":
        c0 = (np.arange(levels) + 0.5) / levels * 2.0 - 1.0
        c0 *= 4.0 / math.sqrt(d)
    else:
        raise ValueError(init)
    # 8-bit Lloyd converges slowly (ratio close to 1): a 1e-13 step still leaves
    # about 7e-10 of error, so the 8-bit table runs to a 1e-15 step.
    tol = 1e-15 if bits >= 8 else 1e-14
    c, _, it = lloyd_max(f, -1.0, 1.0, c0, tol)
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    return c, t, it


def codebook_distortion(d: int, centroids) -> float:
    """d * E (u_i - Q(u_i))^2 = expected squared error of a whole unit vector.

    Quadrature over the Lloyd cells of the normalised density.
    """
    c = np.asarray(centroids, dtype=np.float64)
    f = rotated_coordinate_density(d)
    t = 0.5 * (c[:-1] + c[1:])
    edges = np.concatenate(([-1.0], t, [1.0]))
    z, _ = cell_integrals(f, np.array([-1.0, 1.0]))
    total = 0.0
    for k in range(len(c)):
        g = lambda x, ck=c[k]: (np.asarray(x) - ck) ** 2 * f(x)
        m, _ = cell_integrals(g, edges[k:k + 2])
        total += float(m[0])
    return d * total / float(z[0])


# ---------------------------------------------------------------------------
# Rotation  ([inferrs] §核心技术; [tq-fwht] §2 FWHT 预处理)
# ---------------------------------------------------------------------------

@functools.lru_cache(maxsize=None)
def hadamard(d: int) -> np.ndarray:
    """Sylvester-ordered Hadamard matrix, H[i, j] = (-1)^popcount(i & j).  Built once per d
    (entry by entry) and returned read-only."""
    h = np.empty((d, d), dtype=np.float64)
    for i in range(d):
        for j in range(d):
            h[i, j] = -1.0 if bin(i & j).count("1") % 2 else 1.0
    h.setflags(write=False)
    return h


def rotation_matrix(signs) -> np.ndarray:
    """Dense random-sign Walsh-Hadamard rotation R = H diag(s) / sqrt(d).

    [inferrs] §核心技术 names a Walsh-Hadamard rotation applied before
    quantization; [tq-fwht] §2 says it is orthogonal and exactly invertible.
    The random signs s are an input (drawn by the caller from a seed).
    """
    s = np.asarray(signs, dtype=np.float64)
    d = s.size
    return hadamard(d) * s[None, :] / math.sqrt(d)


def rotate(x, signs) -> np.ndarray:
    """y = R x for row vectors x[..., d], applying the factors of R in order:
    sign flip, integer Hadamard product, then 1/sqrt(d).  (Applying them in this
    order keeps exact zeros exact, e.g. for x = all-ones.)"""
    s = np.asarray(signs, dtype=np.float64)
    d = s.size
    return ((np.asarray(x, dtype=np.float64) * s) @ hadamard(d).T) / math.sqrt(d)


def unrotate(y, signs) -> np.ndarray:
    """x = R^T y = diag(s) H y / sqrt(d) for row vectors y[..., d]."""
    s = np.asarray(signs, dtype=np.float64)
    d = s.size
    return s * ((np.asarray(y, dtype=np.float64) @ hadamard(d)) / math.sqrt(d))


# ---------------------------------------------------------------------------
# Quantization  ([tq-80] §核心创新; [inferrs] §压缩格式对比)
# ---------------------------------------------------------------------------

def fp16_round(x) -> np.ndarray:
    """IEEE binary16 round-to-nearest-even of fp64 values (returned as float16)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def nearest_code_bruteforce(u, centroids) -> np.ndarray:
    """argmin_k |u - c_k|, ties to the lower index (brute force over all levels)."""
    u = np.asarray(u, dtype=np.float64)
    c = np.asarray(centroids, dtype=np.float64)
    dist = np.abs(u[..., None] - c)
    best = dist.min(axis=-1, keepdims=True)
    return np.argmax(dist <= best, axis=-1).astype(np.int64)


def code_by_boundaries(u, boundaries) -> np.ndarray:
    """Number of boundaries strictly below u (nearest centroid, ties low)."""
    return np.searchsorted(np.asarray(boundaries, dtype=np.float64),
                           np.asarray(u, dtype=np.float64), side="left").astype(np.int64)


def quantize(x, signs, centroids, boundaries, method: str = "boundaries"):
    """Quantize head vectors x[..., d] (fp64 values).

    Steps ([tq-80] §核心创新): n = ||x||_2; the norm is kept as fp16; the
    direction u = R x / n is rotated and each coordinate is mapped to its nearest
    codeword.  Returns (codes int64 [..., d], norms float16 [...], u fp64 [..., d]).
    """
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1))
    y = rotate(x, signs)
    safe = np.where(n > 0, n, 1.0)
    u = np.where((n > 0)[..., None], y / safe[..., None], 0.0)
    if method == "bruteforce":
        codes = nearest_code_bruteforce(u, centroids)
    else:
        codes = code_by_boundaries(u, boundaries)
    return codes, fp16_round(n), u


def near_boundary_mask(u, boundaries, band: float = 1e-6) -> np.ndarray:
    """Coordinates whose rotated value lies within `band` of a boundary.

    The band is an absolute distance in unit-vector coordinates, |u_i - t_j| <= band for
    some boundary t_j (the plain reading of "within 1e-6 of a codebook boundary"), taken
    on the oracle's fp64 u.  A code on either side of such a boundary is accepted."""
    u = np.asarray(u, dtype=np.float64)
    t = np.asarray(boundaries, dtype=np.float64)
    return (np.abs(u[..., None] - t) <= band).any(axis=-1)


# ---------------------------------------------------------------------------
# Bit packing  ([google] mlx-vlm kernel list: pack / unpack of low-bit codes)
# ---------------------------------------------------------------------------

LAYOUT_ROWS = 0     # token-major: one contiguous LSB-first row per vector
LAYOUT_GROUP8 = 1   # groups of 8 tokens, coordinate-major inside a group


def code_bit_positions(n_tokens: int, d: int, bits: int, layout: int) -> np.ndarray:
    """Bit offset of bit k of code (t, i) inside one (batch, kv-head) code plane.

    LAYOUT_ROWS:   t*d*b + i*b + k                 (vector t is one LSB-first row)
    LAYOUT_GROUP8: (t//8)*d*8*b + (i*8 + t%8)*b + k (codes of 8 consecutive tokens
                   for one coordinate are adjacent)
    Returns int64 array [n_tokens, d, bits].
    """
    t = np.arange(n_tokens)[:, None, None]
    i = np.arange(d)[None, :, None]
    k = np.arange(bits)[None, None, :]
    if layout == LAYOUT_ROWS:
        return t * d * bits + i * bits + k
    if layout == LAYOUT_GROUP8:
        return (t // 8) * d * 8 * bits + (i * 8 + t % 8) * bits + k
    raise ValueError(layout)


def pack(codes, bits: int, layout: int = LAYOUT_ROWS) -> np.ndarray:
    """Pack codes [T, d] into T*d*b/8 bytes: bit k of a code goes to its bit offset,
    byte = offset >> 3, bit-in-byte = offset & 7 (LSB first)."""
    codes = np.asarray(codes, dtype=np.int64)
    n_tokens, d = codes.shape
    if layout == LAYOUT_GROUP8 and n_tokens % 8:
        raise ValueError("LAYOUT_GROUP8 needs a multiple of 8 tokens")
    pos = code_bit_positions(n_tokens, d, bits, layout)
    bitval = (codes[:, :, None] >> np.arange(bits)[None, None, :]) & 1
    out = np.zeros(n_tokens * d * bits // 8, dtype=np.uint8)
    on = pos[bitval == 1]
    np.bitwise_or.at(out, on >> 3, (1 << (on & 7)).astype(np.uint8))
    return out


def unpack(packed, n_tokens: int, d: int, bits: int, layout: int = LAYOUT_ROWS) -> np.ndarray:
    """Inverse of `pack`: codes [T, d] (int64)."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    pos = code_bit_positions(n_tokens, d, bits, layout)
    bitval = (packed[pos >> 3] >> (pos & 7)) & 1
    return (bitval.astype(np.int64) << np.arange(bits)[None, None, :]).sum(axis=-1)


def packed_bytes_per_vector(d: int, bits: int) -> int:
    """Bytes per cached vector: d*b/8 code bytes plus a 2-byte fp16 norm."""
    return d * bits // 8 + 2


# ---------------------------------------------------------------------------
# Dequantization and attention
# ---------------------------------------------------------------------------

def dequantize(codes, norms16, signs, centroids) -> np.ndarray:
    """x_hat = n16 * R^T c[idx]  (the exact inverse rotation, [tq-fwht] §2)."""
    c = np.asarray(centroids, dtype=np.float64)[np.asarray(codes)]
    n = np.asarray(norms16, dtype=np.float64)
    return n[..., None] * unrotate(c, signs)


def decode_attention(q, k_hat, v_hat, scale: float, seq_lens=None, tau: float = 0.0, valid=None):
    """Decode attention over a dequantized cache, one query per (batch, head).

    q: [B, Hq, d]; k_hat, v_hat: [B, Hkv, T, d]; query head h reads kv head
    h // (Hq // Hkv).  For each (b, h) with length T_b:
      s_t = scale * q . k_hat_t,  M = max s,  LSE = M + log sum exp(s - M),
      p_t = exp(s_t - LSE),       o = sum_t keep_t p_t v_hat_t,
    with keep_t = (p_t >= tau) for Sparse V ([inferrs] §Sparse V: V rows of
    low attention weight are skipped) and keep_t = 1 when tau == 0.  The
    denominator always counts every row (no renormalisation).
    valid: optional bool [B, T]; a position with valid[b, t] False is not part of
    sequence b's context (a paged cache's position whose block-table entry names no
    page, [inferrs] §二 PagedAttention: only allocated pages hold tokens): it is left out
    of the softmax entirely, as if the position were absent.  A row with no valid
    position gives o = 0 and LSE = -inf.
    Returns (out [B, Hq, d], lse [B, Hq], scores [B, Hq, T] with -inf past T_b and at
    positions that are not valid).
    """
    q = np.asarray(q, dtype=np.float64)
    kh = np.asarray(k_hat, dtype=np.float64)
    vh = np.asarray(v_hat, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv, t_max = kh.shape[1], kh.shape[2]
    g = hq // hkv
    out = np.zeros((bsz, hq, d))
    lse = np.full((bsz, hq), -np.inf)
    scores = np.full((bsz, hq, t_max), -np.inf)
    for b in range(bsz):
        tb = t_max if seq_lens is None else int(seq_lens[b])
        for h in range(hq):
            j = h // g
            if tb == 0:
                continue
            live = np.ones(tb, dtype=bool) if valid is None else np.asarray(valid[b][:tb], dtype=bool)
            if not live.any():
                continue
            pos = np.nonzero(live)[0]
            s = scale * (kh[b, j, pos] @ q[b, h])
            m = s.max()
            ssum = np.exp(s - m).sum()
            l_ = m + math.log(ssum)
            p = np.exp(s - l_)
            keep = p >= tau if tau > 0 else np.ones(pos.size, dtype=bool)
            out[b, h] = (p[keep, None] * vh[b, j, pos][keep]).sum(axis=0)
            lse[b, h] = l_
            scores[b, h, pos] = s
    return out, lse, scores


def multi_query_attention(q, k_hat, v_hat, scale: float, seq_lens=None, valid=None):
    """Attention of n_q new query positions per sequence over a dequantized cache that
    already holds them (speculative verify, chunked prefill): the step after single-query
    decode, scored against the same quantized keys ([google], the scoring kernel;
    [inferrs] on prefill speed).

    q: [B, n_q, Hq, d]; k_hat, v_hat: [B, Hkv, T, d]; query head h reads kv head
    h // (Hq // Hkv).  With T_b cached tokens of sequence b, query i sits at position
    T_b - n_q + i and attends causally to positions 0 .. T_b - n_q + i:
      s_t = scale * q . k_hat_t,  LSE = log sum_t exp(s_t),  o = sum_t exp(s_t - LSE) v_hat_t.
    A query with no position to attend to (T_b - n_q + i < 0) gives o = 0, LSE = -inf.
    valid: optional bool [B, T]; positions with valid[b, t] False are not part of the sequence
    (a paged cache's positions on a table entry of no page, as in `decode_attention`) and are
    left out of every query's softmax.
    Returns (out [B, n_q, Hq, d], lse [B, n_q, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    kh = np.asarray(k_hat, dtype=np.float64)
    vh = np.asarray(v_hat, dtype=np.float64)
    bsz, n_q, hq, d = q.shape
    hkv, t_max = kh.shape[1], kh.shape[2]
    g = hq // hkv
    out = np.zeros((bsz, n_q, hq, d))
    lse = np.full((bsz, n_q, hq), -np.inf)
    for b in range(bsz):
        tb = t_max if seq_lens is None else int(seq_lens[b])
        for i in range(n_q):
            n_vis = tb - n_q + i + 1  # positions 0 .. tb - n_q + i
            if n_vis <= 0:
                continue
            pos = np.arange(n_vis) if valid is None else np.nonzero(np.asarray(valid[b][:n_vis], dtype=bool))[0]
            if pos.size == 0:
                continue
            for h in range(hq):
                j = h // g
                s = scale * (kh[b, j, pos] @ q[b, i, h])
                m = s.max()
                l_ = m + math.log(np.exp(s - m).sum())
                out[b, i, h] = (np.exp(s - l_)[:, None] * vh[b, j, pos]).sum(axis=0)
                lse[b, i, h] = l_
    return out, lse


def ip_search(q, codes, norms16, signs, centroids, k: int):
    """Approximate inner-product nearest-neighbour search with the same quantizer ([tq-80]
    §技术背景与学术渊源: the method also serves approximate nearest-neighbour search, with
    higher recall than product quantization and next to no indexing time, the codebook
    being data-independent).

    q: [Q, d] queries; codes [N, d], norms16 [N]: the quantized database.  The score of
    database vector t for query j is the inner product with its dequantized vector,
      s_{j,t} = q_j . x_hat_t,   x_hat_t = n16_t R^T c[codes_t];
    the result for query j is the min(k, N) indices of largest score in descending score
    order, equal scores by ascending index.
    Returns (idx [Q, k'] int64, scores [Q, k'] fp64, all scores [Q, N] fp64)."""
    xh = dequantize(codes, norms16, signs, centroids)
    qq = np.asarray(q, dtype=np.float64)
    s = qq @ xh.T
    n = xh.shape[0]
    kk = min(int(k), n)
    idx = np.zeros((qq.shape[0], kk), dtype=np.int64)
    for j in range(qq.shape[0]):
        order = np.lexsort((np.arange(n), -s[j]))   # primary key: -score; then index
        idx[j] = order[:kk]
    return idx, np.take_along_axis(s, idx, axis=1), s


# ---------------------------------------------------------------------------
# QJL residual variant  ([google] §第二步：QJL —— 1 bit 清理殘差 and the mlx-vlm kernel list
# (_qjl_score_kernel, _prod_score_kernel); [tq-80] §技术背景与学术渊源 (QJL, a residual
# correction built on the Johnson-Lindenstrauss lemma))
# ---------------------------------------------------------------------------

def qjl_scale(m: int) -> float:
    """kappa = sqrt(pi / 2) / m, the factor that makes the sign sketch's inner-product estimate
    unbiased: for a Gaussian row s ~ N(0, I), E[sign(s . r) (s . q)] = sqrt(2 / pi) (q . r) / ||r||,
    so sqrt(pi / 2) ||r|| / m sum_j sign((S r)_j) (S q)_j has mean q . r.  No sketch (m = 0)
    gives no correction."""
    return math.sqrt(math.pi / 2.0) / m if m > 0 else 0.0


def qjl_quantize(x, signs, centroids, boundaries, proj):
    """Quantize head vectors x[..., d] with the QJL residual variant.

    [google] §第二步: after the first stage (here the (b-1)-bit rotate-and-code path of
    `quantize`), one bit per sketch coordinate records the sign of a Johnson-Lindenstrauss
    projection of the remaining error, which removes the bias of inner products (attention
    scores).  Steps:
      codes, n16, u = quantize(x)                      the MSE stage
      r = R x - n16 c[codes]                           residual of the reconstruction the
                                                       decoder makes, in the rotated domain
      rn16 = fp16(||r||)                               its norm, stored as fp16
      z = S r  (S: [m, d] Gaussian, an input)          the sketch
      sigma_j = 1 if z_j >= 0 else 0                   one bit per row of S
    Returns (codes, n16, sigma bool [..., m], rn16, u, z, ||r|| fp64)."""
    codes, n16, u = quantize(x, signs, centroids, boundaries)
    c = np.asarray(centroids, dtype=np.float64)
    y = rotate(x, signs)
    r = y - np.asarray(n16, dtype=np.float64)[..., None] * c[codes]
    rn = np.sqrt(np.sum(r * r, axis=-1))
    z = r @ np.asarray(proj, dtype=np.float64).T
    return codes, n16, z >= 0.0, fp16_round(rn), u, z, rn


def qjl_dequantize(codes, norms16, sigma, res_norms16, signs, centroids, proj) -> np.ndarray:
    """The effective key of the QJL estimate: the vector k_hat with q . k_hat equal to the
    estimate of q . x for every q,
      k_hat = n16 R^T c[codes] + kappa rn16 R^T S^T (2 sigma - 1),   kappa = sqrt(pi/2) / m.
    (The estimate is linear in q, so attention over these keys is attention with the
    QJL-corrected scores.)"""
    s_mat = np.asarray(proj, dtype=np.float64)
    m = s_mat.shape[0]
    base = dequantize(codes, norms16, signs, centroids)
    if m == 0:
        return base
    pm = 2.0 * np.asarray(sigma, dtype=np.float64) - 1.0
    corr = qjl_scale(m) * np.asarray(res_norms16, dtype=np.float64)[..., None] * (pm @ s_mat)
    return base + unrotate(corr, signs)


def qjl_inner_product(q, codes, norms16, sigma, res_norms16, signs, centroids, proj) -> np.ndarray:
    """Estimate of q . x from the QJL code of x, computed in the rotated domain as the
    score kernels do ([google] _prod_score_kernel: MSE part plus QJL correction):
      n16 (R q) . c[codes] + kappa rn16 (S R q) . (2 sigma - 1)."""
    qr = rotate(q, signs)
    c = np.asarray(centroids, dtype=np.float64)[np.asarray(codes)]
    s_mat = np.asarray(proj, dtype=np.float64)
    mse = np.asarray(norms16, dtype=np.float64) * np.sum(qr * c, axis=-1)
    if s_mat.shape[0] == 0:
        return mse
    pm = 2.0 * np.asarray(sigma, dtype=np.float64) - 1.0
    return mse + qjl_scale(s_mat.shape[0]) * np.asarray(res_norms16, dtype=np.float64) * np.sum(
        (qr @ s_mat.T) * pm, axis=-1)


def qjl_near_zero_mask(z, r_norm, proj, band: float = 1e-5) -> np.ndarray:
    """Sketch coordinates whose projection is within `band` of zero relative to its natural
    scale, |z_j| <= band ||S_j|| ||r|| (|cos| of the angle between row j and r): there a sign
    computed in fp32 may differ from the fp64 one, and either bit is accepted."""
    rows = np.linalg.norm(np.asarray(proj, dtype=np.float64), axis=-1)
    return np.abs(np.asarray(z)) <= band * rows * np.asarray(r_norm, dtype=np.float64)[..., None]


def sparse_v_borderline(scores, lse, tau: float, rel: float = 1e-3) -> np.ndarray:
    """Rows whose keep decision is within the score tolerance of the threshold.

    |s_t - (LSE + ln tau)| <= rel * max|s| for the (b, h) row; either decision
    is acceptable there.
    """
    s = np.asarray(scores, dtype=np.float64)
    thr = np.asarray(lse, dtype=np.float64)[..., None] + math.log(tau)
    # only finite scores against a finite threshold are compared: a row with no tokens
    # (LSE = -inf, every score -inf) has no borderline entry, and no -inf - -inf is formed
    finite = np.isfinite(s) & np.isfinite(thr)
    smax = np.where(np.isfinite(s), np.abs(s), 0.0).max(axis=-1, keepdims=True)
    dist = np.abs(np.where(finite, s, 0.0) - np.where(finite, thr, 0.0))
    return finite & (dist <= rel * smax)

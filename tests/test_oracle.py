"""Pins for the CPU oracle: closed forms, library routines, textbook cases, brute force.

None of these re-type the oracle's own formula; each compares it with something
the mathematics or an independent routine fixes.
"""
import math
import os

import numpy as np
import pytest
from scipy import linalg, special

from oracle import tq_oracle as o

D = 128
ALPHA = (D - 3) / 2.0
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- codebook


def _beta_mass(a, b):
    """Closed-form cell mass of (1-x^2)^alpha / Z via the regularized incomplete beta."""
    p = ALPHA + 1.0
    return special.betainc(p, p, (b + 1) / 2) - special.betainc(p, p, (a + 1) / 2)


def _first_moment(a, b):
    """Closed-form int_a^b x (1-x^2)^alpha dx / Z."""
    z = special.beta(0.5, ALPHA + 1.0)
    p = ALPHA + 1.0
    return ((1 - a * a) ** p - (1 - b * b) ** p) / (2 * p * z)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_quadrature_matches_closed_form_moments(bits, golden_codebooks):
    c, t = golden_codebooks[bits]
    edges = np.concatenate(([-1.0], t, [1.0]))
    f = o.rotated_coordinate_density(D)
    mass, mom = o.cell_integrals(f, edges)
    z = special.beta(0.5, ALPHA + 1.0)
    mass_cf = _beta_mass(edges[:-1], edges[1:])
    mom_cf = _first_moment(edges[:-1], edges[1:])
    assert np.allclose(mass / z, mass_cf, rtol=1e-11, atol=1e-16)
    assert np.allclose(mom / z, mom_cf, rtol=1e-10, atol=1e-17)
    # the stored table satisfies the centroid condition with closed-form moments
    assert np.allclose(mom_cf / mass_cf, c, rtol=0, atol=5e-10)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_midpoint_condition_and_symmetry(bits, golden_codebooks):
    c, t = golden_codebooks[bits]
    assert len(c) == 1 << bits and len(t) == (1 << bits) - 1
    assert np.all(np.diff(c) > 0)
    assert np.array_equal(t, 0.5 * (c[:-1] + c[1:]))
    assert np.array_equal(c, -c[::-1])
    assert t[(1 << bits) // 2 - 1] == 0.0


def test_one_bit_closed_form():
    # optimal 1-bit quantizer of a symmetric density: +/- E|x|
    c, _, _ = o.make_codebook(D, 1)
    e_abs = math.exp(special.gammaln(D / 2) - special.gammaln((D + 1) / 2)) / math.sqrt(math.pi)
    assert abs(e_abs - 0.0706616) < 1e-7
    assert np.allclose(c, [-e_abs, e_abs], rtol=1e-13)


def _max_table():
    rows = {}
    with open(os.path.join(GOLDEN, "max1960_gaussian.txt")) as fh:
        for ln in fh:
            if ln.startswith("#") or not ln.strip():
                continue
            head, outs, bnds, mse = [s.strip() for s in ln.split("|")]
            n = int(head.split()[1])
            rows[n] = ([float(x) for x in outs.split()],
                       [float(x) for x in bnds.split()] if bnds else [], float(mse))
    return rows


@pytest.mark.parametrize("levels", [2, 4, 8, 16])
def test_lloyd_routine_reproduces_max_gaussian_table(levels):
    """Textbook special case: the same Lloyd routine on N(0,1) gives Max's table."""
    outs, bnds, mse = _max_table()[levels]
    f = lambda x: np.exp(-0.5 * np.asarray(x) ** 2)
    init = o.gaussian_quantile_init(1, levels)
    c, t, _ = o.lloyd_max(f, -12.0, 12.0, init, 1e-13, max_piece=0.05)
    pos_c = c[levels // 2:]
    pos_t = t[levels // 2:]
    assert np.allclose(pos_c, outs, atol=6e-4, rtol=6e-4)
    assert np.allclose(pos_t, bnds, atol=6e-4, rtol=6e-4)
    # distortion of the result vs the table's mse
    edges = np.concatenate(([-12.0], t, [12.0]))
    tot = 0.0
    for k in range(levels):
        g = lambda x, ck=c[k]: (np.asarray(x) - ck) ** 2 * f(x)
        m, _ = o.cell_integrals(g, edges[k:k + 2], 0.05)
        tot += m[0]
    tot /= math.sqrt(2 * math.pi)
    assert abs(tot - mse) <= 6e-4 * mse + 5e-6


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_scaled_codebook_near_gaussian_limit(bits):
    outs, _, _ = _max_table()[1 << bits]
    c, _, _ = o.make_codebook(D, bits)
    ratio = math.sqrt(D) * c[(1 << bits) // 2:] / np.array(outs)
    assert np.all(np.abs(ratio - 1) < 0.02)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_optimum_is_unique(bits):
    c1, _, _ = o.make_codebook(D, bits, init="gauss")
    c2, _, _ = o.make_codebook(D, bits, init="uniform")
    assert np.allclose(c1, c2, rtol=0, atol=1e-10)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_stored_tables_match_fresh_lloyd(bits, golden_codebooks):
    c, t, _ = o.make_codebook(D, bits)
    assert np.array_equal(c, golden_codebooks[bits][0])
    assert np.array_equal(t, golden_codebooks[bits][1])


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_distortion_matches_monte_carlo_and_bound(bits, golden_codebooks):
    c, t = golden_codebooks[bits]
    d_quad = o.codebook_distortion(D, c)
    rng = np.random.default_rng(1234)
    x = rng.standard_normal((20000, D))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)   # uniform on the sphere
    idx = o.code_by_boundaries(u, t)
    err = ((u - c[idx]) ** 2).sum(axis=1)
    se = err.std() / math.sqrt(err.size)
    assert abs(err.mean() - d_quad) < 4 * se
    # the pages' "about 2.7x the information-theoretic bound" read with the
    # 4^-b lower bound: D_b * 4^b stays below sqrt(3)*pi/2
    assert d_quad * 4 ** bits < math.sqrt(3) * math.pi / 2
    assert d_quad * 4 ** bits > 1.0


# ----------------------------------------------------------------- rotation


def _signs(seed=1):
    rng = np.random.default_rng(seed)
    return 1 - 2 * rng.integers(0, 2, D)


def test_rotation_matches_scipy_hadamard():
    s = _signs()
    r = o.rotation_matrix(s)
    ref = linalg.hadamard(D).astype(np.float64) * s[None, :] / math.sqrt(D)
    assert np.array_equal(r, ref)
    assert np.abs(r @ r.T - np.eye(D)).max() < 1e-14
    x = np.random.default_rng(0).standard_normal((10, D))
    y = x @ r.T
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    assert np.allclose(y @ r, x, atol=1e-13)
    assert np.allclose(o.rotate(x, s), y, atol=1e-13)
    assert np.allclose(o.unrotate(o.rotate(x, s), s), x, atol=1e-13)


# ----------------------------------------------------------------- quantize


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_quantize_basis_vectors(bits, golden_codebooks):
    """x = e_j: every u_i = H[i, j] s_j / sqrt(d) = +/- 1/sqrt(d)."""
    c, t = golden_codebooks[bits]
    s = _signs()
    h = linalg.hadamard(D)
    expect_pos = int(np.argmin(np.abs(c - 1 / math.sqrt(D))))
    expect_neg = int(np.argmin(np.abs(c + 1 / math.sqrt(D))))
    assert expect_pos + expect_neg == len(c) - 1
    assert expect_pos == {2: 3, 3: 5, 4: 11, 8: 184}[bits]
    for j in (0, 5, 77, 127):
        x = np.zeros(D)
        x[j] = 3.0
        codes, n16, u = o.quantize(x[None], s, c, t)
        sign = h[:, j] * s[j]
        assert np.array_equal(codes[0], np.where(sign > 0, expect_pos, expect_neg))
        assert float(n16[0]) == 3.0
        assert np.abs(np.abs(u[0][:, None] - t[None, :])).min() > 7.5e-4


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_quantize_ties_and_zero_vector(bits, golden_codebooks):
    c, t = golden_codebooks[bits]
    levels = 1 << bits
    plus = np.ones(D, dtype=np.int64)
    codes, _, u = o.quantize(np.ones((1, D)), plus, c, t)
    assert abs(u[0, 0] - 1.0) < 1e-15 and np.all(u[0, 1:] == 0.0)
    assert codes[0, 0] == levels - 1
    assert np.all(codes[0, 1:] == levels // 2 - 1)          # ties go to the lower code
    codes0, n0, u0 = o.quantize(np.zeros((1, D)), _signs(), c, t)
    assert float(n0[0]) == 0.0 and np.all(u0 == 0.0)
    assert np.all(codes0 == levels // 2 - 1)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_bruteforce_equals_boundary_search(bits, golden_codebooks):
    c, t = golden_codebooks[bits]
    rng = np.random.default_rng(bits)
    u = np.concatenate([rng.standard_normal(5000) * 0.12, c, [-1.0, 1.0, 0.0]])
    assert np.array_equal(o.nearest_code_bruteforce(u, c), o.code_by_boundaries(u, t))
    # exactly on a boundary both neighbours are nearest (up to the rounding of
    # |u - c|); the boundary rule takes the lower one
    at = o.code_by_boundaries(t, t)
    assert np.array_equal(at, np.arange(len(t)))
    assert np.all(np.abs(o.nearest_code_bruteforce(t, c) - at) <= 1)


def test_fp16_norm_is_round_to_nearest_even():
    vals = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2048 + 1, 65504.0, 1e-8])
    r = o.fp16_round(vals).astype(np.float64)
    assert r[0] == 1.0 and r[1] == 1 + 2 ** -9 and r[2] == 2048.0 and r[3] == 65504.0
    assert r[4] == 0.0


# ----------------------------------------------------------------- packing


def _pack_bit_loop(codes, bits, layout):
    n_tokens, d = codes.shape
    out = bytearray(n_tokens * d * bits // 8)
    for tok in range(n_tokens):
        for i in range(d):
            for k in range(bits):
                if (int(codes[tok, i]) >> k) & 1:
                    if layout == o.LAYOUT_ROWS:
                        pos = (tok * d + i) * bits + k
                    else:
                        grp, r = divmod(tok, 8)
                        pos = grp * d * 8 * bits + (i * 8 + r) * bits + k
                    out[pos // 8] |= 1 << (pos % 8)
    return np.frombuffer(bytes(out), dtype=np.uint8)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("layout", [0, 1])
def test_pack_two_routes_and_roundtrip(bits, layout):
    rng = np.random.default_rng(bits * 10 + layout)
    codes = rng.integers(0, 1 << bits, size=(16, D))
    a = o.pack(codes, bits, layout)
    b = _pack_bit_loop(codes, bits, layout)
    assert np.array_equal(a, b)
    assert np.array_equal(o.unpack(a, 16, D, bits, layout), codes)
    if layout == o.LAYOUT_ROWS:
        bitmat = ((codes[:, :, None] >> np.arange(bits)) & 1).astype(np.uint8).reshape(-1)
        assert np.array_equal(np.packbits(bitmat, bitorder="little"), a)
        # one row per vector, d*b/8 bytes
        assert np.array_equal(a.reshape(16, -1)[3], o.pack(codes[3:4], bits))


# ----------------------------------------------------------------- dequantize / attention


def test_dequantize_norm_and_inverse(golden_codebooks):
    s = _signs()
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, D)) * 3
    for bits in (2, 4, 8):
        c, t = golden_codebooks[bits]
        codes, n16, u = o.quantize(x, s, c, t)
        xh = o.dequantize(codes, n16, s, c)
        assert np.allclose(np.linalg.norm(xh, axis=1),
                           n16.astype(np.float64) * np.linalg.norm(c[codes], axis=1), rtol=1e-13)
        rel = np.linalg.norm(xh - x, axis=1) / np.linalg.norm(x, axis=1)
        assert rel.mean() < 1.5 * math.sqrt(o.codebook_distortion(D, c))


def _small_cache(bits_k=4, bits_v=2, b=2, hkv=2, hq=4, T=37, seed=0, golden=None):
    s = _signs()
    rng = np.random.default_rng(seed)
    ck, tk = golden[bits_k]
    cv, tv = golden[bits_v]
    k = rng.standard_normal((b, hkv, T, D))
    v = rng.standard_normal((b, hkv, T, D))
    kc, kn, _ = o.quantize(k, s, ck, tk)
    vc, vn, _ = o.quantize(v, s, cv, tv)
    kh = o.dequantize(kc, kn, s, ck)
    vh = o.dequantize(vc, vn, s, cv)
    q = rng.standard_normal((b, hq, D))
    return s, q, kc, kn, vc, vn, kh, vh, ck, cv


def test_attention_rotated_domain_identity(golden_codebooks):
    s, q, kc, kn, vc, vn, kh, vh, ck, cv = _small_cache(golden=golden_codebooks)
    scale = 1 / math.sqrt(D)
    out, lse, scores = o.decode_attention(q, kh, vh, scale)
    r = o.rotation_matrix(s)
    g = q.shape[1] // kh.shape[1]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            qt = scale * (r @ q[b, h])
            s_rot = kn[b, h // g].astype(np.float64) * (ck[kc[b, h // g]] @ qt)
            assert np.allclose(scores[b, h], s_rot, rtol=1e-12, atol=1e-12)
            assert abs(lse[b, h] - special.logsumexp(s_rot)) < 1e-12
            p = special.softmax(s_rot)
            o_rot = (p[:, None] * vn[b, h // g].astype(np.float64)[:, None] * cv[vc[b, h // g]]).sum(0)
            assert np.allclose(out[b, h], r.T @ o_rot, atol=1e-12)


def test_attention_special_cases(golden_codebooks):
    s, q, kc, kn, vc, vn, kh, vh, ck, cv = _small_cache(golden=golden_codebooks)
    scale = 1 / math.sqrt(D)
    out1, lse1, _ = o.decode_attention(q, kh[:, :, :1], vh[:, :, :1], scale)
    assert np.allclose(out1, np.repeat(vh[:, :, 0], 2, axis=1))
    out0, _, _ = o.decode_attention(np.zeros_like(q), kh, vh, scale)
    assert np.allclose(out0, np.repeat(vh.mean(axis=2), 2, axis=1))
    vsame = np.broadcast_to(vh[:, :, :1], vh.shape)
    out_same, _, _ = o.decode_attention(q, kh, vsame, scale)
    assert np.allclose(out_same, np.repeat(vh[:, :, 0], 2, axis=1))
    # GQA: query head h reads kv head h // g
    _, lse, scores = o.decode_attention(q, kh, vh, scale)
    for h in range(4):
        assert np.allclose(scores[1, h, :], scale * kh[1, h // 2] @ q[1, h])
    assert np.allclose(np.exp(scores - lse[..., None]).sum(-1), 1.0)
    # per-sequence lengths
    lens = np.array([5, 37])
    out_l, lse_l, sc_l = o.decode_attention(q, kh, vh, scale, seq_lens=lens)
    ref, _, _ = o.decode_attention(q[:1], kh[:1, :, :5], vh[:1, :, :5], scale)
    assert np.allclose(out_l[0], ref[0]) and np.all(np.isneginf(sc_l[0, :, 5:]))


def test_multi_query_attention_pins(golden_codebooks):
    """Multi-query attention: one query position equals single-query decode; query i equals
    decode over the first T - n_q + i + 1 positions; later positions do not reach earlier
    queries; and the whole thing matches torch's scaled-dot-product attention (fp64, CPU)
    with an explicit causal mask."""
    torch = pytest.importorskip("torch")
    s, q1, kc, kn, vc, vn, kh, vh, ck, cv = _small_cache(T=41, golden=golden_codebooks)
    scale = 1 / math.sqrt(D)
    rng = np.random.default_rng(9)
    n_q = 5
    q = rng.standard_normal((2, n_q, 4, D))
    # n_q = 1 is decode
    one, lse1 = o.multi_query_attention(q1[:, None], kh, vh, scale)
    dec, lsed, _ = o.decode_attention(q1, kh, vh, scale)
    assert np.allclose(one[:, 0], dec, atol=1e-13) and np.allclose(lse1[:, 0], lsed, atol=1e-13)
    # query i = decode over a prefix; per-sequence lengths, including one shorter than n_q
    lens = np.array([41, 3])
    out, lse = o.multi_query_attention(q, kh, vh, scale, seq_lens=lens)
    for b in range(2):
        for i in range(n_q):
            n_vis = int(lens[b]) - n_q + i + 1
            if n_vis <= 0:
                assert np.all(out[b, i] == 0.0) and np.all(np.isneginf(lse[b, i]))
                continue
            ref, lref, _ = o.decode_attention(q[b:b + 1, i], kh[b:b + 1], vh[b:b + 1], scale,
                                              seq_lens=np.array([n_vis]))
            assert np.allclose(out[b, i], ref[0], atol=1e-13) and np.allclose(lse[b, i], lref[0])
    # causality: changing positions after a query's last one leaves that query unchanged
    kh2, vh2 = kh.copy(), vh.copy()
    kh2[:, :, 41 - n_q + 2:] += 5.0
    vh2[:, :, 41 - n_q + 2:] -= 3.0
    out2, _ = o.multi_query_attention(q, kh2, vh2, scale)
    out0, _ = o.multi_query_attention(q, kh, vh, scale)
    assert np.allclose(out2[:, :2], out0[:, :2], atol=1e-13)
    assert not np.allclose(out2[:, 2:], out0[:, 2:])
    # torch SDPA with a boolean causal mask, query head h on kv head h // 2
    tq_ = torch.from_numpy(q).permute(0, 2, 1, 3)                   # [B, Hq, n_q, d]
    tk = torch.from_numpy(np.repeat(kh, 2, axis=1))                  # [B, Hq, T, d]
    tv = torch.from_numpy(np.repeat(vh, 2, axis=1))
    T = kh.shape[2]
    mask = torch.arange(T)[None, :] <= (T - n_q + torch.arange(n_q))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq_, tk, tv, attn_mask=mask, scale=scale)
    assert np.allclose(out0, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)


def test_attention_excluded_positions_equal_removed_positions(golden_codebooks):
    """Positions that are not part of the context (valid = False) behave exactly as if they
    had been removed from the cache: the result equals attention over the compacted cache,
    and differs from attending to them as zero vectors (which would add exp(0 - LSE)
    to the denominator)."""
    s, q, kc, kn, vc, vn, kh, vh, ck, cv = _small_cache(T=200, golden=golden_codebooks)
    scale = 1 / math.sqrt(D)
    bsz, T = kh.shape[0], kh.shape[2]
    valid = np.ones((bsz, T), dtype=bool)
    valid[0, 64:128] = False          # a missing page in the middle of sequence 0
    valid[-1, :64] = False            # and the first page of the last sequence
    out, lse, sc = o.decode_attention(q, kh, vh, scale, valid=valid)
    for b in range(bsz):
        keep = np.nonzero(valid[b])[0]
        ref, rlse, rsc = o.decode_attention(q[b:b + 1], kh[b:b + 1][:, :, keep], vh[b:b + 1][:, :, keep], scale)
        assert np.allclose(out[b], ref[0], rtol=1e-13, atol=1e-15)
        assert np.allclose(lse[b], rlse[0], rtol=1e-13)
        assert np.all(np.isneginf(sc[b][:, ~valid[b]]))
        assert np.allclose(sc[b][:, keep], rsc[0], rtol=1e-13)
    zeroed_k, zeroed_v = kh.copy(), vh.copy()
    zeroed_k[0, :, 64:128] = 0.0
    zeroed_v[0, :, 64:128] = 0.0
    as_zero, zlse, _ = o.decode_attention(q, zeroed_k, zeroed_v, scale)
    assert np.all(zlse[0] > lse[0])
    # no valid position at all: o = 0, LSE = -inf; with seq_lens the two rules combine
    none, nlse, _ = o.decode_attention(q, kh, vh, scale, valid=np.zeros((bsz, T), dtype=bool))
    assert np.all(none == 0.0) and np.all(np.isneginf(nlse))
    part, plse, _ = o.decode_attention(q, kh, vh, scale, seq_lens=[100] * bsz, valid=valid)
    ref0, rl0, _ = o.decode_attention(q[:1], kh[:1][:, :, :64], vh[:1][:, :, :64], scale)
    assert np.allclose(part[0], ref0[0], rtol=1e-13, atol=1e-15) and np.allclose(plse[0], rl0[0])


def test_multi_query_excluded_positions_equal_decode_over_prefix(golden_codebooks):
    """Several query positions with positions left out (paged holes): query i equals
    single-query decode over its own prefix with the same positions left out."""
    s, q, kc, kn, vc, vn, kh, vh, ck, cv = _small_cache(T=120, golden=golden_codebooks)
    scale = 1 / math.sqrt(D)
    bsz, T = kh.shape[0], kh.shape[2]
    n_q = 6
    rng = np.random.default_rng(5)
    qm = rng.standard_normal((bsz, n_q, q.shape[1], D))
    valid = np.ones((bsz, T), dtype=bool)
    valid[0, 10:40] = False
    valid[1, 100:] = False                         # the last positions, some queries' own
    out, lse = o.multi_query_attention(qm, kh, vh, scale, valid=valid)
    for b in range(bsz):
        for i in range(n_q):
            n_vis = T - n_q + i + 1
            ref, rl, _ = o.decode_attention(qm[b:b + 1, i], kh[b:b + 1], vh[b:b + 1], scale, seq_lens=[n_vis],
                                            valid=valid[b:b + 1])
            assert np.allclose(out[b, i], ref[0], rtol=1e-12, atol=1e-14)
            assert np.allclose(lse[b, i], rl[0], rtol=1e-12)
    # without a mask it is the unmasked attention
    full, _ = o.multi_query_attention(qm, kh, vh, scale)
    same, _ = o.multi_query_attention(qm, kh, vh, scale, valid=np.ones((bsz, T), dtype=bool))
    assert np.array_equal(full, same)


def test_sparse_v_limits_and_bound(golden_codebooks):
    s, q, kc, kn, vc, vn, kh, vh, ck, cv = _small_cache(T=200, golden=golden_codebooks)
    q = q * 6.0     # sharpen the attention so some rows fall under the threshold
    scale = 1 / math.sqrt(D)
    dense, lse, scores = o.decode_attention(q, kh, vh, scale)
    same, _, _ = o.decode_attention(q, kh, vh, scale, tau=1e-300)
    assert np.allclose(same, dense)
    none, _, _ = o.decode_attention(q, kh, vh, scale, tau=1.01)
    assert np.all(none == 0.0)
    tau = 1e-2
    sparse, _, _ = o.decode_attention(q, kh, vh, scale, tau=tau)
    p = np.exp(scores - lse[..., None])
    dropped = p < tau
    g = q.shape[1] // kh.shape[1]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            bound = (p[b, h] * dropped[b, h] * np.linalg.norm(vh[b, h // g], axis=1)).sum()
            assert np.linalg.norm(sparse[b, h] - dense[b, h]) <= bound + 1e-12
    assert dropped.any() and (~dropped).any()


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_near_boundary_band_is_absolute_and_inclusive(bits, golden_codebooks):
    """The band that excuses a code mismatch: |u - t_j| <= 1e-6 in unit-vector units.
    Constructed values at +-0.5e-6 and +-1.5e-6 of every boundary, plus exactly on it, so a
    band read as relative (|u - t| <= 1e-6 |t|), a strict '<' or a wider band each fails."""
    c, t = golden_codebooks[bits]
    band = 1e-6
    inside = np.concatenate([t - 0.5 * band, t + 0.5 * band, t])
    outside = np.concatenate([t - 1.5 * band, t + 1.5 * band])
    # the cells are far wider than the band: no constructed value is near a second boundary
    assert np.min(np.diff(t)) > 100 * band
    assert np.all(o.near_boundary_mask(inside, t, band))
    assert not np.any(o.near_boundary_mask(outside, t, band))
    # a value at exactly band + a small margin is outside; exactly at the edge is inside
    # (both chosen so the fp64 distance is exact: a boundary with a short mantissa)
    edge = np.array([0.0 + band, 0.0 - band, 0.0 + 2 * band])
    assert list(o.near_boundary_mask(edge, t, band)) == [True, True, False]
    # the centroids themselves are half a cell away: never flagged
    assert not np.any(o.near_boundary_mask(c, t, band))
    # shapes: the mask keeps the leading axes of u
    u = np.stack([inside[:4], outside[:4]])
    assert o.near_boundary_mask(u, t, band).tolist() == [[True] * 4, [False] * 4]


def test_sparse_v_borderline_band_sign_and_empty_rows():
    """Rows whose keep decision is within the score tolerance: |s - (LSE + ln tau)| <=
    1e-3 max|s|.  Scores are placed at +-0.5 and +-1.5 times the tolerance around the
    threshold; a sign slip in ln tau, an absolute 1e-3 band or a band on |s| alone fails."""
    rel, tau = 1e-3, 1e-4
    lse = np.array([[3.0, -2.0]])
    thr = lse + math.log(tau)              # about -6.21 and -11.21
    smax = np.array([[40.0, 25.0]])       # one large score per row sets max|s|
    tol = rel * smax
    offs = np.array([-1.5, -0.5, 0.0, 0.5, 1.5])
    rows = np.zeros((1, 2, 6))
    for h in range(2):
        rows[0, h, :5] = thr[0, h] + offs * tol[0, h]
        rows[0, h, 5] = smax[0, h]
    got = o.sparse_v_borderline(rows, lse, tau, rel)
    want = np.array([False, True, True, True, False, False])
    assert got.tolist() == [[want.tolist(), want.tolist()]]
    # the band scales with the row's largest |s|, not with 1e-3 alone: at +-0.5 tol = 0.02
    # (row 0) an absolute 1e-3 band would flag nothing
    assert 0.5 * tol[0, 0] > 10 * rel
    # the threshold sits below the LSE (ln tau < 0): the mirror image LSE - ln tau is far
    mirror = lse[..., None] - math.log(tau) + np.zeros((1, 2, 1))
    assert not o.sparse_v_borderline(np.concatenate([mirror, rows[..., 5:]], -1), lse, tau, rel).any()
    # the flagged rows are exactly those whose weight exp(s - LSE) lies within a factor
    # exp(tol) of tau
    p = np.exp(rows - lse[..., None])
    near = np.abs(np.log(p / tau)) <= tol[..., None] * (1 + 1e-9)
    assert np.array_equal(near, got)
    # rows with no tokens (LSE = -inf, every score -inf) and -inf entries of a live row are
    # never borderline, and no invalid operation is formed
    mixed = np.array([[[-np.inf] * 6, [-np.inf, thr[0, 1], 1.0, -np.inf, 2.0, -np.inf]]])
    mlse = np.array([[-np.inf, lse[0, 1]]])
    with np.errstate(all="raise"):
        m = o.sparse_v_borderline(mixed, mlse, tau, rel)
    assert m.tolist() == [[[False] * 6, [False, True, False, False, False, False]]]


# ----------------------------------------------------------------- QJL residual variant


def _qjl_case(golden, bits=1, seed=5):
    """One vector with outlier channels and a query correlated with it, so that the MSE
    stage's inner product is visibly biased (the reconstruction shrinks toward the centre)."""
    rng = np.random.default_rng(seed)
    s = _signs()
    x = rng.standard_normal(D)
    x[[3, 40, 77]] *= 8.0
    q = x + 0.5 * rng.standard_normal(D)
    c, t = golden[bits]
    return s, x, q, c, t


def _qjl_draws(s, x, q, c, t, n, seed):
    """The estimate of q . x for n independent Gaussian sketches S (m = d)."""
    rng = np.random.default_rng(seed)
    est = np.empty(n)
    for i in range(n):
        proj = rng.standard_normal((D, D))
        codes, n16, sig, rn16, _, _, _ = o.qjl_quantize(x, s, c, t, proj)
        est[i] = o.qjl_inner_product(q, codes, n16, sig, rn16, s, c, proj)
    return est


@pytest.mark.parametrize("bits", [1, 2])
def test_qjl_estimate_is_unbiased_over_sketches(bits, golden_codebooks):
    """E_S[estimate] = q . x: the sign sketch with kappa = sqrt(pi/2)/m removes the MSE stage's
    bias (Monte Carlo over 3000 sketches; a constant of sqrt(2/pi), 1, or a missing ||r||
    misses by hundreds of standard errors).  The only bias left is the fp16 rounding of ||r||."""
    s, x, q, c, t = _qjl_case(golden_codebooks, bits)
    exact = float(q @ x)
    codes, n16, _, rn16, _, _, rn = o.qjl_quantize(x, s, c, t, np.zeros((0, D)))
    mse_only = float(q @ o.dequantize(codes, n16, s, c))
    est = _qjl_draws(s, x, q, c, t, 3000, seed=11 + bits)
    se = est.std(ddof=1) / math.sqrt(est.size)
    resid_ip = exact - float(q @ o.dequantize(codes, n16, s, c))
    fp16_bias = abs(resid_ip) * abs(float(rn16) / rn - 1.0)
    assert abs(est.mean() - exact) <= 4.0 * se + fp16_bias
    assert abs(mse_only - exact) >= 50.0 * se          # the bias QJL removes is large here


def test_qjl_variance_matches_closed_form(golden_codebooks):
    """Var_S[estimate] = (pi/2) rn16^2 / m (||Rq||^2 - (2/pi) ((Rq) . r / ||r||)^2): the variance
    of one sign-times-projection term, summed over m independent rows and scaled by kappa rn16.
    It pins the 1/m scaling and the ||r|| factor; the bound (pi/2) ||r||^2 ||q||^2 / m holds."""
    s, x, q, c, t = _qjl_case(golden_codebooks, 2, seed=7)
    codes, n16, _, rn16, _, _, rn = o.qjl_quantize(x, s, c, t, np.zeros((0, D)))
    r = o.rotate(x, s) - float(n16) * c[codes]
    qr = o.rotate(q, s)
    rn16 = float(rn16)
    var_exact = (math.pi / 2) * rn16 ** 2 / D * (qr @ qr - (2 / math.pi) * (qr @ r / rn) ** 2)
    est = _qjl_draws(s, x, q, c, t, 6000, seed=21)
    ratio = est.var(ddof=1) / var_exact
    assert 0.92 < ratio < 1.08, ratio
    assert var_exact <= (math.pi / 2) * rn16 ** 2 * (q @ q) / D


def test_qjl_without_sketch_is_the_mse_path(golden_codebooks):
    """m = 0: no correction, the (b-1)-bit rotate-and-code path of quantize / dequantize."""
    s, q, kc, kn, vc, vn, kh, vh, ck, cv = _small_cache(T=20, golden=golden_codebooks)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, D))
    tk = golden_codebooks[4][1]
    empty = np.zeros((0, D))
    codes, n16, sig, rn16, u, z, rn = o.qjl_quantize(x, s, ck, tk, empty)
    c2, n2, u2 = o.quantize(x, s, ck, tk)
    assert np.array_equal(codes, c2) and np.array_equal(n16, n2) and sig.shape == (6, 0)
    assert np.array_equal(o.qjl_dequantize(codes, n16, sig, rn16, s, ck, empty), o.dequantize(codes, n16, s, ck))
    qq = rng.standard_normal((6, D))
    assert np.allclose(o.qjl_inner_product(qq, codes, n16, sig, rn16, s, ck, empty),
                       np.sum(qq * o.dequantize(codes, n16, s, ck), axis=-1), rtol=1e-12, atol=1e-12)


def test_qjl_routes_residual_and_special_vectors(golden_codebooks):
    """Two routes to the same estimate (the effective key in the original domain, and the
    rotated-domain sum the score kernels take); ||r|| equals ||x - x_hat|| of the dequantized
    MSE stage; the zero vector gives r = 0, every sign bit 1 and no correction; the sign bits
    pack as numpy.packbits (little bit order) does."""
    s = _signs()
    rng = np.random.default_rng(9)
    c, t = golden_codebooks[3]
    proj = rng.standard_normal((D, D))
    x = rng.standard_normal((5, D)) * np.array([1.0, 3.0, 0.2, 10.0, 1.0])[:, None]
    x[4] = 0.0
    codes, n16, sig, rn16, u, z, rn = o.qjl_quantize(x, s, c, t, proj)
    xh = o.dequantize(codes, n16, s, c)
    assert np.allclose(rn, np.linalg.norm(x - xh, axis=-1), rtol=1e-12, atol=1e-12)
    assert rn[4] == 0.0 and rn16[4] == 0.0 and sig[4].all()
    qq = rng.standard_normal((5, D))
    k_eff = o.qjl_dequantize(codes, n16, sig, rn16, s, c, proj)
    direct = o.qjl_inner_product(qq, codes, n16, sig, rn16, s, c, proj)
    assert np.allclose(np.sum(qq * k_eff, axis=-1), direct, rtol=1e-12, atol=1e-12)
    assert np.allclose(k_eff[4], 0.0)
    # the correction is kappa rn16 S^T (2 sigma - 1) in the rotated domain
    corr = o.rotate(k_eff - xh, s)
    assert np.allclose(corr[:4], (math.sqrt(math.pi / 2) / D) * rn16[:4, None].astype(np.float64)
                       * ((2.0 * sig[:4] - 1.0) @ proj), rtol=1e-12, atol=1e-12)
    packed = o.pack(sig[:4].astype(np.int64), 1, o.LAYOUT_ROWS)
    assert np.array_equal(packed, np.packbits(sig[:4].reshape(-1), bitorder="little"))
    assert packed.size == 4 * D // 8


def test_qjl_near_zero_band(golden_codebooks):
    """A sign bit may differ only where the projection is within 1e-5 ||S_j|| ||r|| of zero."""
    proj = np.ones((4, D)) * np.array([1.0, 2.0, 0.5, 4.0])[:, None]     # row norms sqrt(D) x
    rows = np.linalg.norm(proj, axis=-1)
    rnorm = np.array([2.0, 0.5])
    band = 1e-5
    z = np.stack([rows * rnorm[0] * band * np.array([0.5, -0.5, 1.0, 0.0]),
                  rows * rnorm[1] * band * np.array([1.5, -1.5, -2.0, 0.9])])
    got = o.qjl_near_zero_mask(z, rnorm, proj, band)
    assert got.tolist() == [[True, True, True, True], [False, False, False, True]]


def _page_figures():
    out = {}
    with open(os.path.join(GOLDEN, "pages_format_figures.txt")) as fh:
        for ln in fh:
            if ln.startswith("#") or not ln.strip():
                continue
            key, val, _ = [x.strip() for x in ln.split("|")]
            out[key] = float(val)
    return out


def test_byte_accounting_against_pages():
    fig = _page_figures()
    fp16 = 2 * D
    per = {b: o.packed_bytes_per_vector(D, b) for b in (2, 3, 4, 8)}
    assert per == {2: 34, 3: 50, 4: 66, 8: 130}
    assert round(fp16 / per[4], 1) == pytest.approx(3.9, abs=0.01) and fp16 / per[4] >= fig["turbo4_ratio_vs_fp16"]
    assert abs(fp16 / per[3] - fig["turbo3_ratio_vs_fp16_max"]) < 0.05
    assert 1 - (per[4] + per[2]) / (2 * fp16) > fig["k4v2_saving_min"]
    assert abs(1 - (per[3] + per[2]) / (2 * fp16) - fig["k3v2_saving"]) < 0.005
    assert (D * 4 // 8) / fp16 == fig["four_bit_cache_fraction"]


# ------------------------------------------------------------------ inner-product search


def test_ip_search_pins(golden_codebooks):
    """Inner-product search: (1) the scores equal the rotated-domain form n16 * (R q) . c[idx]
    (R orthogonal), computed from the codes without dequantizing; (2) database vectors that
    are positive multiples of one direction share their codes, so the ranking is that of the
    stored norms, largest first for a query along the direction and smallest first for its
    opposite; (3) duplicated vectors tie and come out by ascending index; (4) a brute-force
    double loop on a tiny case; (5) k beyond N returns all N."""
    rng = np.random.default_rng(11)
    d = 128
    signs = rng.choice([-1.0, 1.0], d)
    c, t = golden_codebooks[4]
    x = rng.standard_normal((40, d)) * rng.uniform(0.5, 3.0, (40, 1))
    codes, n16, _ = o.quantize(x, signs, c, t)
    q = rng.standard_normal((3, d))
    idx, sc, s_all = o.ip_search(q, codes, n16, signs, c, 7)
    rot = (q @ o.rotation_matrix(signs).T)                       # R q per query
    s_rot = n16.astype(np.float64)[None, :] * (rot @ np.asarray(c, dtype=np.float64)[codes].T)
    assert np.allclose(s_all, s_rot, rtol=0, atol=1e-11 * np.abs(s_rot).max())
    # (2) multiples of one direction: lambda_t = 1 + t / 8 is exact in fp16
    v = rng.standard_normal(d)
    lam = 1.0 + np.arange(24)[rng.permutation(24)] / 8.0
    cm, nm, _ = o.quantize(lam[:, None] * v[None, :], signs, c, t)
    assert np.all(cm == cm[0])
    i_up, _, _ = o.ip_search(v[None], cm, nm, signs, c, 5)
    i_dn, _, _ = o.ip_search(-v[None], cm, nm, signs, c, 5)
    assert list(i_up[0]) == list(np.argsort(-lam)[:5])
    assert list(i_dn[0]) == list(np.argsort(lam)[:5])
    # (3) ties: vector 5 repeated at 9 and 17
    x3 = x.copy()
    x3[9] = x3[5]
    x3[17] = x3[5]
    c3, n3, _ = o.quantize(x3, signs, c, t)
    qq = x3[5][None]
    i3, s3, _ = o.ip_search(qq, c3, n3, signs, c, 40)
    pos = [list(i3[0]).index(j) for j in (5, 9, 17)]
    assert s3[0][pos[0]] == s3[0][pos[1]] == s3[0][pos[2]]
    assert pos == sorted(pos) and pos[1] == pos[0] + 1 and pos[2] == pos[1] + 1
    # (4) brute force
    xh = o.dequantize(codes[:6], n16[:6], signs, c)
    qb = q[1]
    sb = [sum(qb[i] * xh[r][i] for i in range(d)) for r in range(6)]
    ib, _, _ = o.ip_search(qb[None], codes[:6], n16[:6], signs, c, 4)
    assert list(ib[0]) == sorted(range(6), key=lambda r: (-sb[r], r))[:4]
    # (5)
    i5, _, _ = o.ip_search(q[:1], codes[:3], n16[:3], signs, c, 10)
    assert i5.shape == (1, 3)

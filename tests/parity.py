"""Helpers that compare the HIP path with the CPU oracle (tests only).

Comparison rules (tolerances of the workload statement):
  packing   re-packing the GPU's own codes with the oracle packer reproduces the GPU bytes
  codes     GPU codes equal the oracle's except where the oracle's rotated value lies
            within 1e-6 of a codebook boundary (those are counted, not failed)
  norms     fp16 norms within 1e-3 relative
  scores    per (batch, head) row: max |ds| <= 1e-3 * max |s|
  outputs   per (batch, head): ||do|| <= 1e-3 * ||o|| (+ the Sparse-V borderline allowance)
Attention parity runs the oracle on the GPU-produced packed cache, so code flips near
boundaries cannot contaminate it.
"""
import math

import numpy as np

from oracle import tq_oracle as o

BAND = 1e-6
REL = 1e-3


def to_f64(t):
    """Exact fp64 copy of a torch tensor (fp32 / bf16 / fp16)."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def gpu_plane_codes(cache, b, h, n_tokens):
    """GPU codes [n_tokens, d] of one plane, unpacked with the oracle's unpacker."""
    raw = cache.plane_codes(b, h).cpu().numpy()
    nbytes = n_tokens * cache.d * cache.bits // 8
    return o.unpack(raw[:nbytes], n_tokens, cache.d, cache.bits, cache.layout), raw[:nbytes]


def gpu_plane_norms(cache, b, h, n_tokens):
    return cache.plane_norms(b, h)[:n_tokens].cpu().numpy()


def check_plane(cache, b, h, x64, start, signs, table, end=None):
    """Codes and norms of plane (b, h) at positions [start, start + n) against the oracle's
    quantization of x64 [n, d]; returns the number of near-boundary coordinates."""
    c, t = table
    n = x64.shape[0]
    end = start + n if end is None else end
    pad = (end + 7) // 8 * 8
    codes_g, raw = gpu_plane_codes(cache, b, h, pad)
    # packing is bit-exact: re-packing the GPU's own codes gives the GPU bytes
    assert np.array_equal(o.pack(codes_g, cache.bits, cache.layout), raw), (b, h)
    codes_o, n16_o, u = o.quantize(x64, signs, c, t)
    near = o.near_boundary_mask(u, t, BAND)
    got = codes_g[start:start + n]
    mism = (got != codes_o) & ~near
    assert not mism.any(), (b, h, np.argwhere(mism)[:5])
    n16_g = gpu_plane_norms(cache, b, h, end)[start:start + n].astype(np.float64)
    ref = n16_o.astype(np.float64)
    assert np.all(np.abs(n16_g - ref) <= REL * np.abs(ref) + 1e-30), (b, h)
    return int(near.sum())


def check_quantize(cache, x64, start, signs, table, written_upto=None, report=None):
    """x64: fp64 [batch, n, n_kv_heads, d] quantized into [start, start + n)."""
    bsz, n, hkv, d = x64.shape
    near_total = 0
    for b in range(bsz):
        for h in range(hkv):
            near_total += check_plane(cache, b, h, x64[b, :, h], start, signs, table, written_upto)
    if report is not None:
        report["near_boundary"] = report.get("near_boundary", 0) + near_total
    return near_total


def oracle_plane(cache, b, h, signs, table, n_tokens):
    """Dequantized plane (b, h) [n_tokens, d] computed by the oracle from the GPU codes."""
    c, _ = table
    pad = (n_tokens + 7) // 8 * 8
    codes, _ = gpu_plane_codes(cache, b, h, pad)
    n16 = gpu_plane_norms(cache, b, h, n_tokens).astype(np.float16)
    return o.dequantize(codes[:n_tokens], n16, signs, c)


def oracle_cache_view(cache, signs, table, n_tokens):
    """Dequantized cache [batch, n_kv_heads, n_tokens, d] computed by the oracle from the
    GPU-produced codes and norms."""
    out = np.zeros((cache.batch, cache.n_kv_heads, n_tokens, cache.d))
    for b in range(cache.batch):
        for h in range(cache.n_kv_heads):
            out[b, h] = oracle_plane(cache, b, h, signs, table, n_tokens)
    return out


def check_rows(got, ref, what, rel=REL, allowance=None):
    """Normwise per-row check on the last axis."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.linalg.norm(got - ref, axis=-1)
    lim = rel * np.linalg.norm(ref, axis=-1)
    if allowance is not None:
        lim = lim + allowance
    bad = err > lim + 1e-30
    assert not bad.any(), f"{what}: {np.argwhere(bad)[:5]} err={err[bad][:5]} lim={lim[bad][:5]}"
    return float(np.max(err / np.maximum(np.linalg.norm(ref, axis=-1), 1e-300)))


def check_scores(got, ref, seq_lens):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    worst = 0.0
    for b in range(ref.shape[0]):
        tb = ref.shape[2] if seq_lens is None else int(seq_lens[b])
        assert np.all(np.isneginf(got[b, :, tb:])), "scores past the sequence length must be -inf"
        if tb == 0:
            continue
        d = np.abs(got[b, :, :tb] - ref[b, :, :tb]).max(axis=-1)
        m = np.abs(ref[b, :, :tb]).max(axis=-1)
        assert np.all(d <= REL * m), (b, d / m)
        worst = max(worst, float((d / m).max()))
    return worst


def sparse_allowance(scores, lse, v_hat, tau, group):
    """sum over borderline rows of p_t ||v_hat_t|| per (b, h): either decision is allowed."""
    border = o.sparse_v_borderline(scores, lse, tau, REL)
    ok = np.isfinite(scores) & np.isfinite(lse)[..., None]
    p = np.where(ok, np.exp(np.where(ok, scores, 0.0) - np.where(ok, lse[..., None], 0.0)), 0.0)
    vn = np.linalg.norm(v_hat, axis=-1)                # [B, Hkv, T]
    vn_q = np.repeat(vn, group, axis=1)                # [B, Hq, T]
    return (p * border * vn_q).sum(-1), int(border.sum())


def check_qjl_plane(cache, sketch, b, h, x64, start, signs, table, proj64):
    """QJL keys of plane (b, h) at positions [start, start + n): codes and norms as
    check_plane; on every token whose codes all equal the oracle's, the sign bits equal the
    oracle's except where the projection is within 1e-5 ||S_j|| ||r|| of zero, and the fp16
    residual norm is within 1e-3 relative.  (A code flip inside the boundary band moves the
    residual by a centroid step and so may move many of its signs: such tokens are counted.)
    Returns (near-boundary coordinates, near-zero sign bits, tokens with a code flip)."""
    c, t = table
    n = x64.shape[0]
    near = check_plane(cache, b, h, x64, start, signs, table)
    codes_g, _ = gpu_plane_codes(cache, b, h, start + n)
    codes_g = codes_g[start:start + n]
    codes_o, n16_o, sig_o, rn16_o, u, z, rn = o.qjl_quantize(x64, signs, c, t, proj64)
    m = proj64.shape[0]
    raw = sketch.plane_bits(b, h).cpu().numpy()[: (start + n) * m // 8]
    sig_g = o.unpack(raw, start + n, m, 1, o.LAYOUT_ROWS)[start:].astype(bool)
    same = np.all(codes_g == codes_o, axis=-1)
    zero_band = o.qjl_near_zero_mask(z, rn, proj64, 1e-5)
    bad = (sig_g != sig_o) & ~zero_band & same[:, None]
    assert not bad.any(), (b, h, np.argwhere(bad)[:5])
    rn_g = sketch.plane_res_norms(b, h)[start:start + n].cpu().numpy().astype(np.float64)
    ref = rn16_o.astype(np.float64)
    ok = np.abs(rn_g - ref) <= REL * np.abs(ref) + 1e-30
    assert np.all(ok | ~same), (b, h, np.argwhere(~ok & same)[:5])
    return near, int((zero_band & same[:, None]).sum()), int((~same).sum())


def oracle_qjl_view(cache, sketch, signs, table, proj64, n_tokens):
    """Effective QJL keys [batch, n_kv_heads, n_tokens, d] computed by the oracle from the
    GPU-written codes, norms, sign bits and residual norms."""
    c, _ = table
    m = proj64.shape[0]
    out = np.zeros((cache.batch, cache.n_kv_heads, n_tokens, cache.d))
    for b in range(cache.batch):
        for h in range(cache.n_kv_heads):
            codes, _ = gpu_plane_codes(cache, b, h, n_tokens)
            n16 = gpu_plane_norms(cache, b, h, n_tokens).astype(np.float16)
            raw = sketch.plane_bits(b, h).cpu().numpy()[: n_tokens * m // 8]
            sig = o.unpack(raw, n_tokens, m, 1, o.LAYOUT_ROWS).astype(bool)
            rn16 = sketch.plane_res_norms(b, h)[:n_tokens].cpu().numpy().astype(np.float16)
            out[b, h] = o.qjl_dequantize(codes, n16, sig, rn16, signs, c, proj64)
    return out

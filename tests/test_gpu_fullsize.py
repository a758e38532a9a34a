"""Parity at the full workload sizes, in the launch configuration the benchmark times.

The oracle cannot take whole outputs at these sizes, so sampled outputs are compared:
  decode    a few (batch, query head) rows of attention (output and LSE) against the
            oracle's attention over its dequantization of the GPU-written planes, and the
            codes and norms of those planes against the oracle's quantizer;
  prefill   a boundary (8/8-bit) layer and a middle (K4/V3) layer of the 32768-token
            cache, two kv-head planes each, against the oracle's quantizer;
  chunk     two kv heads' rows of a 512-position prefill chunk;
  QJL       three kv heads' rows and scores of the QJL decode step, and the new key's codes
            and sign bits.
Caches, queries and launches are those of the benchmark: the context minus one token is
appended, then the last token goes in with the attention (one fused append-and-attend launch
for dense decode, the key-and-value append and the decode call for Sparse V); the paged and
multi-query lines likewise use their benchmark's calls.
"""
import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import compressed_decode_attention_tq_amd as tq  # noqa: E402
from compressed_decode_attention_tq_amd import inputs  # noqa: E402
from oracle import tq_oracle as o  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("workload,tau", [("llama8k", 0.0), ("batch32k", 0.0), ("batch32k", 1e-4),
                                          ("ctx131k", 0.0), ("ctx131k", 1e-4)])
def test_decode_full_size_sampled(workload, tau, golden_codebooks):
    w = inputs.WORKLOADS[workload]
    _say("full-size decode", workload, tau)
    batch, hq, hkv, ctx, g = w.batch, w.n_q_heads, w.n_kv_heads, w.ctx, w.group
    signs = inputs.rotation_signs()
    sd = signs.to(DEV)
    x = inputs.generate(w, device=DEV)
    kc = tq.PackedCache(batch, hkv, ctx, w.bits_k, tq.LAYOUT_ROWS, sd, device=DEV)
    vc = tq.PackedCache(batch, hkv, ctx, w.bits_v, tq.LAYOUT_GROUP8, sd, device=DEV)
    tq.quantize_append(kc, x["k"][:, : ctx - 1].contiguous(), 0)
    tq.quantize_append(vc, x["v"][:, : ctx - 1].contiguous(), 0)
    k_new, v_new = x["k"][:, ctx - 1:].contiguous(), x["v"][:, ctx - 1:].contiguous()
    q = x["q"].contiguous()
    scale = 1.0 / math.sqrt(128)
    bufs = tq.DecodeBuffers(batch, hq, hkv, ctx, tau, device=DEV)
    if tau == 0.0:
        tq.decode_attn_append(kc, vc, k_new, v_new, q, ctx, scale, buffers=bufs)
    else:
        tq.quantize_append_kv(kc, vc, k_new, v_new, ctx - 1)
        tq.decode_attn(kc, vc, q, ctx, scale, tau=tau, buffers=bufs)
    torch.cuda.synchronize()
    out_g, lse_g = bufs.out.cpu().numpy(), bufs.lse.cpu().numpy()
    # the scores output on the same cache (a call of its own: the benchmark's call writes none)
    sbuf = tq.decode_attn(kc, vc, q, ctx, scale, tau=tau, want_scores=True)
    torch.cuda.synchronize()
    s64 = signs.numpy().astype(np.float64)
    rng = np.random.default_rng(w.seed)
    rows = {(0, 0), (batch - 1, hq - 1), (batch // 2, min(hq - 1, hq // 2 + 1))}
    rows |= {(int(rng.integers(batch)), int(rng.integers(hq))) for _ in range(5)}
    checked = set()
    for b, h in sorted(rows):
        kvh = h // g
        kh = parity.oracle_plane(kc, b, kvh, s64, golden_codebooks[w.bits_k], ctx)
        vh = parity.oracle_plane(vc, b, kvh, s64, golden_codebooks[w.bits_v], ctx)
        q64 = parity.to_f64(q[b, h])
        out, lse, scores = o.decode_attention(q64[None, None], kh[None, None], vh[None, None], scale, tau=tau)
        allowance, nb = (None, 0)
        if tau > 0:
            allowance, nb = parity.sparse_allowance(scores, lse, vh[None, None], tau, 1)
        worst = parity.check_rows(out_g[b, h][None, None], out, f"out[{b},{h}]", allowance=allowance)
        assert abs(lse_g[b, h] - lse[0, 0]) <= 1e-3 * max(1.0, abs(lse[0, 0])), (b, h, lse_g[b, h], lse[0, 0])
        sw = parity.check_scores(sbuf.scores[b, h].cpu().numpy()[None, None], scores, None)
        _say(f"  row ({b},{h}): rel err {worst:.2e}, borderline rows {nb}, scores {sw:.1e}")
        if (b, kvh) in checked:
            continue
        checked.add((b, kvh))
        for cache, xx, bits in ((kc, x["k"], w.bits_k), (vc, x["v"], w.bits_v)):
            near = parity.check_plane(cache, b, kvh, parity.to_f64(xx[b, :, kvh]), 0, s64, golden_codebooks[bits])
            _say(f"  plane ({b},{kvh}) {bits}-bit: near-boundary coordinates {near}")


@pytest.mark.parametrize("layer", [0, 5])
def test_prefill_layer_full_size_sampled(layer, golden_codebooks):
    w = inputs.WORKLOADS["prefill"]
    bk, bv = inputs.layer_bits(w, layer)
    _say("full-size prefill layer", layer, bk, bv)
    signs = inputs.rotation_signs()
    sd = signs.to(DEV)
    x = inputs.generate(w, device=DEV, layer=layer, with_query=False)
    k, v = x["k"].contiguous(), x["v"].contiguous()
    kc = tq.PackedCache(1, w.n_kv_heads, w.ctx, bk, tq.LAYOUT_ROWS, sd, device=DEV)
    vc = tq.PackedCache(1, w.n_kv_heads, w.ctx, bv, tq.LAYOUT_GROUP8, sd, device=DEV)
    tq.quantize_append_kv(kc, vc, k, v, 0)
    torch.cuda.synchronize()
    s64 = signs.numpy().astype(np.float64)
    for h in (0, w.n_kv_heads - 1):
        for cache, xx, bits in ((kc, k, bk), (vc, v, bv)):
            near = parity.check_plane(cache, 0, h, parity.to_f64(xx[0, :, h]), 0, s64, golden_codebooks[bits])
            _say(f"  plane (0,{h}) {bits}-bit: near-boundary coordinates {near}")


def test_paged_full_size_sampled(golden_codebooks):
    """paged32k: the batched long-context shape in 256-token pages in random pool order,
    filled through the paged append, then the last token appended and attended in the one
    fused paged launch the benchmark times."""
    w = inputs.WORKLOADS["paged32k"]
    _say("full-size paged decode")
    batch, hq, hkv, ctx, g, P = w.batch, w.n_q_heads, w.n_kv_heads, w.ctx, w.group, w.page_tokens
    signs = inputs.rotation_signs()
    sd = signs.to(DEV)
    x = inputs.generate(w, device=DEV)
    max_pages = ctx // P
    n_pages = batch * max_pages
    rng = np.random.default_rng(w.seed)
    table = torch.tensor(rng.permutation(n_pages).reshape(batch, max_pages), dtype=torch.int32, device=DEV)
    kc = tq.PagedCache(batch, hkv, P, n_pages, max_pages, w.bits_k, tq.LAYOUT_ROWS, sd, block_table=table,
                       device=DEV)
    vc = tq.PagedCache(batch, hkv, P, n_pages, max_pages, w.bits_v, tq.LAYOUT_GROUP8, sd, block_table=table,
                       device=DEV)
    zeros = torch.zeros(batch, dtype=torch.int32, device=DEV)
    tq.paged_quantize_append_kv(kc, vc, x["k"][:, : ctx - 1].contiguous(), x["v"][:, : ctx - 1].contiguous(), zeros)
    q = x["q"].contiguous()
    scale = 1.0 / math.sqrt(128)
    lens = torch.full((batch,), ctx, dtype=torch.int32, device=DEV)
    got = tq.paged_decode_attn_append(kc, vc, x["k"][:, ctx - 1:].contiguous(), x["v"][:, ctx - 1:].contiguous(), q,
                                      lens, ctx, scale)
    torch.cuda.synchronize()
    out_g, lse_g = got.out.cpu().numpy(), got.lse.cpu().numpy()
    s64 = signs.numpy().astype(np.float64)
    tab = table.cpu().numpy()
    rows = {(0, 0), (batch - 1, hq - 1), (batch // 2, hq // 2 + 1)}
    rows |= {(int(rng.integers(batch)), int(rng.integers(hq))) for _ in range(3)}
    for b, h in sorted(rows):
        kvh = h // g
        planes = []
        for cache, bits, xx in ((kc, w.bits_k, x["k"]), (vc, w.bits_v, x["v"])):
            flat = tq.PackedCache(1, 1, ctx, bits, cache.layout, sd, device=DEV)
            per = P * 16 * bits
            for slot in range(max_pages):
                flat.codes[slot * per:(slot + 1) * per] = cache.page_codes(int(tab[b, slot]), kvh)
                flat.norms[slot * P:(slot + 1) * P] = cache.page_norms(int(tab[b, slot]), kvh)
            near = parity.check_plane(flat, 0, 0, parity.to_f64(xx[b, :, kvh]), 0, s64, golden_codebooks[bits])
            _say(f"  plane ({b},{kvh}) {bits}-bit: near-boundary coordinates {near}")
            planes.append(parity.oracle_plane(flat, 0, 0, s64, golden_codebooks[bits], ctx))
        q64 = parity.to_f64(q[b, h])
        out, lse, _ = o.decode_attention(q64[None, None], planes[0][None, None], planes[1][None, None], scale)
        worst = parity.check_rows(out_g[b, h][None, None], out, f"out[{b},{h}]")
        assert abs(lse_g[b, h] - lse[0, 0]) <= 1e-3 * max(1.0, abs(lse[0, 0])), (b, h)
        _say(f"  row ({b},{h}): rel err {worst:.2e}")


def test_verify_full_size_sampled(golden_codebooks):
    """verify8k: 4 positions appended through the key-and-value append, then causal
    multi-query attention over the 8192-token cache."""
    w = inputs.WORKLOADS["verify8k"]
    _say("full-size multi-query")
    batch, hq, hkv, ctx, g, n_q = w.batch, w.n_q_heads, w.n_kv_heads, w.ctx, w.group, w.n_q
    signs = inputs.rotation_signs()
    sd = signs.to(DEV)
    x = inputs.generate(w, device=DEV)
    kc = tq.PackedCache(batch, hkv, ctx, w.bits_k, tq.LAYOUT_ROWS, sd, device=DEV)
    vc = tq.PackedCache(batch, hkv, ctx, w.bits_v, tq.LAYOUT_GROUP8, sd, device=DEV)
    tq.quantize_append(kc, x["k"][:, : ctx - n_q].contiguous(), 0)
    tq.quantize_append(vc, x["v"][:, : ctx - n_q].contiguous(), 0)
    tq.quantize_append_kv(kc, vc, x["k"][:, ctx - n_q:].contiguous(), x["v"][:, ctx - n_q:].contiguous(), ctx - n_q)
    q = x["q"].contiguous()
    scale = 1.0 / math.sqrt(128)
    got = tq.decode_attn_multi(kc, vc, q, ctx, scale)
    torch.cuda.synchronize()
    out_g, lse_g = got.out.cpu().numpy(), got.lse.cpu().numpy()
    s64 = signs.numpy().astype(np.float64)
    for kvh in (0, hkv - 1):
        kh = parity.oracle_plane(kc, 0, kvh, s64, golden_codebooks[w.bits_k], ctx)
        vh = parity.oracle_plane(vc, 0, kvh, s64, golden_codebooks[w.bits_v], ctx)
        heads = list(range(kvh * g, (kvh + 1) * g))
        q64 = parity.to_f64(q[0][:, heads])[None]                     # [1, n_q, g, d]
        out, lse = o.multi_query_attention(q64, kh[None, None], vh[None, None], scale)
        worst = parity.check_rows(out_g[0][:, heads], out[0], f"multi out kv head {kvh}")
        assert np.allclose(lse_g[0][:, heads], lse[0], rtol=0, atol=1e-3 * np.maximum(1, np.abs(lse[0])))
        _say(f"  kv head {kvh}: rel err {worst:.2e}")


def test_chunk_full_size_sampled(golden_codebooks):
    """chunk8k: a 512-position prefill chunk appended through the key-and-value append, then
    causal multi-query attention over the 8192-token cache in prefill mode (8 row groups per
    workgroup), the benchmark's calls; two kv heads' 512 x 4 rows against the oracle."""
    w = inputs.WORKLOADS["chunk8k"]
    _say("full-size prefill chunk")
    batch, hq, hkv, ctx, g, n_q = w.batch, w.n_q_heads, w.n_kv_heads, w.ctx, w.group, w.n_q
    signs = inputs.rotation_signs()
    sd = signs.to(DEV)
    x = inputs.generate(w, device=DEV)
    kc = tq.PackedCache(batch, hkv, ctx, w.bits_k, tq.LAYOUT_ROWS, sd, device=DEV)
    vc = tq.PackedCache(batch, hkv, ctx, w.bits_v, tq.LAYOUT_GROUP8, sd, device=DEV)
    tq.quantize_append(kc, x["k"][:, : ctx - n_q].contiguous(), 0)
    tq.quantize_append(vc, x["v"][:, : ctx - n_q].contiguous(), 0)
    tq.quantize_append_kv(kc, vc, x["k"][:, ctx - n_q:].contiguous(), x["v"][:, ctx - n_q:].contiguous(), ctx - n_q)
    q = x["q"].contiguous()
    scale = 1.0 / math.sqrt(128)
    got = tq.decode_attn_multi(kc, vc, q, ctx, scale)
    torch.cuda.synchronize()
    out_g, lse_g = got.out.cpu().numpy(), got.lse.cpu().numpy()
    s64 = signs.numpy().astype(np.float64)
    for kvh in (0, hkv - 1):
        kh = parity.oracle_plane(kc, 0, kvh, s64, golden_codebooks[w.bits_k], ctx)
        vh = parity.oracle_plane(vc, 0, kvh, s64, golden_codebooks[w.bits_v], ctx)
        heads = list(range(kvh * g, (kvh + 1) * g))
        q64 = parity.to_f64(q[0][:, heads])[None]                     # [1, n_q, g, d]
        out, lse = o.multi_query_attention(q64, kh[None, None], vh[None, None], scale)
        worst = parity.check_rows(out_g[0][:, heads], out[0], f"chunk out kv head {kvh}")
        assert np.allclose(lse_g[0][:, heads], lse[0], rtol=0, atol=1e-3 * np.maximum(1, np.abs(lse[0])))
        _say(f"  kv head {kvh}: rel err {worst:.2e}")


def test_qjl_full_size_sampled(golden_codebooks):
    """qjl8k: 8191 keys through the QJL quantize and values through the quantize, the last token
    through the step's own append (keys and values in one launch), then the QJL decode on matrix cores
    with scores; three kv heads' query heads against the oracle's attention over its effective
    keys from the GPU-written codes, sign bits and norms, and the new key against the oracle's
    QJL quantizer."""
    w = inputs.WORKLOADS["qjl8k"]
    _say("full-size QJL decode")
    batch, hq, hkv, ctx, g, m = w.batch, w.n_q_heads, w.n_kv_heads, w.ctx, w.group, w.extra["qjl_m"]
    signs = inputs.rotation_signs()
    sd = signs.to(DEV)
    proj = inputs.qjl_projection(m)
    x = inputs.generate(w, device=DEV)
    kc = tq.PackedCache(batch, hkv, ctx, w.bits_k, tq.LAYOUT_ROWS, sd, device=DEV)
    vc = tq.PackedCache(batch, hkv, ctx, w.bits_v, tq.LAYOUT_GROUP8, sd, device=DEV)
    sk = tq.QjlSketch(kc, proj, device=DEV)
    tq.qjl_quantize_append(kc, sk, x["k"][:, : ctx - 1].contiguous(), 0)
    tq.quantize_append(vc, x["v"][:, : ctx - 1].contiguous(), 0)
    tq.qjl_quantize_append_kv(kc, sk, vc, x["k"][:, ctx - 1:].contiguous(), x["v"][:, ctx - 1:].contiguous(),
                              ctx - 1)
    q = x["q"].contiguous()
    scale = 1.0 / math.sqrt(128)
    got = tq.qjl_decode_attn(kc, sk, vc, q, ctx, scale, want_scores=True)
    torch.cuda.synchronize()
    out_g, lse_g, sc_g = got.out.cpu().numpy(), got.lse.cpu().numpy(), got.scores.cpu().numpy()
    s64 = signs.numpy().astype(np.float64)
    p64 = proj.numpy().astype(np.float64)
    c, _ = golden_codebooks[w.bits_k]
    for kvh in (0, 3, hkv - 1):
        codes, _ = parity.gpu_plane_codes(kc, 0, kvh, ctx)
        n16 = parity.gpu_plane_norms(kc, 0, kvh, ctx).astype(np.float16)
        raw = sk.plane_bits(0, kvh).cpu().numpy()[: ctx * m // 8]
        sig = o.unpack(raw, ctx, m, 1, o.LAYOUT_ROWS).astype(bool)
        rn16 = sk.plane_res_norms(0, kvh)[:ctx].cpu().numpy().astype(np.float16)
        kh = o.qjl_dequantize(codes, n16, sig, rn16, s64, c, p64)
        vh = parity.oracle_plane(vc, 0, kvh, s64, golden_codebooks[w.bits_v], ctx)
        heads = list(range(kvh * g, (kvh + 1) * g))
        q64 = parity.to_f64(q[0][heads])[None]                        # [1, g, d]
        out, lse, scores = o.decode_attention(q64, kh[None, None], vh[None, None], scale)
        parity.check_scores(sc_g[0][heads][None], scores, None)
        worst = parity.check_rows(out_g[0][heads][None], out, f"qjl out kv head {kvh}")
        assert np.allclose(lse_g[0][heads], lse[0], rtol=0, atol=1e-3 * np.maximum(1, np.abs(lse[0])))
        xk = parity.to_f64(x["k"][0, ctx - 1:, kvh])
        r = parity.check_qjl_plane(kc, sk, 0, kvh, xk, ctx - 1, s64, golden_codebooks[w.bits_k], p64)
        _say(f"  kv head {kvh}: rel err {worst:.2e}; new key: near-boundary {r[0]}, near-zero bits {r[1]}")


def test_search_full_size(golden_codebooks):
    """search1m: 8 queries over 2^20 quantized vectors, the benchmark's call; the oracle ranks
    the whole database from the GPU-written codes and norms."""
    spec = inputs.SEARCH["search1m"]
    _say("full-size search")
    n, nq, k, bits = spec["n"], spec["n_queries"], spec["top_k"], spec["bits"]
    signs = inputs.rotation_signs()
    g = inputs.generate_search(spec, device=DEV)
    db = tq.PackedCache(1, 1, n, bits, tq.LAYOUT_ROWS, signs.to(DEV), device=DEV)
    tq.quantize_append(db, g["x"][None, :, None, :].contiguous(), 0)
    res = tq.ip_search(db, g["q"].contiguous(), n, k)
    torch.cuda.synchronize()
    s64 = signs.numpy().astype(np.float64)
    c, _ = golden_codebooks[bits]
    codes = o.unpack(db.plane_codes(0, 0).cpu().numpy(), n, 128, bits, 0)
    n16 = db.plane_norms(0, 0).cpu().numpy().astype(np.float16)
    idx_o, sc_o, s_all = o.ip_search(parity.to_f64(g["q"]), codes, n16, s64, c, k)
    idx_g, sc_g = res.idx.cpu().numpy(), res.score.cpu().numpy()
    for j in range(nq):
        tol = 1e-3 * np.abs(s_all[j]).max()
        assert np.all(np.abs(sc_g[j] - s_all[j][idx_g[j]]) <= tol), j
        kth = sc_o[j, k - 1]
        assert np.all(s_all[j][idx_g[j]] >= kth - 2 * tol), j
        assert set(np.nonzero(s_all[j] > kth + 2 * tol)[0].tolist()) <= set(idx_g[j].tolist()), j
        _say(f"  query {j}: {len(set(idx_g[j].tolist()) & set(idx_o[j].tolist()))}/{k} of the oracle's top {k}")

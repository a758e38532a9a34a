"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Sizes are ones the oracle finishes in seconds but that still span several 64-token chunks,
several 256-token decode steps and splits, and ragged tails.
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


@pytest.fixture(scope="module")
def signs():
    return inputs.rotation_signs()


def _table(golden, bits):
    return golden[bits]


_SIGNS_DEV = {}


def _new_cache(batch, hkv, cap, bits, layout, signs):
    key = tuple(signs.tolist())
    if key not in _SIGNS_DEV:
        _SIGNS_DEV[key] = signs.to(DEV)
    return tq.PackedCache(batch, hkv, cap, bits, layout, _SIGNS_DEV[key], device=DEV)


def _fill(cache, x, start=0):
    tq.quantize_append(cache, x, start)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ quantize


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_quantize_matches_oracle(bits, layout, dtype, signs, golden_codebooks):
    _say("quantize", bits, layout, dtype)
    w = inputs.WORKLOADS["llama8k"]
    g = inputs.generate(w, device="cpu", batch=2, ctx=200, n_kv_heads=3, with_query=False)
    x = g["k"].to({"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}[dtype])
    cache = _new_cache(2, 3, 256, bits, layout, signs)
    _fill(cache, x.to(DEV))
    s64 = signs.numpy().astype(np.float64)
    parity.check_quantize(cache, parity.to_f64(x), 0, s64, _table(golden_codebooks, bits))


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("bits", [2, 3])
def test_append_in_pieces_keeps_earlier_tokens(layout, bits, signs, golden_codebooks):
    """Ragged appends (including single tokens inside an 8-token group) read-modify-write
    the edges of the range and leave every other position untouched."""
    _say("append pieces", layout, bits)
    w = inputs.WORKLOADS["batch32k"]
    g = inputs.generate(w, device="cpu", batch=2, ctx=203, n_kv_heads=2, with_query=False)
    x = g["v"]
    cache = _new_cache(2, 2, 256, bits, layout, signs)
    for a, e in [(0, 37), (37, 38), (38, 101), (101, 190), (190, 191), (191, 203)]:
        tq.quantize_append(cache, x[:, a:e].contiguous().to(DEV), a)
    torch.cuda.synchronize()
    s64 = signs.numpy().astype(np.float64)
    parity.check_quantize(cache, parity.to_f64(x), 0, s64, _table(golden_codebooks, bits))


@pytest.mark.parametrize("bits_k,bits_v,dtype", [(4, 2, "bf16"), (3, 2, "f16"), (4, 3, "f32"), (8, 8, "bf16"),
                                                (2, 4, "f16")])
def test_quantize_append_kv_equals_two_appends(bits_k, bits_v, dtype, signs, golden_codebooks):
    """The one-launch key-and-value append writes exactly what two single-cache appends write,
    over ragged ranges that start and end inside 8-token groups and 64-token chunks."""
    _say("append kv", bits_k, bits_v, dtype)
    w = inputs.WORKLOADS["llama8k"]
    g = inputs.generate(w, device="cpu", batch=2, ctx=150, n_kv_heads=3, with_query=False)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    k, v = g["k"].to(tdt), g["v"].to(tdt)
    one = (_new_cache(2, 3, 192, bits_k, 0, signs), _new_cache(2, 3, 192, bits_v, 1, signs))
    two = (_new_cache(2, 3, 192, bits_k, 0, signs), _new_cache(2, 3, 192, bits_v, 1, signs))
    for c in one + two:  # the same stale contents outside the written ranges
        c.codes.fill_(0xA5)
        c.norms.fill_(0x3C00)
    for a, e in [(0, 5), (5, 70), (70, 71), (71, 150)]:
        ks, vs = k[:, a:e].contiguous().to(DEV), v[:, a:e].contiguous().to(DEV)
        tq.quantize_append_kv(one[0], one[1], ks, vs, a)
        tq.quantize_append(two[0], ks, a)
        tq.quantize_append(two[1], vs, a)
    torch.cuda.synchronize()
    for c1, c2 in zip(one, two):
        assert torch.equal(c1.codes, c2.codes)
        assert torch.equal(c1.norms, c2.norms)
    s64 = signs.numpy().astype(np.float64)
    if dtype == "f32":
        parity.check_quantize(one[0], parity.to_f64(g["k"]), 0, s64, _table(golden_codebooks, bits_k))
        parity.check_quantize(one[1], parity.to_f64(g["v"]), 0, s64, _table(golden_codebooks, bits_v))


@pytest.mark.parametrize("bits_k,bits_v,dtype,single", [(4, 2, "bf16", False), (3, 2, "f32", False),
                                                       (2, 4, "f16", False), (8, 3, "bf16", False),
                                                       (4, 8, "f32", False), (3, 2, "bf16", True),
                                                       (4, 3, "f16", True), (8, 2, "f32", True)])
def test_small_appends_match_oracle(bits_k, bits_v, dtype, single, signs, golden_codebooks):
    """Appends of 1..8 tokens (one wave per plane, tokens in order) against the oracle, over
    ranges that start, end and cross inside 8-token value groups; everything outside the
    written positions keeps its stale contents.  `single`: each cache through its own
    tq_quantize_append call (the same kernel, one cache)."""
    _say("small appends", bits_k, bits_v, dtype, single)
    w = inputs.WORKLOADS["llama8k"]
    g = inputs.generate(w, device="cpu", batch=2, ctx=61, n_kv_heads=3, with_query=False)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    k, v = g["k"].to(tdt), g["v"].to(tdt)
    kc, vc = _new_cache(2, 3, 128, bits_k, 0, signs), _new_cache(2, 3, 128, bits_v, 1, signs)
    for c in (kc, vc):
        c.codes.fill_(0xA5)
        c.norms.fill_(0x3C00)
    edges = [0, 1, 4, 12, 13, 21, 22, 30, 37, 45, 46, 53, 61]
    for a, e in zip(edges[:-1], edges[1:]):
        assert 1 <= e - a <= 8
        if single:
            tq.quantize_append(kc, k[:, a:e].contiguous().to(DEV), a)
            tq.quantize_append(vc, v[:, a:e].contiguous().to(DEV), a)
        else:
            tq.quantize_append_kv(kc, vc, k[:, a:e].contiguous().to(DEV), v[:, a:e].contiguous().to(DEV), a)
    torch.cuda.synchronize()
    s64 = signs.numpy().astype(np.float64)
    parity.check_quantize(kc, parity.to_f64(k), 0, s64, _table(golden_codebooks, bits_k))
    parity.check_quantize(vc, parity.to_f64(v), 0, s64, _table(golden_codebooks, bits_v))
    for c, bits in ((kc, bits_k), (vc, bits_v)):
        for b in range(2):
            for h in range(3):
                raw = c.plane_codes(b, h).cpu().numpy()
                tail = 64 * 16 * bits if c.layout == 1 else 61 * 16 * bits   # past the last group / row
                assert np.all(raw[tail:] == 0xA5), (b, h)
                assert np.all(c.plane_norms(b, h)[61:].cpu().numpy() == 0x3C00), (b, h)
        if c.layout == 1:  # positions 61..63 share the last value group: their codes are kept
            for b in range(2):
                for h in range(3):
                    got = o.unpack(c.plane_codes(b, h).cpu().numpy()[:64 * 16 * bits], 64, 128, bits, 1)
                    stale = o.unpack(np.full(64 * 16 * bits, 0xA5, dtype=np.uint8), 64, 128, bits, 1)
                    assert np.array_equal(got[61:], stale[61:]), (b, h)


def test_quantize_special_vectors(signs, golden_codebooks):
    """Basis vectors, the all-ones vector (exact ties on the middle boundary) and zeros."""
    _say("special vectors")
    x = torch.zeros((1, 64, 1, 128), dtype=torch.float32)
    for j in range(60):
        x[0, j, 0, (j * 37) % 128] = 1.0 + j
    x[0, 60, 0, :] = 1.0
    x[0, 62, 0, :] = -2.0
    plus = torch.ones(128, dtype=torch.int8)
    for bits in (2, 3, 4, 8):
        cache = _new_cache(1, 1, 64, bits, 0, plus)
        _fill(cache, x.to(DEV))
        codes, _ = parity.gpu_plane_codes(cache, 0, 0, 64)
        c, t = _table(golden_codebooks, bits)
        ref, n16, _ = o.quantize(parity.to_f64(x)[0, :, 0], np.ones(128), c, t)
        assert np.array_equal(codes, ref)          # no value is near a boundary except exact ties
        levels = 1 << bits
        assert codes[60, 0] == levels - 1 and np.all(codes[60, 1:] == levels // 2 - 1)
        assert np.all(codes[61] == levels // 2 - 1)      # zero vector
        norms = parity.gpu_plane_norms(cache, 0, 0, 64).astype(np.float64)
        assert norms[61] == 0.0 and norms[60] == float(np.float16(math.sqrt(128)))
        assert np.array_equal(norms[:60], 1.0 + np.arange(60))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_quantize_tiny_and_wide_range_inputs(dtype, signs, golden_codebooks):
    """16-bit inputs whose entries span many orders of magnitude: fp16 vectors with half of
    the entries in the subnormal range (below 6.1e-5), fp16 vectors that are subnormal
    throughout, and bf16 vectors with entries from 1e-30 to 1e3.  Every input value must
    reach the rotation unchanged (no flushing of subnormal inputs)."""
    _say("tiny inputs", dtype)
    g = torch.Generator().manual_seed(11)
    x = torch.randn((2, 128, 3, 128), generator=g, dtype=torch.float64)
    if dtype == "f16":
        x[:, :64, :, 64:] *= 3e-6            # subnormal halves next to normal values
        x[:, 64:96] *= 2e-6                  # subnormal throughout
        x[:, 96:] *= 1e-4 * torch.rand((2, 32, 3, 128), generator=g, dtype=torch.float64)
        tx = x.to(torch.float16)
    else:
        e = torch.randint(-30, 4, (2, 128, 3, 128), generator=g).to(torch.float64)
        tx = (x * torch.pow(10.0, e)).to(torch.bfloat16)
    for bits, layout in ((4, 0), (3, 1), (2, 0), (8, 1)):
        cache = _new_cache(2, 3, 128, bits, layout, signs)
        _fill(cache, tx.to(DEV))
        s64 = signs.numpy().astype(np.float64)
        parity.check_quantize(cache, parity.to_f64(tx), 0, s64, _table(golden_codebooks, bits))


@pytest.mark.parametrize("layout", [0, 1])
def test_dequantize_matches_oracle(layout, signs, golden_codebooks):
    _say("dequantize", layout)
    w = inputs.WORKLOADS["llama8k"]
    g = inputs.generate(w, device="cpu", batch=2, ctx=150, n_kv_heads=2, with_query=False)
    for bits in (2, 4, 8):
        cache = _new_cache(2, 2, 192, bits, layout, signs)
        _fill(cache, g["k"].to(DEV))
        got = tq.dequantize(cache, 10, 130)
        torch.cuda.synchronize()
        ref = parity.oracle_cache_view(cache, signs.numpy().astype(np.float64),
                                       _table(golden_codebooks, bits), 140)[:, :, 10:140]
        parity.check_rows(parity.to_f64(got).transpose(0, 2, 1, 3), ref, f"dequantize b{bits}")


# ------------------------------------------------------------------ decode


def _decode_case(w, signs, golden, batch, hq, hkv, ctx, cap, bits_k, bits_v, tau=0.0,
                 seq_lens=None, q_dtype=None, scale=None, want_caches=False):
    g = inputs.generate(w, device="cpu", batch=batch, ctx=ctx, n_kv_heads=hkv, n_q_heads=hq)
    kc = _new_cache(batch, hkv, cap, bits_k, 0, signs)
    vc = _new_cache(batch, hkv, cap, bits_v, 1, signs)
    _fill(kc, g["k"].to(DEV))
    _fill(vc, g["v"].to(DEV))
    q = g["q"] if q_dtype is None else g["q"].to(q_dtype)
    scale = 1.0 / math.sqrt(128) if scale is None else scale
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    buf = tq.decode_attn(kc, vc, q.to(DEV).contiguous(), ctx, scale, tau=tau, seq_lens=sl,
                         want_scores=True)
    torch.cuda.synchronize()
    s64 = signs.numpy().astype(np.float64)
    kh = parity.oracle_cache_view(kc, s64, golden[bits_k], ctx)
    vh = parity.oracle_cache_view(vc, s64, golden[bits_v], ctx)
    out, lse, scores = o.decode_attention(parity.to_f64(q), kh, vh, scale, seq_lens=seq_lens, tau=tau)
    got_scores = buf.scores.cpu().numpy()
    parity.check_scores(got_scores, scores, seq_lens)
    fin = np.isfinite(lse)
    assert np.all(np.isneginf(buf.lse.cpu().numpy()[~fin]))
    assert np.allclose(buf.lse.cpu().numpy()[fin], lse[fin], rtol=0, atol=1e-3 * np.maximum(1, np.abs(lse[fin])))
    allowance, nb = None, 0
    if tau > 0:
        allowance, nb = parity.sparse_allowance(scores, lse, vh, tau, hq // hkv)
    worst = parity.check_rows(buf.out.cpu().numpy(), out, "decode out", allowance=allowance)
    _say(f"  worst rel err {worst:.2e} borderline {nb}")
    if want_caches:
        return buf, out, (kc, vc, g)
    return buf, out


def test_decode_tiny_workload(signs, golden_codebooks):
    """The smallest workload exactly as stated: 1 kv head, 1 query head, 1024 fp32 tokens with
    4 outlier channels x10, K 4-bit and V 2-bit, fp32 query, scale 1/sqrt(128), no Sparse V.
    Every code and norm of the 1024 keys and values is checked against the oracle's own
    quantization (code mismatches allowed only within 1e-6 of a boundary, counted), then the
    attention against the oracle on the GPU-written cache, and end to end against the oracle
    on its own cache."""
    _say("decode tiny")
    w = inputs.WORKLOADS["tiny"]
    buf, out, (kc, vc, g) = _decode_case(w, signs, golden_codebooks, 1, 1, 1, 1024, 1024, 4, 2,
                                         want_caches=True)
    s64 = signs.numpy().astype(np.float64)
    k64, v64 = parity.to_f64(g["k"]), parity.to_f64(g["v"])
    near_k = parity.check_quantize(kc, k64, 0, s64, golden_codebooks[4])
    near_v = parity.check_quantize(vc, v64, 0, s64, golden_codebooks[2])
    _say(f"  tiny: near-boundary coordinates K {near_k} / {1024 * 128}, V {near_v} / {1024 * 128}")
    # end to end: the oracle quantizes, packs and attends on its own; the GPU output may differ
    # from it only through near-boundary codes (none are expected at this size)
    ck, tk = golden_codebooks[4]
    cv, tv = golden_codebooks[2]
    codes_k, n_k, _ = o.quantize(k64[0, :, 0], s64, ck, tk)
    codes_v, n_v, _ = o.quantize(v64[0, :, 0], s64, cv, tv)
    kh = o.dequantize(o.unpack(o.pack(codes_k, 4, 0), 1024, 128, 4, 0), n_k, s64, ck)[None, None]
    vh = o.dequantize(o.unpack(o.pack(codes_v, 2, 1), 1024, 128, 2, 1), n_v, s64, cv)[None, None]
    e2e, _, _ = o.decode_attention(parity.to_f64(g["q"]), kh, vh, 1.0 / math.sqrt(128))
    if near_k == 0 and near_v == 0:
        parity.check_rows(buf.out.cpu().numpy(), e2e, "tiny end to end")


@pytest.mark.parametrize("case", [
    # (workload, batch, hq, hkv, ctx, cap, bits_k, bits_v)
    ("llama8k", 1, 32, 8, 700, 768, 4, 2),
    ("llama8k", 2, 8, 2, 1000, 1024, 4, 2),
    ("batch32k", 2, 8, 2, 1300, 1344, 3, 2),
    ("ctx131k", 2, 16, 2, 1500, 1536, 4, 2),
    ("ctx131k", 1, 16, 1, 600, 640, 4, 3),
    ("llama8k", 1, 2, 2, 333, 384, 8, 8),
    ("llama8k", 1, 4, 2, 64, 64, 2, 4),
    ("llama8k", 1, 16, 1, 500, 512, 4, 2),
    # 256 (batch, kv head) planes with splits of 3072+ tokens: 12 waves per workgroup
    ("batch32k", 32, 32, 8, 3100, 3136, 3, 2),
    ("llama8k", 32, 16, 8, 3200, 3200, 4, 2),
])
def test_decode_dense_matches_oracle(case, signs, golden_codebooks):
    name, *shape = case
    _say("decode dense", case)
    _decode_case(inputs.WORKLOADS[name], signs, golden_codebooks, *shape)


def _append_case(w, signs, golden, batch, hq, hkv, ctx, cap, bits_k, bits_v, seq_lens=None, x_dtype=None):
    """Caches hold garbage at each sequence's last position T_b - 1; decode_attn_append must
    write the new token there (codes and norm as the oracle quantizes it), leave every other
    position as it was, and attend over the result."""
    g = inputs.generate(w, device="cpu", batch=batch, ctx=ctx, n_kv_heads=hkv, n_q_heads=hq)
    k, v = g["k"], g["v"]
    if x_dtype is not None:
        k, v = k.to(x_dtype), v.to(x_dtype)
    lens = [ctx] * batch if seq_lens is None else list(seq_lens)
    k_pre, v_pre = k.clone(), v.clone()
    k_new = torch.zeros((batch, 1, hkv, 128), dtype=k.dtype)
    v_new = torch.zeros((batch, 1, hkv, 128), dtype=v.dtype)
    for b, tb in enumerate(lens):
        if tb >= 1:
            k_new[b, 0], v_new[b, 0] = k[b, tb - 1], v[b, tb - 1]
            k_pre[b, tb - 1] = k[b, (tb * 7) % ctx] * -3.0       # garbage in the slot to be written
            v_pre[b, tb - 1] = v[b, (tb * 5) % ctx] * 2.5
    kc = _new_cache(batch, hkv, cap, bits_k, 0, signs)
    vc = _new_cache(batch, hkv, cap, bits_v, 1, signs)
    _fill(kc, k_pre.to(DEV))
    _fill(vc, v_pre.to(DEV))
    before = {(id(c), b, h): (parity.gpu_plane_codes(c, b, h, cap)[0], parity.gpu_plane_norms(c, b, h, cap))
              for c in (kc, vc) for b in range(batch) for h in range(hkv)}
    scale = 1.0 / math.sqrt(128)
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    q = g["q"].to(DEV).contiguous()
    buf = tq.decode_attn_append(kc, vc, k_new.to(DEV).contiguous(), v_new.to(DEV).contiguous(), q, ctx, scale,
                                seq_lens=sl)
    torch.cuda.synchronize()
    s64 = signs.numpy().astype(np.float64)
    for cache, xnew, table in ((kc, k_new, golden[bits_k]), (vc, v_new, golden[bits_v])):
        for b, tb in enumerate(lens):
            for h in range(hkv):
                codes0, norms0 = before[(id(cache), b, h)]
                keep = np.ones(cap, dtype=bool)
                if tb >= 1:
                    keep[tb - 1] = False
                    parity.check_plane(cache, b, h, parity.to_f64(xnew[b, :, h]), tb - 1, s64, table)
                assert np.array_equal(parity.gpu_plane_codes(cache, b, h, cap)[0][keep], codes0[keep]), (b, h)
                assert np.array_equal(parity.gpu_plane_norms(cache, b, h, cap)[keep], norms0[keep]), (b, h)
    kh = parity.oracle_cache_view(kc, s64, golden[bits_k], ctx)
    vh = parity.oracle_cache_view(vc, s64, golden[bits_v], ctx)
    out, lse, _ = o.decode_attention(parity.to_f64(g["q"]), kh, vh, scale, seq_lens=seq_lens)
    fin = np.isfinite(lse)
    got_lse = buf.lse.cpu().numpy()
    assert np.all(np.isneginf(got_lse[~fin]))
    assert np.allclose(got_lse[fin], lse[fin], rtol=0, atol=1e-3 * np.maximum(1, np.abs(lse[fin])))
    worst = parity.check_rows(buf.out.cpu().numpy(), out, "append+decode out")
    _say(f"  worst rel err {worst:.2e}")


@pytest.mark.parametrize("case", [
    # (workload, batch, hq, hkv, ctx, cap, bits_k, bits_v, tau, seq_lens)
    ("ctx131k", 2, 16, 2, 1500, 1536, 4, 2, 1e-4, [1500, 1]),            # 8-wave key pass
    # 256 planes with splits of 3072+ tokens: the 16-wave (4-head groups) and 12-wave (8-head
    # groups) key passes, 3-bit rows assembled behind the 3-bit table; ragged, one empty
    ("batch32k", 32, 32, 8, 3100, 3136, 3, 2, 1e-3, [3100 - 37 * i for i in range(31)] + [0]),
    ("ctx131k", 32, 64, 8, 3100, 3136, 4, 2, 1e-4, [3100 - 41 * i for i in range(31)] + [0]),
    ("batch32k", 32, 64, 8, 3100, 3136, 3, 2, 1e-3, [3100 - 43 * i for i in range(31)] + [0]),
    ("llama8k", 1, 8, 2, 333, 384, 8, 8, 1e-3, None),                    # other widths: two launches
])
def test_decode_append_sparse_equals_append_then_decode(case, signs, golden_codebooks):
    """Sparse V with the decode step's append (tq_decode_attn_append_sparse): the key pass writes
    each sequence's new key and value at T_b - 1 before reading that tile.  The caches must hold
    exactly the bytes the dense append-and-attend call writes, and the outputs and LSE must equal
    those of tq_decode_attn at the same tau on those caches (itself checked against the oracle
    in the Sparse V tests)."""
    name, batch, hq, hkv, ctx, cap, bk, bv, tau, seq_lens = case
    _say("append + sparse decode", case)
    w = inputs.WORKLOADS[name]
    g = inputs.generate(w, device="cpu", batch=batch, ctx=ctx, n_kv_heads=hkv, n_q_heads=hq)
    lens = [ctx] * batch if seq_lens is None else list(seq_lens)
    k_new = torch.zeros((batch, 1, hkv, 128), dtype=g["k"].dtype)
    v_new = torch.zeros((batch, 1, hkv, 128), dtype=g["v"].dtype)
    for b, tb in enumerate(lens):
        if tb >= 1:
            k_new[b, 0], v_new[b, 0] = g["k"][b, tb - 1], g["v"][b, tb - 1]
    k_new, v_new = k_new.to(DEV).contiguous(), v_new.to(DEV).contiguous()
    scale = 1.0 / math.sqrt(128)
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    q = g["q"].to(DEV).contiguous()
    caches = []
    for _ in range(2):
        kc = _new_cache(batch, hkv, cap, bk, 0, signs)
        vc = _new_cache(batch, hkv, cap, bv, 1, signs)
        _fill(kc, (g["k"] * -0.5).to(DEV))  # stale contents at every T_b - 1
        _fill(vc, (g["v"] * 1.5).to(DEV))
        _fill(kc, g["k"][:, : ctx - 1].to(DEV).contiguous())
        _fill(vc, g["v"][:, : ctx - 1].to(DEV).contiguous())
        caches.append((kc, vc))
    (ka, va), (kb, vb) = caches
    got = tq.decode_attn_append(ka, va, k_new, v_new, q, ctx, scale, seq_lens=sl, tau=tau)
    if seq_lens is None:  # the reference append: the small-append kernel at the common position
        tq.quantize_append_kv(kb, vb, k_new, v_new, ctx - 1)
    else:  # the dense append-and-attend call writes each sequence's token at T_b - 1
        tq.decode_attn_append(kb, vb, k_new, v_new, q, ctx, scale, seq_lens=sl)
    ref = tq.decode_attn(kb, vb, q, ctx, scale, tau=tau, seq_lens=sl)
    torch.cuda.synchronize()
    for what, x, y in (("key codes", ka.codes, kb.codes), ("key norms", ka.norms, kb.norms),
                       ("value codes", va.codes, vb.codes), ("value norms", va.norms, vb.norms)):
        assert torch.equal(x, y), what
    d_out = (got.out - ref.out).abs().max().item()
    scale_out = ref.out.abs().max().item()
    fin = torch.isfinite(ref.lse)
    assert torch.equal(torch.isfinite(got.lse), fin)
    d_lse = (got.lse[fin] - ref.lse[fin]).abs().max().item() if bool(fin.any()) else 0.0
    _say(f"  max |out diff| {d_out:.2e} (of {scale_out:.2e}), max |lse diff| {d_lse:.2e}")
    assert d_out <= 1e-6 * max(scale_out, 1e-30) and d_lse <= 1e-6 * max(1.0, ref.lse[fin].abs().max().item())


@pytest.mark.parametrize("case", [
    # (workload, batch, hq, hkv, ctx, cap, bits_k, bits_v, seq_lens, x dtype)
    ("llama8k", 1, 32, 8, 700, 768, 4, 2, None, None),
    ("batch32k", 2, 8, 2, 1300, 1344, 3, 2, None, None),
    ("ctx131k", 2, 16, 2, 1500, 1536, 4, 2, [1500, 1], None),
    ("llama8k", 3, 8, 2, 520, 576, 3, 2, [520, 0, 9], "f32"),
    ("llama8k", 2, 4, 4, 300, 320, 4, 2, [257, 64], "f16"),
    ("llama8k", 1, 8, 2, 333, 384, 8, 3, None, None),      # other widths: two launches
    # 12 waves per workgroup (splits of 3072+ tokens), ragged lengths: the new token lands in
    # various waves' tiles, one sequence is empty
    ("batch32k", 32, 32, 8, 3100, 3136, 3, 2, [3100 - 37 * i for i in range(31)] + [0], None),
])
def test_decode_append_matches_oracle(case, signs, golden_codebooks):
    name, *shape, xdt = case
    _say("append + decode", case)
    xdt = {None: None, "f32": torch.float32, "f16": torch.float16}[xdt]
    _append_case(inputs.WORKLOADS[name], signs, golden_codebooks, *shape, x_dtype=xdt)


def _gather_pages(kc, vc, table, signs, max_ctx):
    """The contiguous copy of paged caches (slot p of sequence b = pool page table[b, p]) and
    the mask of positions that lie on a page of the table."""
    batch, max_pages = table.shape
    page, hkv = kc.page_tokens, kc.n_kv_heads
    cap = max_pages * page
    kf = _new_cache(batch, hkv, cap, kc.bits, 0, signs)
    vf = _new_cache(batch, hkv, cap, vc.bits, 1, signs)
    for pc, fc in ((kc, kf), (vc, vf)):
        per = page * 16 * pc.bits
        for b in range(batch):
            for h in range(hkv):
                dst, dn = fc.plane_codes(b, h), fc.plane_norms(b, h)
                for slot in range(max_pages):
                    pg = int(table[b, slot])
                    if pg < 0:
                        continue
                    dst[slot * per:(slot + 1) * per] = pc.page_codes(pg, h)
                    dn[slot * page:(slot + 1) * page] = pc.page_norms(pg, h)
    torch.cuda.synchronize()
    valid = np.ones((batch, max_ctx), dtype=bool)
    for b in range(batch):
        for slot in range(max_pages):
            if int(table[b, slot]) < 0:
                valid[b, slot * page:(slot + 1) * page] = False
    return kf, vf, valid


def _paged_case(w, signs, golden, batch, hq, hkv, page, seq_lens, bits_k, x_dtype=None, hole=None, seed=0,
                fused=False):
    """Paged caches with shuffled pages (and optionally table entries of no page) filled by
    the paged append (a long call, then a decode step with per-sequence starts: the paged
    append and paged decode, or, fused, the one-launch paged append-and-attend over a slot
    that held garbage); the pages, gathered in table order, must hold the oracle's codes.
    A position on a table entry of no page is not part of its sequence ([inferrs] §二,
    PagedAttention: tokens live only in allocated pages): the oracle leaves it out of the
    softmax.  Paged decode must equal the oracle within tolerance, and, for every sequence
    without such a hole, the contiguous decode on the gathered cache bit for bit."""
    holes = [] if hole is None else ([hole] if isinstance(hole[0], int) else list(hole))
    max_ctx = max(seq_lens)
    max_pages = (max_ctx + page - 1) // page + 1
    n_pages = batch * max_pages + 3
    rng = np.random.default_rng(seed)
    table = torch.tensor(rng.permutation(n_pages)[:batch * max_pages].reshape(batch, max_pages), dtype=torch.int32)
    for hb, hs in holes:
        table[hb, hs] = -1
    kc = tq.PagedCache(batch, hkv, page, n_pages, max_pages, bits_k, 0, signs.to(DEV),
                       block_table=table.to(DEV).contiguous(), device=DEV)
    vc = tq.PagedCache(batch, hkv, page, n_pages, max_pages, 2, 1, kc.signs, block_table=kc.block_table, device=DEV)
    for c in (kc, vc):
        c.codes.fill_(0xA5)
        c.norms.fill_(0x3C00)
    g = inputs.generate(w, device="cpu", batch=batch, ctx=max_ctx, n_kv_heads=hkv, n_q_heads=hq)
    k, v = g["k"], g["v"]
    if x_dtype is not None:
        k, v = k.to(x_dtype), v.to(x_dtype)
    # every position in one call, then each sequence's last position again (a decode step:
    # per-sequence starts, T_b = 0 gives start -1, which is skipped)
    zeros = torch.zeros(batch, dtype=torch.int32, device=DEV)
    k_fill, v_fill = k.clone(), v.clone()
    if fused:  # garbage in each sequence's last slot: the fused step must overwrite it
        for b, tb in enumerate(seq_lens):
            if tb >= 1:
                k_fill[b, tb - 1] = k[b, 0] * -3.0
                v_fill[b, tb - 1] = v[b, 0] * 2.5
    tq.paged_quantize_append_kv(kc, vc, k_fill.contiguous().to(DEV), v_fill.contiguous().to(DEV), zeros)
    last = torch.tensor([tb - 1 for tb in seq_lens], dtype=torch.int32)
    idx = last.clamp(min=0).long()
    k1 = k[torch.arange(batch), idx].unsqueeze(1).contiguous()
    v1 = v[torch.arange(batch), idx].unsqueeze(1).contiguous()
    sl = torch.tensor(list(seq_lens), dtype=torch.int32, device=DEV)
    q = g["q"].to(DEV).contiguous()
    scale = 1.0 / math.sqrt(128)
    if fused:
        got = tq.paged_decode_attn_append(kc, vc, k1.to(DEV), v1.to(DEV), q, sl, max_ctx, scale)
    else:
        tq.paged_quantize_append_kv(kc, vc, k1.to(DEV), v1.to(DEV), last.to(DEV))
        got = tq.paged_decode_attn(kc, vc, q, sl, max_ctx, scale)
    torch.cuda.synchronize()
    kf, vf, valid = _gather_pages(kc, vc, table, signs, max_ctx)
    s64 = signs.numpy().astype(np.float64)
    lens = list(seq_lens)
    for fc, x, table_b in ((kf, k, golden[bits_k]), (vf, v, golden[2])):
        for b in range(batch):
            # each run of positions on allocated pages holds the oracle's codes (the appends
            # skipped the positions with no page)
            edges = np.flatnonzero(np.diff(np.concatenate(([0], valid[b].astype(np.int8), [0]))))
            for a, e in zip(edges[0::2], edges[1::2]):
                for h in range(hkv):
                    parity.check_plane(fc, b, h, parity.to_f64(x[b, a:e, h]), int(a), s64, table_b)
    ref = tq.decode_attn(kf, vf, q, max_ctx, scale, seq_lens=sl)
    torch.cuda.synchronize()
    whole = [b for b in range(batch) if valid[b, :max(lens[b], 0)].all()]
    assert torch.equal(got.out[whole], ref.out[whole]) and torch.equal(got.lse[whole], ref.lse[whole])
    kh = parity.oracle_cache_view(kf, s64, golden[bits_k], max_ctx)
    vh = parity.oracle_cache_view(vf, s64, golden[2], max_ctx)
    out, lse, _ = o.decode_attention(parity.to_f64(g["q"]), kh, vh, scale, seq_lens=lens, valid=valid)
    fin = np.isfinite(lse)
    got_lse = got.lse.cpu().numpy()
    assert np.all(np.isneginf(got_lse[~fin]))
    assert np.allclose(got_lse[fin], lse[fin], rtol=0, atol=1e-3 * np.maximum(1, np.abs(lse[fin])))
    worst = parity.check_rows(got.out.cpu().numpy(), out, "paged decode out")
    _say(f"  worst rel err {worst:.2e}")


@pytest.mark.parametrize("case", [
    # (workload, batch, hq, hkv, page tokens, seq_lens, bits_k, x dtype, hole, fused step)
    ("llama8k", 3, 32, 8, 64, [700, 1, 333], 4, None, (0, 5), False),
    ("batch32k", 2, 8, 2, 256, [1300, 1024], 3, None, None, False),
    ("ctx131k", 2, 16, 2, 128, [1500, 0], 4, None, None, False),
    ("llama8k", 2, 4, 4, 64, [64, 65], 4, "f32", None, False),
    ("llama8k", 1, 8, 2, 512, [2100], 3, "f16", (0, 3), False),
    ("llama8k", 3, 32, 8, 64, [700, 1, 0], 4, None, None, True),
    ("batch32k", 2, 8, 2, 256, [1300, 513], 3, "f32", (1, 2), True),
    ("ctx131k", 1, 16, 2, 128, [1500], 4, None, None, True),
    # a sequence with no page at all (o = 0, LSE = -inf) beside one with two holes, the new
    # token of the fused step falling into a hole
    ("llama8k", 3, 16, 4, 64, [300, 450, 129], 4, None, [(0, s) for s in range(6)] + [(1, 1), (1, 7), (2, 2)], True),
    ("batch32k", 2, 8, 2, 64, [640, 200], 3, "f16", [(0, 0), (0, 9), (1, 3)], False),
    # splits of 3072+ tokens over pages: 12 waves per workgroup, plain and fused step
    ("batch32k", 32, 32, 8, 256, [3200] * 30 + [1500, 0], 3, None, [(3, 2)], False),
    ("llama8k", 32, 16, 8, 256, [3200 - 50 * i for i in range(32)], 4, None, [(5, 12)], True),
])
def test_paged_cache_matches_contiguous_and_oracle(case, signs, golden_codebooks):
    name, batch, hq, hkv, page, lens, bk, xdt, hole, fused = case
    _say("paged", case)
    xdt = {None: None, "f32": torch.float32, "f16": torch.float16}[xdt]
    _paged_case(inputs.WORKLOADS[name], signs, golden_codebooks, batch, hq, hkv, page, lens, bk, x_dtype=xdt, hole=hole,
                fused=fused)


def _paged_ext_case(w, signs, golden, batch, hq, hkv, page, seq_lens, bits_k, n_q=1, tau=0.0, holes=(), seed=0,
                    q_dtype=None):
    """Paged attention of several query positions, or paged Sparse V, through
    tq_paged_decode_attn_ext: shuffled pages (some table entries naming no page) filled by the
    paged append; the result must equal the oracle on the gathered cache with the positions of
    no page left out (multi_query_attention / decode_attention with tau), and, for several
    positions, the contiguous multi-query call on the gathered cache bit for bit on every
    sequence without a hole whenever both calls split the context alike."""
    max_ctx = max(seq_lens)
    max_pages = (max_ctx + page - 1) // page + 1
    n_pages = batch * max_pages + 3
    rng = np.random.default_rng(seed)
    table = torch.tensor(rng.permutation(n_pages)[:batch * max_pages].reshape(batch, max_pages), dtype=torch.int32)
    for hb, hs in holes:
        table[hb, hs] = -1
    kc = tq.PagedCache(batch, hkv, page, n_pages, max_pages, bits_k, 0, signs.to(DEV),
                       block_table=table.to(DEV).contiguous(), device=DEV)
    vc = tq.PagedCache(batch, hkv, page, n_pages, max_pages, 2, 1, kc.signs, block_table=kc.block_table, device=DEV)
    for c in (kc, vc):
        c.codes.fill_(0xA5)
        c.norms.fill_(0x3C00)
    g = inputs.generate(w, device="cpu", batch=batch, ctx=max_ctx, n_kv_heads=hkv, n_q_heads=hq, n_q=n_q)
    zeros = torch.zeros(batch, dtype=torch.int32, device=DEV)
    tq.paged_quantize_append_kv(kc, vc, g["k"].contiguous().to(DEV), g["v"].contiguous().to(DEV), zeros)
    q = g["q"] if q_dtype is None else g["q"].to(q_dtype)
    qd = q.to(DEV).contiguous()
    sl = torch.tensor(list(seq_lens), dtype=torch.int32, device=DEV)
    scale = 1.0 / math.sqrt(128)
    got = tq.paged_decode_attn_ext(kc, vc, qd, sl, max_ctx, scale, tau=tau)
    torch.cuda.synchronize()
    kf, vf, valid = _gather_pages(kc, vc, table, signs, max_ctx)
    s64 = signs.numpy().astype(np.float64)
    lens = list(seq_lens)
    kh = parity.oracle_cache_view(kf, s64, golden[bits_k], max_ctx)
    vh = parity.oracle_cache_view(vf, s64, golden[2], max_ctx)
    whole = [b for b in range(batch) if valid[b, :max(lens[b], 0)].all()]
    allowance, nb = None, 0
    if n_q > 1:
        if max_ctx <= 4096:  # the contiguous call takes the same splits (prefill mode or not)
            ref = tq.decode_attn_multi(kf, vf, qd, max_ctx, scale, seq_lens=sl)
            torch.cuda.synchronize()
            assert torch.equal(got.out[whole], ref.out[whole]) and torch.equal(got.lse[whole], ref.lse[whole])
        out, lse = o.multi_query_attention(parity.to_f64(q), kh, vh, scale, seq_lens=lens, valid=valid)
    else:
        out, lse, scores = o.decode_attention(parity.to_f64(q), kh, vh, scale, seq_lens=lens, tau=tau, valid=valid)
        if tau > 0:
            allowance, nb = parity.sparse_allowance(scores, lse, vh, tau, hq // hkv)
    fin = np.isfinite(lse)
    got_lse = got.lse.cpu().numpy()
    got_out = got.out.cpu().numpy()
    assert np.all(np.isneginf(got_lse[~fin])) and np.all(got_out[~fin] == 0.0)
    assert np.allclose(got_lse[fin], lse[fin], rtol=0, atol=1e-3 * np.maximum(1, np.abs(lse[fin])))
    worst = parity.check_rows(got_out, out, "paged ext out", allowance=allowance)
    _say(f"  worst rel err {worst:.2e} borderline {nb}")


@pytest.mark.parametrize("case", [
    # (workload, batch, hq, hkv, page tokens, seq_lens, bits_k, n_q, tau, holes)
    ("llama8k", 3, 32, 8, 64, [700, 5, 333], 4, 4, 0.0, [(0, 5)]),
    ("batch32k", 2, 8, 2, 256, [1300, 1024], 3, 7, 0.0, []),
    ("ctx131k", 2, 16, 2, 128, [1500, 0], 4, 3, 0.0, [(0, 0), (0, 11)]),
    # a chunk of 96 positions (48 row groups per kv head: prefill mode) whose last page is missing
    ("llama8k", 1, 8, 2, 64, [1400], 4, 96, 0.0, [(0, 21)]),
    # prefill mode over pages: contexts past 4096 tokens (capped splits), 8-head groups, 3-bit
    # keys, holes, and row groups past the last one in a workgroup
    ("llama8k", 2, 8, 2, 128, [6000, 4500], 4, 64, 0.0, [(1, 7)]),
    ("batch32k", 2, 16, 2, 256, [5000, 2100], 3, 20, 0.0, []),
    ("ctx131k", 1, 16, 2, 64, [3000], 4, 9, 0.0, []),       # equals the contiguous call bit for bit
    ("llama8k", 2, 16, 4, 64, [300, 450], 3, 2, 0.0, [(0, s) for s in range(5)] + [(1, 1)]),
    # Sparse V over pages
    ("ctx131k", 2, 16, 2, 128, [1500, 900], 4, 1, 1e-4, []),
    ("batch32k", 2, 8, 2, 256, [1300, 513], 3, 1, 1e-3, [(1, 1)]),
    ("llama8k", 3, 16, 4, 64, [300, 450, 129], 4, 1, 1e-2, [(0, s) for s in range(6)] + [(1, 1), (1, 6)]),
    ("ctx131k", 1, 16, 2, 64, [4000], 4, 1, 1e-3, [(0, 3), (0, 40)]),
    # long splits: the paged key pass with 12 waves (8-head groups)
    ("ctx131k", 32, 64, 8, 256, [3200] * 31 + [700], 4, 1, 1e-4, [(2, 4)]),
])
def test_paged_multi_query_and_sparse_v(case, signs, golden_codebooks):
    name, batch, hq, hkv, page, lens, bk, n_q, tau, holes = case
    _say("paged ext", case)
    _paged_ext_case(inputs.WORKLOADS[name], signs, golden_codebooks, batch, hq, hkv, page, lens, bk, n_q=n_q,
                    tau=tau, holes=holes)


def test_paged_ext_query_dtypes(signs, golden_codebooks):
    _say("paged ext dtypes")
    w = inputs.WORKLOADS["llama8k"]
    _paged_ext_case(w, signs, golden_codebooks, 2, 8, 2, 64, [640, 200], 4, n_q=3, q_dtype=torch.float32)
    _paged_ext_case(w, signs, golden_codebooks, 2, 8, 2, 64, [640, 200], 4, tau=1e-3, q_dtype=torch.float16)


def _multi_case(w, signs, golden, batch, hq, hkv, ctx, cap, bits_k, n_q, seq_lens=None, q_dtype=None):
    g = inputs.generate(w, device="cpu", batch=batch, ctx=ctx, n_kv_heads=hkv, n_q_heads=hq, n_q=n_q)
    kc = _new_cache(batch, hkv, cap, bits_k, 0, signs)
    vc = _new_cache(batch, hkv, cap, 2, 1, signs)
    _fill(kc, g["k"].to(DEV))
    _fill(vc, g["v"].to(DEV))
    q = g["q"] if n_q > 1 else g["q"][:, None]
    q = q if q_dtype is None else q.to(q_dtype)
    scale = 1.0 / math.sqrt(128)
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    buf = tq.decode_attn_multi(kc, vc, q.to(DEV).contiguous(), ctx, scale, seq_lens=sl)
    torch.cuda.synchronize()
    s64 = signs.numpy().astype(np.float64)
    kh = parity.oracle_cache_view(kc, s64, golden[bits_k], ctx)
    vh = parity.oracle_cache_view(vc, s64, golden[2], ctx)
    out, lse = o.multi_query_attention(parity.to_f64(q), kh, vh, scale, seq_lens=seq_lens)
    got_lse = buf.lse.cpu().numpy()
    fin = np.isfinite(lse)
    assert np.all(np.isneginf(got_lse[~fin]))
    assert np.allclose(got_lse[fin], lse[fin], rtol=0, atol=1e-3 * np.maximum(1, np.abs(lse[fin])))
    got = buf.out.cpu().numpy()
    assert np.all(got[~fin] == 0.0)
    worst = parity.check_rows(got[fin], out[fin], "multi-query out")
    _say(f"  worst rel err {worst:.2e}")
    return buf, out


@pytest.mark.parametrize("case", [
    # (workload, batch, hq, hkv, ctx, cap, bits_k, n_q)
    ("llama8k", 1, 32, 8, 700, 768, 4, 1),
    ("llama8k", 1, 32, 8, 700, 768, 4, 2),
    ("llama8k", 1, 32, 8, 700, 768, 4, 4),
    ("llama8k", 2, 8, 2, 1000, 1024, 4, 7),
    ("batch32k", 2, 8, 2, 1300, 1344, 3, 3),
    ("ctx131k", 2, 16, 2, 1500, 1536, 4, 5),
    ("llama8k", 1, 2, 2, 333, 384, 4, 8),
    ("llama8k", 1, 4, 4, 200, 256, 3, 64),
    # prefill chunks (8 or more row groups of 8 rows per kv head: a workgroup's waves take
    # different row groups over the same tiles)
    ("llama8k", 1, 8, 2, 1400, 1408, 4, 256),
    ("batch32k", 2, 16, 2, 900, 960, 3, 96),
    ("ctx131k", 1, 16, 2, 700, 704, 4, 33),
    # prefill chunks over one split (contexts of at most 512 tokens): each wave writes its rows'
    # outputs itself, with no partials and no merge
    ("llama8k", 1, 8, 2, 500, 512, 4, 64),
    ("batch32k", 2, 16, 2, 448, 448, 3, 40),
])
def test_multi_query_matches_oracle(case, signs, golden_codebooks):
    """Several query positions per sequence (speculative verification, chunked prefill):
    causal attention of each position over the packed cache, rows taken up to 8 at a time."""
    name, *shape = case
    _say("multi-query", case)
    _multi_case(inputs.WORKLOADS[name], signs, golden_codebooks, *shape)


@pytest.mark.parametrize("case", [
    # (workload, batch, hq, hkv, ctx, cap, bits_k, n_q, seq_lens)
    ("llama8k", 2, 32, 8, 1000, 1024, 4, 4, None),     # 16 rows per kv head: two work items
    ("llama8k", 1, 32, 8, 1026, 1088, 4, 4, None),     # new tokens on both sides of a tile edge
    ("llama8k", 1, 32, 8, 1004, 1024, 4, 8, None),     # 8 tokens over two value groups of one tile
    ("batch32k", 2, 8, 2, 1300, 1344, 3, 5, None),     # 3-bit rows
    ("ctx131k", 2, 16, 2, 1500, 1536, 4, 3, None),     # 8-head groups
    ("llama8k", 4, 8, 2, 900, 960, 4, 4, [900, 863, 3, 0]),   # ragged: a short and an empty sequence
    ("llama8k", 1, 8, 2, 700, 704, 4, 64, None),       # a prefill chunk: append kernel, then attention
])
def test_multi_query_append_equals_append_then_attend(case, signs, golden_codebooks):
    """tq_decode_attn_multi_append writes each sequence's n_q new tokens at T_b - n_q .. T_b - 1
    (those >= 0) and attends: the caches must hold exactly the bytes of the append kernels at
    those positions (every other byte unchanged) and the outputs and LSE must equal
    tq_decode_attn_multi on them (itself checked against the oracle above)."""
    name, batch, hq, hkv, ctx, cap, bk, n_q, seq_lens = case
    _say("multi-query append", case)
    w = inputs.WORKLOADS[name]
    g = inputs.generate(w, device="cpu", batch=batch, ctx=ctx, n_kv_heads=hkv, n_q_heads=hq, n_q=n_q)
    lens = [ctx] * batch if seq_lens is None else list(seq_lens)
    k_new = torch.zeros((batch, n_q, hkv, 128), dtype=g["k"].dtype)
    v_new = torch.zeros((batch, n_q, hkv, 128), dtype=g["v"].dtype)
    for b, tb in enumerate(lens):
        for j in range(n_q):
            p = tb - n_q + j
            if p >= 0:
                k_new[b, j], v_new[b, j] = g["k"][b, p], g["v"][b, p]
    k_new, v_new = k_new.to(DEV).contiguous(), v_new.to(DEV).contiguous()
    scale = 1.0 / math.sqrt(128)
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    q = g["q"].to(DEV).contiguous()

    def filled(bsz, kx, vx):
        kc = _new_cache(bsz, hkv, cap, bk, 0, signs)
        vc = _new_cache(bsz, hkv, cap, 2, 1, signs)
        _fill(kc, (kx * -0.5).to(DEV))  # stale contents at the positions to be written
        _fill(vc, (vx * 1.5).to(DEV))
        _fill(kc, kx[:, : ctx - n_q].to(DEV).contiguous())
        _fill(vc, vx[:, : ctx - n_q].to(DEV).contiguous())
        return kc, vc

    ka, va = filled(batch, g["k"], g["v"])
    got = tq.decode_attn_multi_append(ka, va, k_new, v_new, q, ctx, scale, seq_lens=sl)
    torch.cuda.synchronize()
    # reference caches: each sequence's tokens through the append kernels into a cache of its own
    kb, vb = filled(batch, g["k"], g["v"])
    for b, tb in enumerate(lens):
        j0 = max(0, n_q - tb)
        if tb == 0 or j0 >= n_q:
            continue
        k1, v1 = filled(1, g["k"][b:b + 1], g["v"][b:b + 1])
        tq.quantize_append_kv(k1, v1, k_new[b:b + 1, j0:].contiguous(), v_new[b:b + 1, j0:].contiguous(),
                              tb - n_q + j0)
        torch.cuda.synchronize()
        for h in range(hkv):
            for big, one in ((kb, k1), (vb, v1)):
                big.plane_codes(b, h).copy_(one.plane_codes(0, h))
                big.plane_norms(b, h).copy_(one.plane_norms(0, h))
    ref = tq.decode_attn_multi(kb, vb, q, ctx, scale, seq_lens=sl)
    torch.cuda.synchronize()
    for what, x, y in (("key codes", ka.codes, kb.codes), ("key norms", ka.norms, kb.norms),
                       ("value codes", va.codes, vb.codes), ("value norms", va.norms, vb.norms)):
        assert torch.equal(x, y), what
    d_out = (got.out - ref.out).abs().max().item()
    fin = torch.isfinite(ref.lse)
    assert torch.equal(torch.isfinite(got.lse), fin)
    d_lse = (got.lse[fin] - ref.lse[fin]).abs().max().item() if bool(fin.any()) else 0.0
    _say(f"  max |out diff| {d_out:.2e}, max |lse diff| {d_lse:.2e}")
    assert d_out <= 1e-6 * max(ref.out.abs().max().item(), 1e-30)
    assert d_lse <= 1e-6 * max(1.0, ref.lse[fin].abs().max().item() if bool(fin.any()) else 1.0)


def test_multi_query_ragged_lengths_and_dtypes(signs, golden_codebooks):
    """Per-sequence lengths, including one shorter than the number of query positions (its
    first queries see nothing: o = 0, LSE = -inf) and an empty one; fp32 and fp16 queries."""
    _say("multi-query ragged")
    w = inputs.WORKLOADS["llama8k"]
    _multi_case(w, signs, golden_codebooks, 3, 8, 2, 900, 960, 4, 6, seq_lens=[900, 3, 0])
    _multi_case(w, signs, golden_codebooks, 2, 8, 2, 300, 320, 4, 3, seq_lens=[129, 300],
                q_dtype=torch.float32)
    _multi_case(w, signs, golden_codebooks, 1, 16, 2, 260, 320, 3, 2, q_dtype=torch.float16)
    # a prefill chunk longer than one sequence (its first queries see nothing) and an empty one
    _multi_case(w, signs, golden_codebooks, 3, 8, 2, 700, 704, 4, 80, seq_lens=[700, 50, 0],
                q_dtype=torch.float32)
    # the same over one split (the rows' outputs written without partials)
    _multi_case(w, signs, golden_codebooks, 3, 8, 2, 480, 512, 4, 80, seq_lens=[480, 50, 0])


def test_decode_seq_lens_and_query_dtypes(signs, golden_codebooks):
    _say("decode seq_lens")
    w = inputs.WORKLOADS["llama8k"]
    _decode_case(w, signs, golden_codebooks, 4, 8, 2, 900, 960, 4, 2, seq_lens=[900, 0, 1, 513])
    _decode_case(w, signs, golden_codebooks, 2, 8, 2, 300, 320, 4, 2, q_dtype=torch.float32)
    _decode_case(w, signs, golden_codebooks, 2, 8, 2, 300, 320, 4, 2, q_dtype=torch.float16, scale=0.3)


def test_decode_empty_context(signs, golden_codebooks):
    _say("decode empty")
    kc = _new_cache(1, 2, 64, 4, 0, signs)
    vc = _new_cache(1, 2, 64, 2, 1, signs)
    q = torch.randn((1, 4, 128), device=DEV)
    buf = tq.decode_attn(kc, vc, q, 0, 0.1)
    torch.cuda.synchronize()
    assert torch.all(buf.out == 0) and torch.all(torch.isneginf(buf.lse))


@pytest.mark.parametrize("case", [
    ("ctx131k", 2, 16, 2, 1500, 1536, 4, 2, 1e-4),
    ("batch32k", 2, 8, 2, 1300, 1344, 3, 2, 1e-4),
    ("llama8k", 1, 8, 2, 777, 832, 4, 2, 1e-2),
    ("ctx131k", 1, 16, 1, 700, 704, 4, 2, 0.3),
    ("llama8k", 1, 2, 2, 333, 384, 8, 8, 1e-3),
    ("ctx131k", 1, 16, 1, 600, 640, 4, 3, 1e-3),
    ("llama8k", 1, 6, 2, 500, 512, 4, 4, 1e-3),
    # splits of 3072+ tokens: the key pass runs 16 waves (4-head groups) or 12 (8-head groups)
    ("batch32k", 32, 32, 8, 3100, 3136, 3, 2, 1e-3),
    ("ctx131k", 32, 64, 8, 3100, 3136, 4, 2, 1e-4),
])
def test_decode_sparse_v_matches_oracle(case, signs, golden_codebooks):
    name, *shape, tau = case
    _say("decode sparse", case)
    _decode_case(inputs.WORKLOADS[name], signs, golden_codebooks, *shape, tau=tau)


def test_decode_sparse_v_ragged_lengths(signs, golden_codebooks):
    _say("decode sparse seq_lens")
    w = inputs.WORKLOADS["llama8k"]
    _decode_case(w, signs, golden_codebooks, 4, 8, 2, 900, 960, 4, 2, seq_lens=[900, 0, 1, 513],
                 tau=1e-3)


def test_decode_is_deterministic(signs):
    _say("determinism")
    w = inputs.WORKLOADS["llama8k"]
    g = inputs.generate(w, device="cpu", batch=2, ctx=900, n_kv_heads=2, n_q_heads=8)
    kc = _new_cache(2, 2, 960, 4, 0, signs)
    vc = _new_cache(2, 2, 960, 2, 1, signs)
    _fill(kc, g["k"].to(DEV))
    _fill(vc, g["v"].to(DEV))
    q = g["q"].to(DEV)
    for tau in (0.0, 1e-3):
        a = tq.decode_attn(kc, vc, q, 900, 0.0884, tau=tau).out.clone()
        b = tq.decode_attn(kc, vc, q, 900, 0.0884, tau=tau).out.clone()
        torch.cuda.synchronize()
        assert torch.equal(a, b)
    # 256 planes, splits of 3072+ tokens: the 12-wave decode and the 16-wave key pass
    w = inputs.WORKLOADS["batch32k"]
    g = inputs.generate(w, device="cpu", batch=32, ctx=3100, n_kv_heads=8, n_q_heads=32)
    kc = _new_cache(32, 8, 3136, 3, 0, signs)
    vc = _new_cache(32, 8, 3136, 2, 1, signs)
    _fill(kc, g["k"].to(DEV))
    _fill(vc, g["v"].to(DEV))
    q = g["q"].to(DEV)
    for tau in (0.0, 1e-3):
        a = tq.decode_attn(kc, vc, q, 3100, 0.0884, tau=tau).out.clone()
        b = tq.decode_attn(kc, vc, q, 3100, 0.0884, tau=tau).out.clone()
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_stream_read_probe_runs():
    """The measurement probe reads a buffer and leaves it untouched (it only loads)."""
    _say("stream-read probe")
    buf = torch.arange(1 << 18, dtype=torch.int32, device=DEV)
    ref = buf.clone()
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    tq.probe_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)


# ------------------------------------------------------------------ inner-product search


def _search_case(signs, golden, n, nq, k, bits, q_dtype=None, dup=False, seed=0):
    spec = dict(inputs.SEARCH["search1m"])
    spec["seed"] = 20 + seed
    g = inputs.generate_search(spec, device="cpu", n=n, n_queries=nq)
    x, q = g["x"], g["q"]
    if dup == "all":  # every vector the same: every block ties, the lowest indices win
        x[:] = x[0]
    elif dup:  # exact duplicates: equal codes, equal scores, ascending indices
        x[7] = x[3]
        x[n - 1] = x[3]
        q[0] = x[3]
    if q_dtype is not None:
        q = q.to(q_dtype)
    cap = (n + 63) // 64 * 64
    db = _new_cache(1, 1, cap, bits, 0, signs)
    _fill(db, x[None, :, None, :].contiguous().to(DEV))
    res = tq.ip_search(db, q.to(DEV).contiguous(), n, k)
    torch.cuda.synchronize()
    s64 = signs.numpy().astype(np.float64)
    c, _ = golden[bits]
    codes, _ = parity.gpu_plane_codes(db, 0, 0, cap)
    n16 = parity.gpu_plane_norms(db, 0, 0, n).astype(np.float16)
    idx_o, sc_o, s_all = o.ip_search(parity.to_f64(q), codes[:n], n16, s64, c, k)
    idx_g, sc_g = res.idx.cpu().numpy(), res.score.cpu().numpy()
    kk = min(k, n)
    for j in range(nq):
        tol = 1e-3 * np.abs(s_all[j]).max()
        got = idx_g[j, :kk]
        assert np.all(got >= 0) and len(set(got.tolist())) == kk, (j, got)
        # scores of the returned vectors, and the order the GPU gave them
        assert np.all(np.abs(sc_g[j, :kk] - s_all[j][got]) <= tol), j
        assert np.all(np.diff(sc_g[j, :kk]) <= 0), j
        for a in range(kk - 1):
            if sc_g[j, a] == sc_g[j, a + 1]:
                assert got[a] < got[a + 1], (j, a)
        # the set: everything clearly above the k-th oracle score is found, nothing clearly
        # below it is returned (near-ties may go either way)
        kth = sc_o[j, kk - 1]
        assert np.all(s_all[j][got] >= kth - 2 * tol), j
        must = np.nonzero(s_all[j] > kth + 2 * tol)[0]
        assert set(must.tolist()) <= set(got.tolist()), j
        if k > n:
            assert np.all(idx_g[j, n:] == -1) and np.all(np.isneginf(sc_g[j, n:]))
    if dup == "all":
        assert np.all(idx_g[:, :kk] == np.arange(kk)[None, :])
        assert np.all(sc_g[:, :kk] == sc_g[:, :1])
    elif dup:
        got0 = idx_g[0, :kk].tolist()
        assert got0[:3] == [3, 7, n - 1] and sc_g[0, 0] == sc_g[0, 1] == sc_g[0, 2]
    return idx_g


@pytest.mark.parametrize("case", [
    # (n vectors, queries, top_k, bits, q dtype, duplicates)
    (20000, 11, 10, 4, None, False),
    (20000, 8, 64, 3, None, False),
    (9000, 3, 5, 4, "f32", True),
    (40, 2, 64, 4, None, False),          # fewer vectors than k
    (8192, 1, 1, 3, "f16", False),
    (300000, 3, 64, 4, None, False),      # 293 blocks x 64 candidates
    (20000, 2, 64, 4, None, "all"),       # all tied: 20 blocks x 64 candidates pass the bound
    (70000, 9, 7, 3, "f16", "all"),       # all tied, two query groups
    (300000, 1, 64, 4, None, "all"),      # all tied: 18752 candidates reach the bound
])
def test_ip_search_matches_oracle(case, signs, golden_codebooks):
    n, nq, k, bits, qdt, dup = case
    _say("ip search", case)
    qdt = {None: None, "f32": torch.float32, "f16": torch.float16}[qdt]
    _search_case(signs, golden_codebooks, n, nq, k, bits, q_dtype=qdt, dup=dup)


def test_ip_search_repeated_calls_share_workspace(signs):
    """The search state in the workspace returns to zero after every call: calls in a row on
    one set of buffers (a smaller database second, then the first again) give the outputs of
    calls on fresh buffers, bit for bit."""
    _say("ip search repeated calls")
    spec = dict(inputs.SEARCH["search1m"])
    n, nq, k = 150000, 12, 16
    g = inputs.generate_search(spec, device="cpu", n=n, n_queries=nq)
    cap = (n + 63) // 64 * 64
    db = _new_cache(1, 1, cap, 4, 0, signs)
    _fill(db, g["x"][None, :, None, :].contiguous().to(DEV))
    q = g["q"].to(DEV).contiguous()
    shared = tq.SearchBuffers(nq, n, k, device=DEV)
    for m in (n, 33333, n):
        fresh = tq.ip_search(db, q, m, k)
        tq.ip_search(db, q, m, k, buffers=shared)
        torch.cuda.synchronize()
        assert torch.equal(fresh.idx, shared.idx) and torch.equal(fresh.score, shared.score), m
        assert int(fresh.idx.max()) < m

"""GPU parity of the QJL residual variant ([google] §第二步：QJL: a 1-bit Johnson-Lindenstrauss
sketch of the first stage's error, for unbiased attention scores): the quantize kernel's codes,
sign bits and residual norms against the oracle's, and decode attention with QJL-corrected
scores against the oracle's attention over its effective keys, on the GPU-written cache."""
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


@pytest.mark.parametrize("bits,dtype,n_tok,start", [(3, "bf16", 200, 0), (2, "f32", 130, 7), (4, "f16", 64, 64),
                                                    (8, "bf16", 70, 1), (3, "f32", 1, 100),
                                                    # up to 8 tokens: sketch rows shared out over workgroups
                                                    (4, "bf16", 8, 33), (2, "f16", 3, 0), (8, "f32", 5, 60),
                                                    (3, "bf16", 9, 20)])
def test_qjl_quantize_matches_oracle(bits, dtype, n_tok, start, golden_codebooks):
    _say("qjl quantize", bits, dtype, n_tok, start)
    w = inputs.WORKLOADS["qjl8k"]
    g = inputs.generate(w, device="cpu", batch=2, ctx=n_tok, n_kv_heads=3, with_query=False)
    x = g["k"].to({"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}[dtype])
    signs = inputs.rotation_signs()
    proj = inputs.qjl_projection()
    cap = ((start + n_tok + 63) // 64) * 64
    kc = tq.PackedCache(2, 3, cap, bits, tq.LAYOUT_ROWS, signs.to(DEV), device=DEV)
    sk = tq.QjlSketch(kc, proj, device=DEV)
    kc.codes.fill_(0x5A)
    sk.bits.fill_(0xC3)
    tq.qjl_quantize_append(kc, sk, x.to(DEV).contiguous(), start)
    torch.cuda.synchronize()
    s64 = signs.numpy().astype(np.float64)
    p64 = proj.numpy().astype(np.float64)
    x64 = parity.to_f64(x)
    tot = [0, 0, 0]
    for b in range(2):
        for h in range(3):
            r = parity.check_qjl_plane(kc, sk, b, h, x64[b, :, h], start, s64, golden_codebooks[bits], p64)
            tot = [a + c for a, c in zip(tot, r)]
            if start > 0:  # positions before the range keep their stale sign bits
                before = sk.plane_bits(b, h)[: start * 16].cpu().numpy()
                assert np.all(before == 0xC3)
    _say(f"  near-boundary coords {tot[0]}, near-zero sign bits {tot[1]}, tokens with a code flip {tot[2]}")


@pytest.mark.parametrize("bk,bv,dtype,n_tok,start", [(3, 2, "bf16", 1, 8191), (3, 2, "f32", 3, 6), (4, 3, "f16", 8, 37),
                                                     (2, 4, "bf16", 5, 0), (3, 2, "bf16", 20, 3)])
def test_qjl_append_kv_equals_separate_calls(bk, bv, dtype, n_tok, start, golden_codebooks):
    """The key-and-value call (one launch up to 8 tokens, two launches beyond) writes exactly the
    bytes of tq_qjl_quantize_append on the keys and tq_quantize_append on the values: codes, norms,
    sign bits, residual norms and every value group, including groups the range only partly
    covers (their other tokens kept).  The separate calls themselves are checked against the
    oracle above and in the small-append tests."""
    _say("qjl append kv", bk, bv, dtype, n_tok, start)
    w = inputs.WORKLOADS["qjl8k"]
    g = inputs.generate(w, device="cpu", batch=2, ctx=n_tok, n_kv_heads=3, with_query=False)
    dt = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}[dtype]
    xk, xv = g["k"].to(dt).to(DEV).contiguous(), g["v"].to(dt).to(DEV).contiguous()
    signs = inputs.rotation_signs().to(DEV)
    proj = inputs.qjl_projection()
    cap = ((start + n_tok + 63) // 64) * 64
    out = []
    for fused in (False, True):
        kc = tq.PackedCache(2, 3, cap, bk, tq.LAYOUT_ROWS, signs, device=DEV)
        vc = tq.PackedCache(2, 3, cap, bv, tq.LAYOUT_GROUP8, signs, device=DEV)
        sk = tq.QjlSketch(kc, proj, device=DEV)
        for t, v in ((kc.codes, 0x5A), (kc.norms, 7), (vc.codes, 0xA5), (vc.norms, 9), (sk.bits, 0xC3),
                     (sk.res_norms, 11)):
            t.fill_(v)
        if fused:
            tq.qjl_quantize_append_kv(kc, sk, vc, xk, xv, start)
        else:
            tq.qjl_quantize_append(kc, sk, xk, start)
            tq.quantize_append(vc, xv, start)
        torch.cuda.synchronize()
        out.append([t.clone() for t in (kc.codes, kc.norms, vc.codes, vc.norms, sk.bits, sk.res_norms)])
    for name, a, b in zip(("key codes", "key norms", "value codes", "value norms", "sign bits", "residual norms"),
                          *out):
        assert torch.equal(a, b), name


def _qjl_decode_case(name, batch, hq, hkv, ctx, cap, bits_k, golden, tau=0.0, seq_lens=None, q_dtype=None):
    _say("qjl decode", name, batch, hq, hkv, ctx, bits_k, tau, seq_lens, q_dtype)
    w = inputs.WORKLOADS[name]
    g = inputs.generate(w, device="cpu", batch=batch, ctx=ctx, n_kv_heads=hkv, n_q_heads=hq)
    signs = inputs.rotation_signs()
    sd = signs.to(DEV)
    proj = inputs.qjl_projection()
    kc = tq.PackedCache(batch, hkv, cap, bits_k, tq.LAYOUT_ROWS, sd, device=DEV)
    vc = tq.PackedCache(batch, hkv, cap, 2, tq.LAYOUT_GROUP8, sd, device=DEV)
    sk = tq.QjlSketch(kc, proj, device=DEV)
    tq.qjl_quantize_append(kc, sk, g["k"].to(DEV).contiguous(), 0)
    tq.quantize_append(vc, g["v"].to(DEV).contiguous(), 0)
    scale = 1.0 / math.sqrt(128)
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    q = g["q"] if q_dtype is None else g["q"].to(q_dtype)
    buf = tq.qjl_decode_attn(kc, sk, vc, q.to(DEV).contiguous(), ctx, scale, tau=tau, seq_lens=sl,
                             want_scores=True)
    torch.cuda.synchronize()
    s64 = signs.numpy().astype(np.float64)
    p64 = proj.numpy().astype(np.float64)
    kh = parity.oracle_qjl_view(kc, sk, s64, golden[bits_k], p64, ctx)
    vh = parity.oracle_cache_view(vc, s64, golden[2], ctx)
    out, lse, scores = o.decode_attention(parity.to_f64(q), kh, vh, scale, seq_lens=seq_lens, tau=tau)
    parity.check_scores(buf.scores.cpu().numpy(), scores, seq_lens)
    fin = np.isfinite(lse)
    got_lse = buf.lse.cpu().numpy()
    assert np.all(np.isneginf(got_lse[~fin]))
    assert np.allclose(got_lse[fin], lse[fin], rtol=0, atol=1e-3 * np.maximum(1, np.abs(lse[fin])))
    allowance, nb = None, 0
    if tau > 0:
        allowance, nb = parity.sparse_allowance(scores, lse, vh, tau, hq // hkv)
    worst = parity.check_rows(buf.out.cpu().numpy(), out, "qjl decode out", allowance=allowance)
    # the correction is not a no-op: the same codes without the sketch give other scores
    kh_mse = parity.oracle_cache_view(kc, s64, golden[bits_k], ctx)
    _, _, mse_scores = o.decode_attention(parity.to_f64(q), kh_mse, vh, scale, seq_lens=seq_lens)
    live = np.isfinite(scores)
    if live.any():
        diff = np.max(np.abs(scores[live] - mse_scores[live]))
        assert diff > 1e-2 * np.max(np.abs(scores[live]))
    _say(f"  worst rel err {worst:.2e} borderline {nb}")


@pytest.mark.parametrize("case", [
    # (workload, batch, hq, hkv, ctx, cap, bits_k, tau, seq_lens)
    ("qjl8k", 1, 32, 8, 700, 768, 3, 0.0, None),
    ("qjl8k", 2, 8, 2, 1000, 1024, 2, 0.0, [1000, 333]),
    ("batch32k", 2, 8, 2, 1300, 1344, 3, 1e-4, None),
    ("ctx131k", 1, 16, 2, 900, 960, 4, 1e-4, [900]),
    ("qjl8k", 3, 16, 1, 300, 320, 3, 0.0, [300, 0, 1]),
    # 3-bit codes, groups up to 8, no Sparse V: the matrix-core kernel (sign products on fp16
    # +/-1 operands against the query's sketch)
    ("qjl8k", 2, 16, 2, 1000, 1024, 3, 0.0, [1000, 1]),
    ("qjl8k", 3, 8, 2, 640, 640, 3, 0.0, [640, 0, 65]),
    ("ctx131k", 1, 16, 2, 2000, 2048, 3, 0.0, None),
    ("batch32k", 2, 8, 2, 1300, 1344, 3, 0.0, None),
    ("qjl8k", 1, 12, 4, 4100, 4160, 3, 0.0, None),
    # Sparse V on matrix cores: the key pass (QJL scores, LSE partials, tile maxima), then the
    # masked value pass recomputing the QJL scores of the tiles it needs
    ("qjl8k", 2, 16, 2, 1000, 1024, 3, 1e-3, [1000, 1]),
    ("ctx131k", 1, 16, 2, 5000, 5056, 3, 1e-4, None),
    ("qjl8k", 3, 8, 2, 640, 640, 3, 1e-2, [640, 0, 65]),
    ("batch32k", 1, 8, 2, 3100, 3136, 3, 1e-4, None),
])
def test_qjl_decode_matches_oracle(case, golden_codebooks):
    name, batch, hq, hkv, ctx, cap, bk, tau, sl = case
    _qjl_decode_case(name, batch, hq, hkv, ctx, cap, bk, golden_codebooks, tau=tau, seq_lens=sl)


def test_qjl_decode_query_dtypes(golden_codebooks):
    _qjl_decode_case("qjl8k", 2, 8, 2, 500, 512, 3, golden_codebooks, q_dtype=torch.float32)
    _qjl_decode_case("qjl8k", 2, 8, 2, 500, 512, 3, golden_codebooks, q_dtype=torch.float16, seq_lens=[500, 77])

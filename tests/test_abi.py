"""CPU-only checks of the C-ABI library: it loads, exports what include/tq.h declares,
its host codebook equals the oracle's, and argument validation rejects bad calls
before any HIP call (so these run without a GPU)."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import compressed_decode_attention_tq_amd as tq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(tq_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = tq.lib()
    names = _declared_symbols()
    assert {"tq_make_codebook_table", "tq_quantize_append", "tq_quantize_append_kv", "tq_decode_attn",
            "tq_dequantize", "tq_decode_workspace_bytes", "tq_status_string", "tq_code_bytes",
            "tq_probe_stream_read"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_host_codebook_equals_oracle_table(bits, golden_codebooks):
    c, t = tq.make_codebook_table(128, bits)
    gc, gt = golden_codebooks[bits]
    assert np.array_equal(c, gc.astype(np.float32))
    assert np.array_equal(t, gt.astype(np.float32))


def test_value_table_scale_makes_both_magnitudes_fp16_exact():
    """tq_value_table_scale: for the 2-bit tables, s in [1, 2) makes s a an fp16 value and
    leaves s b off an fp16 value by no more than the best rational approximation p/q of b/a with
    p < 2048 allows (brute force over every q), far below fp16's 2^-12; any other codebook
    gets 1."""
    for d in (64, 128, 256, 512):
        c, _ = tq.make_codebook_table(d, 2)
        s = tq.value_table_scale(c)
        assert 1.0 <= s < 2.0
        a, b = float(np.float32(c[2])), float(np.float32(c[3]))
        r = b / a
        best = min(abs(r - round(r * q) / q) / r for q in range(1, 2048) if round(r * q) <= 2047)
        sa, sb = np.float32(s) * np.float32(a), np.float32(s) * np.float32(b)
        assert abs(float(np.float16(sa)) - float(sa)) <= 1e-7 * float(sa), d
        assert abs(float(np.float16(sb)) - float(sb)) <= (best + 2e-7) * float(sb), (d, best)
        assert best < 2.0 ** -12
    assert tq.value_table_scale(tq.make_codebook_table(128, 3)[0]) == 1.0
    assert tq.value_table_scale(np.array([-0.2, -0.05, 0.04, 0.2], np.float32)) == 1.0   # not symmetric
    assert tq.value_table_scale(np.array([-3.0, -1.0, 1.0, 3.0], np.float32)) == 1.0     # both exact already
    assert tq.value_table_scale(np.array([-0.3, -0.1, 0.1, 0.3], np.float32)) == 1.25    # 3/1: s a = 1/8


def test_cache_table_scale_validation():
    for bad in (-1.0, 0.5, 2.5, float("nan"), float("inf")):
        assert _quant(_cache(table_scale=bad)) == tq.TQ_ERR_INVALID_ARG, bad


def test_codebook_argument_errors():
    c = np.zeros(16, np.float32)
    L = tq.lib()
    assert L.tq_make_codebook_table(128, 9, c.ctypes.data, c.ctypes.data) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_make_codebook_table(128, 4, None, c.ctypes.data) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_make_codebook_table(2, 4, c.ctypes.data, c.ctypes.data) == tq.TQ_ERR_INVALID_ARG


def test_status_strings_and_sizes():
    assert tq.status_string(0) == "ok"
    assert "workspace" in tq.status_string(tq.TQ_ERR_WORKSPACE)
    assert tq.code_bytes(128, 4, 2, 8, 1024) == 2 * 8 * 1024 * 64
    assert tq.code_bytes(128, 3, 1, 1, 64) == 64 * 48
    assert tq.decode_workspace_bytes(1, 32, 8, 8192, 0.0) > 0
    assert tq.decode_workspace_bytes(1, 32, 8, 8192, 1e-4) > tq.decode_workspace_bytes(1, 32, 8, 8192, 0.0)
    assert tq.decode_workspace_bytes(1, 30, 8, 8192, 0.0) == 0       # group not integral
    assert tq.decode_workspace_bytes(1, 32, 8, -1, 0.0) == 0
    assert tq.decode_workspace_bytes(1, 32, 8, 8192, 1.0) == 0
    assert tq.decode_workspace_bytes(1, 32, 8, 8192, float("nan")) == 0


# Fake, suitably aligned addresses: validation fails before anything dereferences them.
FAKE = 0x7F0000000000


def _cache(**kw):
    base = dict(d=128, bits=4, layout=0, batch=1, n_kv_heads=2, capacity=1024,
                codes=FAKE, norms=FAKE + 0x100000, centroids=FAKE + 0x200000,
                boundaries=FAKE + 0x300000, signs=FAKE + 0x400000, table_scale=0.0)
    base.update(kw)
    return tq.CacheStruct(base["d"], base["bits"], base["layout"], base["batch"], base["n_kv_heads"],
                          base["capacity"], base["codes"], base["norms"], base["centroids"],
                          base["boundaries"], base["signs"], base["table_scale"])


def _quant(cache, x=FAKE + 0x500000, dtype=1, start=0, n=16):
    return tq.lib().tq_quantize_append(ctypes.byref(cache), x, dtype, start, n, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=64), tq.TQ_ERR_UNSUPPORTED),
    (dict(bits=5), tq.TQ_ERR_UNSUPPORTED),
    (dict(bits=1), tq.TQ_ERR_UNSUPPORTED),
    (dict(layout=7), tq.TQ_ERR_INVALID_ARG),
    (dict(batch=0), tq.TQ_ERR_INVALID_ARG),
    (dict(capacity=1000), tq.TQ_ERR_UNSUPPORTED),
    (dict(codes=0), tq.TQ_ERR_INVALID_ARG),
    (dict(codes=FAKE + 4), tq.TQ_ERR_INVALID_ARG),
    (dict(norms=FAKE + 2), tq.TQ_ERR_INVALID_ARG),
    (dict(signs=0), tq.TQ_ERR_INVALID_ARG),
])
def test_quantize_rejects_bad_cache(kw, status):
    assert _quant(_cache(**kw)) == status


def test_quantize_rejects_bad_ranges():
    c = _cache()
    assert _quant(c, start=-1) == tq.TQ_ERR_INVALID_ARG
    assert _quant(c, n=-3) == tq.TQ_ERR_INVALID_ARG
    assert _quant(c, start=1000, n=25) == tq.TQ_ERR_CAPACITY
    assert _quant(c, dtype=9) == tq.TQ_ERR_INVALID_ARG
    assert _quant(c, x=0) == tq.TQ_ERR_INVALID_ARG
    assert _quant(c, x=FAKE + 0x500008) == tq.TQ_ERR_INVALID_ARG
    assert _quant(c, n=0) == tq.TQ_OK            # nothing to do, no launch
    assert tq.lib().tq_dequantize(ctypes.byref(c), 1020, 8, FAKE, 0, None) == tq.TQ_ERR_CAPACITY
    assert tq.lib().tq_dequantize(ctypes.byref(c), 0, 8, FAKE, 5, None) == tq.TQ_ERR_INVALID_ARG


def test_quantize_kv_rejects_mismatched_caches():
    k, v = _cache(layout=0), _cache(layout=1, bits=2)

    def qkv(k, v, xk=FAKE + 0x500000, xv=FAKE + 0x580000, dtype=1, start=0, n=16):
        return tq.lib().tq_quantize_append_kv(ctypes.byref(k), ctypes.byref(v), xk, xv, dtype, start, n, None)

    assert qkv(k, v, n=0) == tq.TQ_OK                                     # nothing to do, no launch
    assert qkv(v, k) == tq.TQ_ERR_INVALID_ARG                             # layouts swapped
    assert qkv(k, _cache(layout=1, bits=2, batch=2)) == tq.TQ_ERR_INVALID_ARG
    assert qkv(k, _cache(layout=1, bits=2, n_kv_heads=1)) == tq.TQ_ERR_INVALID_ARG
    assert qkv(k, _cache(layout=1, bits=2, capacity=2048)) == tq.TQ_ERR_INVALID_ARG
    assert qkv(k, _cache(layout=1, bits=5)) == tq.TQ_ERR_UNSUPPORTED
    assert qkv(k, v, xv=0) == tq.TQ_ERR_INVALID_ARG
    assert qkv(k, v, xk=FAKE + 0x500004) == tq.TQ_ERR_INVALID_ARG
    assert qkv(k, v, dtype=9) == tq.TQ_ERR_INVALID_ARG
    assert qkv(k, v, start=-1) == tq.TQ_ERR_INVALID_ARG
    assert qkv(k, v, start=1000, n=25) == tq.TQ_ERR_CAPACITY


def _decode(k, v, q=FAKE + 0x600000, hq=8, seq=None, ctx=512, scale=0.088, tau=0.0,
            out=FAKE + 0x700000, ws=FAKE + 0x800000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = tq.decode_workspace_bytes(k.batch, hq, k.n_kv_heads, max(ctx, 0), tau) or 1
    return tq.lib().tq_decode_attn(ctypes.byref(k), ctypes.byref(v), q, 1, hq, seq, ctx, scale, tau,
                                   out, None, None, ws, ws_bytes, None)


def test_decode_argument_validation():
    k, v = _cache(layout=0), _cache(layout=1, bits=2)
    assert _decode(k, v, hq=7) == tq.TQ_ERR_INVALID_ARG            # not a multiple of n_kv_heads
    assert _decode(k, v, hq=64) == tq.TQ_ERR_UNSUPPORTED           # group 32 > 16
    assert _decode(k, v, ctx=2048) == tq.TQ_ERR_CAPACITY
    assert _decode(k, v, ctx=-1) == tq.TQ_ERR_INVALID_ARG
    assert _decode(k, v, tau=1.5) == tq.TQ_ERR_INVALID_ARG
    assert _decode(k, v, tau=float("nan")) == tq.TQ_ERR_INVALID_ARG
    assert _decode(k, v, scale=float("inf")) == tq.TQ_ERR_INVALID_ARG
    assert _decode(k, v, ws_bytes=16) == tq.TQ_ERR_WORKSPACE
    assert _decode(k, v, ws=FAKE + 0x800010) == tq.TQ_ERR_INVALID_ARG
    assert _decode(k, v, out=0) == tq.TQ_ERR_INVALID_ARG
    assert _decode(k, v, q=FAKE + 0x600002) == tq.TQ_ERR_INVALID_ARG
    assert _decode(k, _cache(layout=0, bits=2)) == tq.TQ_ERR_UNSUPPORTED   # V must be GROUP8
    assert _decode(k, _cache(layout=1, bits=2, capacity=2048)) == tq.TQ_ERR_INVALID_ARG
    assert _decode(k, _cache(layout=1, bits=2, signs=FAKE + 0x400100)) == tq.TQ_ERR_INVALID_ARG
    assert _decode(k, v, seq=FAKE + 0x900002) == tq.TQ_ERR_INVALID_ARG


def _multi(k, v, q=FAKE + 0x600000, hq=8, n_q=4, seq=None, ctx=512, scale=0.088,
           out=FAKE + 0x700000, ws=FAKE + 0x800000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = tq.lib().tq_decode_attn_multi_workspace_bytes(k.batch, hq, k.n_kv_heads, max(n_q, 1),
                                                                 max(ctx, 0)) or 1
    return tq.lib().tq_decode_attn_multi(ctypes.byref(k), ctypes.byref(v), q, 1, hq, n_q, seq, ctx, scale,
                                         out, None, ws, ws_bytes, None)


def test_multi_query_argument_validation():
    k, v = _cache(layout=0), _cache(layout=1, bits=2)
    wsb = tq.lib().tq_decode_attn_multi_workspace_bytes
    assert wsb(1, 8, 2, 4, 512) > 0
    assert wsb(1, 8, 2, 8, 512) > wsb(1, 8, 2, 4, 512)      # more query rows, more partials
    assert wsb(1, 8, 2, 0, 512) == 0 and wsb(1, 8, 2, 4097, 512) == 0 and wsb(1, 7, 2, 4, 512) == 0
    assert _multi(k, v, n_q=0) == tq.TQ_ERR_INVALID_ARG
    assert _multi(k, v, n_q=4097) == tq.TQ_ERR_INVALID_ARG
    assert _multi(k, v, hq=7) == tq.TQ_ERR_INVALID_ARG
    assert _multi(k, v, ctx=2048) == tq.TQ_ERR_CAPACITY
    assert _multi(k, v, ctx=-1) == tq.TQ_ERR_INVALID_ARG
    assert _multi(k, v, scale=float("nan")) == tq.TQ_ERR_INVALID_ARG
    assert _multi(k, v, ws_bytes=16) == tq.TQ_ERR_WORKSPACE
    assert _multi(k, v, ws=FAKE + 0x800010) == tq.TQ_ERR_INVALID_ARG
    assert _multi(k, v, out=FAKE + 0x700004) == tq.TQ_ERR_INVALID_ARG
    assert _multi(k, v, q=0) == tq.TQ_ERR_INVALID_ARG
    assert _multi(k, _cache(layout=0, bits=2)) == tq.TQ_ERR_UNSUPPORTED        # V must be GROUP8
    assert _multi(_cache(layout=0, bits=8), v) == tq.TQ_ERR_UNSUPPORTED        # 8-bit keys: no kernel
    assert _multi(k, _cache(layout=1, bits=3)) == tq.TQ_ERR_UNSUPPORTED        # 3-bit values: no kernel
    assert _multi(k, _cache(layout=1, bits=2, n_kv_heads=1)) == tq.TQ_ERR_INVALID_ARG


def test_multi_query_append_argument_validation():
    """The multi-query append-and-attend call checks the new tokens' inputs, then everything the
    multi-query call checks, before any HIP call."""
    k, v = _cache(layout=0), _cache(layout=1, bits=2)

    def call(xk=FAKE + 0x500000, xv=FAKE + 0x580000, xdt=1, n_q=4, ctx=512, seq=None, hq=8, ws_bytes=None):
        wsb = ws_bytes if ws_bytes is not None else (
            tq.lib().tq_decode_attn_multi_workspace_bytes(1, hq, 2, max(n_q, 1), max(ctx, 0)) or 1)
        return tq.lib().tq_decode_attn_multi_append(ctypes.byref(k), ctypes.byref(v), xk, xv, xdt, FAKE + 0x600000, 1,
                                                   hq, n_q, seq, ctx, 0.088, FAKE + 0x700000, None,
                                                   FAKE + 0x800000, wsb, None)

    assert call(xk=0) == tq.TQ_ERR_INVALID_ARG
    assert call(xv=FAKE + 4) == tq.TQ_ERR_INVALID_ARG          # misaligned input
    assert call(xdt=7) == tq.TQ_ERR_INVALID_ARG                # no such dtype
    assert call(n_q=0) == tq.TQ_ERR_INVALID_ARG
    assert call(ctx=2048) == tq.TQ_ERR_CAPACITY
    assert call(hq=7) == tq.TQ_ERR_INVALID_ARG
    assert call(ws_bytes=16) == tq.TQ_ERR_WORKSPACE
    # a prefill chunk (64 positions at 4 heads per kv head) takes the two-launch path, which needs
    # one common length and at least n_q positions
    assert call(n_q=64, seq=FAKE + 0x900000) == tq.TQ_ERR_UNSUPPORTED
    assert call(n_q=64, ctx=32) == tq.TQ_ERR_UNSUPPORTED


def test_append_decode_argument_validation():
    k, v = _cache(layout=0), _cache(layout=1, bits=2)

    def ad(k, v, xk=FAKE + 0x500000, xv=FAKE + 0x580000, xdt=1, hq=8, seq=None, ctx=512,
           ws_bytes=None, out=FAKE + 0x700000):
        if ws_bytes is None:
            ws_bytes = tq.decode_workspace_bytes(k.batch, hq, k.n_kv_heads, max(ctx, 0), 0.0) or 1
        return tq.lib().tq_decode_attn_append(ctypes.byref(k), ctypes.byref(v), xk, xv, xdt, FAKE + 0x600000, 1,
                                              hq, seq, ctx, 0.088, out, None, FAKE + 0x800000, ws_bytes, None)

    assert ad(k, v, xk=0) == tq.TQ_ERR_INVALID_ARG
    assert ad(k, v, xv=FAKE + 0x580004) == tq.TQ_ERR_INVALID_ARG
    assert ad(k, v, xdt=7) == tq.TQ_ERR_INVALID_ARG
    assert ad(k, v, hq=7) == tq.TQ_ERR_INVALID_ARG
    assert ad(k, v, hq=64) == tq.TQ_ERR_UNSUPPORTED
    assert ad(k, v, ctx=2048) == tq.TQ_ERR_CAPACITY
    assert ad(k, v, ws_bytes=16) == tq.TQ_ERR_WORKSPACE
    assert ad(k, v, out=0) == tq.TQ_ERR_INVALID_ARG
    assert ad(v, k) == tq.TQ_ERR_UNSUPPORTED                                    # layouts swapped
    # widths without the one-launch kernel take two launches, which need one common position
    assert ad(_cache(layout=0, bits=8), _cache(layout=1, bits=8), seq=FAKE + 0x900000) == tq.TQ_ERR_UNSUPPORTED


def test_noalloc_decode_step_argument_validation():
    """The allocation-free decode step validates like tq_decode_attn_append, refuses the widths
    of the two-launch path, and refuses problems beyond its static scratch, all before any HIP
    call."""
    def na(k, v, xk=FAKE + 0x500000, hq=8, ctx=512, out=FAKE + 0x700000):
        return tq.lib().tq_decode_attn_append_noalloc(ctypes.byref(k), ctypes.byref(v), xk, FAKE + 0x580000, 1,
                                                      FAKE + 0x600000, 1, hq, None, ctx, 0.088, out, None, None)

    k, v = _cache(layout=0), _cache(layout=1, bits=2)
    assert na(k, v, xk=0) == tq.TQ_ERR_INVALID_ARG
    assert na(k, v, out=FAKE + 0x700004) == tq.TQ_ERR_INVALID_ARG
    assert na(k, v, hq=7) == tq.TQ_ERR_INVALID_ARG
    assert na(k, v, ctx=2048) == tq.TQ_ERR_CAPACITY
    assert na(v, k) == tq.TQ_ERR_UNSUPPORTED
    assert na(_cache(layout=0, bits=8), _cache(layout=1, bits=8)) == tq.TQ_ERR_UNSUPPORTED
    assert na(k, v, hq=32) == tq.TQ_ERR_UNSUPPORTED                        # group 16: two-launch path only
    # more (batch, kv head) counters than the static scratch holds
    big_k, big_v = _cache(layout=0, batch=4096, n_kv_heads=8), _cache(layout=1, bits=2, batch=4096, n_kv_heads=8)
    assert na(big_k, big_v, hq=64) == tq.TQ_ERR_WORKSPACE
    # partials beyond the rest of the 8 MiB: 2048 sequences x 64 query heads x 1 split x 520 bytes
    mid_k, mid_v = _cache(layout=0, batch=2048, n_kv_heads=8), _cache(layout=1, bits=2, batch=2048, n_kv_heads=8)
    assert na(mid_k, mid_v, hq=64) == tq.TQ_ERR_WORKSPACE


def test_qjl_argument_validation():
    """The QJL calls check the sketch (pointers, alignment, m = d) and the key cache's layout
    before any HIP call."""
    L = tq.lib()

    def sk(**kw):
        base = dict(m=128, bits=FAKE + 0xA00000, res_norms=FAKE + 0xB00000, proj=FAKE + 0xC00000)
        base.update(kw)
        return tq.QjlSketchStruct(base["m"], base["bits"], base["res_norms"], base["proj"])

    k = _cache(layout=0, bits=3)
    x = FAKE + 0x500000
    quant = lambda kk, ss, start=0, n=16: L.tq_qjl_quantize_append(ctypes.byref(kk), ctypes.byref(ss), x, 1, start, n,
                                                                   None)
    assert quant(k, sk(m=64)) == tq.TQ_ERR_UNSUPPORTED
    assert quant(k, sk(bits=0)) == tq.TQ_ERR_INVALID_ARG
    assert quant(k, sk(bits=FAKE + 8)) == tq.TQ_ERR_INVALID_ARG
    assert quant(k, sk(res_norms=FAKE + 1)) == tq.TQ_ERR_INVALID_ARG
    assert quant(_cache(layout=1, bits=3), sk()) == tq.TQ_ERR_INVALID_ARG
    assert quant(k, sk(), start=1020, n=16) == tq.TQ_ERR_CAPACITY
    assert quant(k, sk(), n=0) == tq.TQ_OK
    vg = _cache(layout=1, bits=2)

    def kv(kk, ss, vv, start=0, n=16, xv=FAKE + 0x580000):
        return L.tq_qjl_quantize_append_kv(ctypes.byref(kk), ctypes.byref(ss), ctypes.byref(vv), x, xv, 1, start, n,
                                           None)

    assert kv(k, sk(), vg, n=0) == tq.TQ_OK
    assert kv(k, sk(m=64), vg) == tq.TQ_ERR_UNSUPPORTED
    assert kv(k, sk(bits=FAKE + 8), vg) == tq.TQ_ERR_INVALID_ARG
    assert kv(k, sk(), _cache(layout=0, bits=2)) == tq.TQ_ERR_INVALID_ARG          # values in groups of 8
    assert kv(_cache(layout=1, bits=3), sk(), vg) == tq.TQ_ERR_INVALID_ARG         # keys in rows
    assert kv(k, sk(), _cache(layout=1, bits=2, batch=2)) == tq.TQ_ERR_INVALID_ARG  # caches disagree
    assert kv(k, sk(), _cache(layout=1, bits=2, capacity=2048)) == tq.TQ_ERR_INVALID_ARG
    assert kv(k, sk(), vg, xv=FAKE + 4) == tq.TQ_ERR_INVALID_ARG                   # misaligned input
    assert kv(k, sk(), vg, xv=0) == tq.TQ_ERR_INVALID_ARG
    assert kv(k, sk(), vg, start=1020, n=16) == tq.TQ_ERR_CAPACITY
    assert kv(k, sk(), vg, start=-1, n=1) == tq.TQ_ERR_INVALID_ARG
    v = _cache(layout=1, bits=2)
    ws = tq.decode_workspace_bytes(1, 8, 2, 512, 0.0)

    def dec(ss, hq=8, ctx=512, tau=0.0, wsb=ws):
        return L.tq_qjl_decode_attn(ctypes.byref(k), ctypes.byref(ss), ctypes.byref(v), FAKE + 0x600000, 1, hq, None,
                                    ctx, 0.088, tau, FAKE + 0x700000, None, None, FAKE + 0x800000, wsb, None)

    assert dec(sk(m=0)) == tq.TQ_ERR_UNSUPPORTED
    assert dec(sk(proj=0)) == tq.TQ_ERR_INVALID_ARG
    assert dec(sk(proj=FAKE + 0xC00004)) == tq.TQ_ERR_INVALID_ARG     # S is read 16 bytes at a time
    assert dec(sk(), hq=7) == tq.TQ_ERR_INVALID_ARG
    assert dec(sk(), ctx=4096) == tq.TQ_ERR_CAPACITY
    assert dec(sk(), wsb=16) == tq.TQ_ERR_WORKSPACE
    assert dec(sk(), tau=1.5) == tq.TQ_ERR_INVALID_ARG


def _paged(**kw):
    base = dict(d=128, bits=4, layout=0, batch=2, n_kv_heads=2, page_tokens=256, n_pages=64, max_pages=16,
                codes=FAKE, norms=FAKE + 0x1000000, block_table=FAKE + 0x1100000, centroids=FAKE + 0x200000,
                boundaries=FAKE + 0x300000, signs=FAKE + 0x400000, table_scale=0.0)
    base.update(kw)
    return tq.PagedCacheStruct(*(base[f] for f, _ in tq.PagedCacheStruct._fields_))


def test_paged_argument_validation():
    L = tq.lib()
    k, v = _paged(), _paged(layout=1, bits=2, codes=FAKE + 0x2000000, norms=FAKE + 0x3000000)
    sp, x = FAKE + 0x900000, FAKE + 0x500000

    def app(k, v, x=x, dt=1, start=sp, n=1):
        return L.tq_paged_quantize_append_kv(ctypes.byref(k), ctypes.byref(v), x, x + 0x80000, dt, start, n, None)

    assert app(k, v, n=0) == tq.TQ_OK                                   # nothing to do, no launch
    assert app(k, v, start=0) == tq.TQ_ERR_INVALID_ARG
    assert app(k, v, start=sp + 2) == tq.TQ_ERR_INVALID_ARG
    assert app(k, v, n=-1) == tq.TQ_ERR_INVALID_ARG
    assert app(k, v, dt=5) == tq.TQ_ERR_INVALID_ARG
    assert app(v, k) == tq.TQ_ERR_INVALID_ARG                            # layouts swapped
    assert app(_paged(page_tokens=100), v) == tq.TQ_ERR_UNSUPPORTED      # not a multiple of 64
    assert app(_paged(block_table=0), v) == tq.TQ_ERR_INVALID_ARG
    assert app(_paged(block_table=FAKE + 0x1100002), v) == tq.TQ_ERR_INVALID_ARG
    assert app(_paged(max_pages=32), v) == tq.TQ_ERR_INVALID_ARG         # tables differ
    assert app(k, _paged(layout=1, bits=2, table_scale=3.0)) == tq.TQ_ERR_INVALID_ARG
    assert app(_paged(n_pages=1 << 20, page_tokens=64, n_kv_heads=8),
               _paged(n_pages=1 << 20, page_tokens=64, n_kv_heads=8, layout=1, bits=2)) == tq.TQ_ERR_UNSUPPORTED
    ws = tq.paged_decode_workspace_bytes(2, 16, 2, 4096)
    assert ws > 0 and tq.paged_decode_workspace_bytes(2, 15, 2, 4096) == 0

    def dec(k, v, hq=16, seq=sp, ctx=4096, wsb=ws, out=FAKE + 0x700000):
        return L.tq_paged_decode_attn(ctypes.byref(k), ctypes.byref(v), FAKE + 0x600000, 1, hq, seq, ctx, 0.088,
                                      out, None, FAKE + 0x800000, wsb, None)

    assert dec(k, v, seq=0) == tq.TQ_ERR_INVALID_ARG                    # lengths are required
    assert dec(k, v, ctx=4097) == tq.TQ_ERR_CAPACITY                    # 16 pages of 256
    assert dec(k, v, hq=7) == tq.TQ_ERR_INVALID_ARG
    assert dec(k, v, hq=64) == tq.TQ_ERR_UNSUPPORTED                    # group 32
    assert dec(k, v, wsb=16) == tq.TQ_ERR_WORKSPACE
    assert dec(k, v, out=0) == tq.TQ_ERR_INVALID_ARG
    assert dec(_paged(bits=8), v) == tq.TQ_ERR_UNSUPPORTED
    assert dec(k, _paged(layout=1, bits=3)) == tq.TQ_ERR_UNSUPPORTED

    def dec_app(xk=x, xdt=1, wsb=ws):
        return L.tq_paged_decode_attn_append(ctypes.byref(k), ctypes.byref(v), xk, x + 0x80000, xdt, FAKE + 0x600000,
                                             1, 16, sp, 4096, 0.088, FAKE + 0x700000, None, FAKE + 0x800000, wsb, None)

    assert dec_app(xk=0) == tq.TQ_ERR_INVALID_ARG
    assert dec_app(xk=x + 8) == tq.TQ_ERR_INVALID_ARG
    assert dec_app(xdt=4) == tq.TQ_ERR_INVALID_ARG
    assert dec_app(wsb=16) == tq.TQ_ERR_WORKSPACE


def test_paged_ext_argument_validation():
    """tq_paged_decode_attn_ext: several positions or Sparse V (not both), the same page,
    width and workspace rules as the paged decode."""
    L = tq.lib()
    k, v = _paged(), _paged(layout=1, bits=2, codes=FAKE + 0x2000000, norms=FAKE + 0x3000000)
    sp = FAKE + 0x900000
    ws_multi = tq.paged_decode_ext_workspace_bytes(2, 16, 2, 4, 4096)
    ws_sparse = tq.paged_decode_ext_workspace_bytes(2, 16, 2, 1, 4096, 1e-4)
    assert ws_multi > 0 and ws_sparse > 0
    assert tq.paged_decode_ext_workspace_bytes(2, 16, 2, 4, 4096, 1e-4) == 0   # not both
    assert tq.paged_decode_ext_workspace_bytes(2, 16, 2, 0, 4096) == 0
    assert tq.paged_decode_ext_workspace_bytes(2, 16, 2, 1, 4096, 1.0) == 0
    assert tq.paged_decode_ext_workspace_bytes(2, 15, 2, 1, 4096) == 0

    def ext(k=k, v=v, hq=16, n_q=4, seq=sp, ctx=4096, tau=0.0, wsb=ws_multi, ws=FAKE + 0x800000, q=FAKE + 0x600000):
        return L.tq_paged_decode_attn_ext(ctypes.byref(k), ctypes.byref(v), q, 1, hq, n_q, seq, ctx, 0.088, tau,
                                          FAKE + 0x700000, None, ws, wsb, None)

    assert ext(seq=0) == tq.TQ_ERR_INVALID_ARG                          # lengths are required
    assert ext(ctx=4097) == tq.TQ_ERR_CAPACITY                          # 16 pages of 256
    assert ext(n_q=0) == tq.TQ_ERR_INVALID_ARG
    assert ext(n_q=1 << 20) == tq.TQ_ERR_INVALID_ARG
    assert ext(hq=7) == tq.TQ_ERR_INVALID_ARG
    assert ext(hq=64) == tq.TQ_ERR_UNSUPPORTED                          # group 32
    assert ext(tau=1e-4) == tq.TQ_ERR_UNSUPPORTED                       # Sparse V takes one position
    assert ext(n_q=1, tau=1.0) == tq.TQ_ERR_INVALID_ARG
    assert ext(n_q=1, tau=float("nan")) == tq.TQ_ERR_INVALID_ARG
    assert ext(n_q=1, tau=1e-4, wsb=ws_sparse - 1) == tq.TQ_ERR_WORKSPACE
    assert ext(wsb=ws_multi - 1) == tq.TQ_ERR_WORKSPACE
    assert ext(ws=FAKE + 0x800010) == tq.TQ_ERR_INVALID_ARG             # not 256-aligned
    assert ext(q=FAKE + 0x600002) == tq.TQ_ERR_INVALID_ARG
    assert ext(k=_paged(bits=8)) == tq.TQ_ERR_UNSUPPORTED
    assert ext(v=_paged(layout=1, bits=3)) == tq.TQ_ERR_UNSUPPORTED
    assert ext(v=k) == tq.TQ_ERR_INVALID_ARG                            # layouts


def test_ip_search_argument_validation():
    L = tq.lib()
    db = _cache(batch=1, n_kv_heads=1, capacity=65536)
    ws = tq.ip_search_workspace_bytes(4, 65536, 10)
    assert ws > 0
    assert tq.ip_search_workspace_bytes(4, 65536, 65) == 0          # top_k above 64
    assert tq.ip_search_workspace_bytes(4, 2 << 20, 64) > ws        # lists grow with blocks and k

    def srch(db=db, nq=4, n=65536, k=10, wsb=ws, out=FAKE + 0x700000, qdt=1):
        return L.tq_ip_search(ctypes.byref(db), FAKE + 0x600000, qdt, nq, n, k, out, FAKE + 0x780000,
                              FAKE + 0x800000, wsb, None)

    assert srch(n=65537) == tq.TQ_ERR_CAPACITY
    assert srch(k=0) == tq.TQ_ERR_INVALID_ARG
    assert srch(k=65) == tq.TQ_ERR_UNSUPPORTED
    assert srch(nq=0) == tq.TQ_ERR_INVALID_ARG
    assert srch(wsb=16) == tq.TQ_ERR_WORKSPACE
    assert srch(out=0) == tq.TQ_ERR_INVALID_ARG
    assert srch(qdt=3) == tq.TQ_ERR_INVALID_ARG
    assert srch(db=_cache(batch=2, n_kv_heads=1, capacity=65536)) == tq.TQ_ERR_UNSUPPORTED
    assert srch(db=_cache(batch=1, n_kv_heads=1, capacity=65536, bits=2)) == tq.TQ_ERR_UNSUPPORTED
    assert srch(db=_cache(batch=1, n_kv_heads=1, capacity=65536, layout=1)) == tq.TQ_ERR_UNSUPPORTED


def test_probe_rejects_bad_arguments():
    f = tq.lib().tq_probe_stream_read
    assert f(None, 1 << 20, FAKE, None) == tq.TQ_ERR_INVALID_ARG
    assert f(FAKE, 1 << 20, None, None) == tq.TQ_ERR_INVALID_ARG
    assert f(FAKE + 8, 1 << 20, FAKE, None) == tq.TQ_ERR_INVALID_ARG
    assert f(FAKE, 1000, FAKE, None) == tq.TQ_ERR_INVALID_ARG
    assert f(FAKE, 0, FAKE, None) == tq.TQ_ERR_INVALID_ARG


def test_binding_rejects_buffers_of_another_shape():
    """The binding checks caller-supplied output buffers, q and seq_lens against the call's
    (batch, query heads, context) before any launch: the kernels write scores with the call's
    ctx_len as row stride, so a buffer made for a shorter context must be refused.  Runs on
    CPU tensors: every check here comes before the device-pointer checks."""
    torch = pytest.importorskip("torch")
    signs = torch.ones(128, dtype=torch.int8)
    kc = tq.PackedCache(2, 2, 256, 4, tq.LAYOUT_ROWS, signs, device="cpu")
    vc = tq.PackedCache(2, 2, 256, 2, tq.LAYOUT_GROUP8, signs, device="cpu")
    q = torch.zeros(2, 8, 128)
    short = tq.DecodeBuffers(2, 8, 2, 128, 0.0, device="cpu", want_scores=True)
    with pytest.raises(ValueError, match="scores"):
        tq.decode_attn(kc, vc, q, 256, 0.1, buffers=short)
    other_heads = tq.DecodeBuffers(2, 4, 2, 256, 0.0, device="cpu")
    with pytest.raises(ValueError, match="out"):
        tq.decode_attn(kc, vc, q, 256, 0.1, buffers=other_heads)
    with pytest.raises(ValueError, match="batch"):
        tq.decode_attn(kc, vc, torch.zeros(3, 8, 128), 256, 0.1)
    with pytest.raises(ValueError, match="seq_lens"):
        tq.decode_attn(kc, vc, q, 256, 0.1, seq_lens=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="seq_lens"):
        tq.decode_attn(kc, vc, q, 256, 0.1, seq_lens=torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError, match="kv heads"):
        tq.decode_attn(kc, vc, torch.zeros(2, 7, 128), 256, 0.1)
    new = torch.zeros(2, 1, 2, 128)
    with pytest.raises(ValueError, match="out"):
        tq.decode_attn_append(kc, vc, new, new, q, 256, 0.1, buffers=other_heads)
    mq = tq.MultiQueryBuffers(2, 3, 8, 2, 256, device="cpu")
    with pytest.raises(ValueError, match="out"):
        tq.decode_attn_multi(kc, vc, torch.zeros(2, 4, 8, 128), 256, 0.1, buffers=mq)
    pk = tq.PagedCache(2, 2, 64, 8, 4, 4, tq.LAYOUT_ROWS, signs, device="cpu")
    pv = tq.PagedCache(2, 2, 64, 8, 4, 2, tq.LAYOUT_GROUP8, signs, block_table=pk.block_table, device="cpu")
    pb = tq.PagedDecodeBuffers(1, 8, 2, 256, device="cpu")
    lens = torch.full((2,), 256, dtype=torch.int32)
    with pytest.raises(ValueError, match="out"):
        tq.paged_decode_attn(pk, pv, q, lens, 256, 0.1, buffers=pb)
    with pytest.raises(ValueError, match="seq_lens"):
        tq.paged_decode_attn(pk, pv, q, None, 256, 0.1)
    # a correctly shaped call gets past every shape check and stops at the device check
    ok = tq.DecodeBuffers(2, 8, 2, 256, 0.0, device="cpu", want_scores=True)
    with pytest.raises(ValueError, match="device tensor"):
        tq.decode_attn(kc, vc, q, 256, 0.1, buffers=ok)

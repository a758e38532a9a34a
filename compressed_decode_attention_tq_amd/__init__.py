"""TurboQuant compressed-KV quantize and decode attention for MI355X (gfx950).

Thin Python binding over the C ABI of libtq.so (declared in include/tq.h).  It only
marshals arguments: every step of quantize, decode attention and dequantize runs in the
HIP kernels of the library.  PyTorch provides device memory and the current stream.
There is no CPU fallback: if libtq.so has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import functools
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtq.so")

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_WORKSPACE, TQ_ERR_HIP = (
    0, -1, -2, -3, -4, -5)
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
LAYOUT_ROWS, LAYOUT_GROUP8 = 0, 1
D = 128


class TQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class CacheStruct(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32), ("bits", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("capacity", ctypes.c_int32),
        ("codes", ctypes.c_void_p), ("norms", ctypes.c_void_p), ("centroids", ctypes.c_void_p),
        ("boundaries", ctypes.c_void_p), ("signs", ctypes.c_void_p), ("table_scale", ctypes.c_float),
    ]


class QjlSketchStruct(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("bits", ctypes.c_void_p), ("res_norms", ctypes.c_void_p),
                ("proj", ctypes.c_void_p)]


class PagedCacheStruct(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32), ("bits", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
        ("n_pages", ctypes.c_int32), ("max_pages", ctypes.c_int32),
        ("codes", ctypes.c_void_p), ("norms", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("centroids", ctypes.c_void_p), ("boundaries", ctypes.c_void_p), ("signs", ctypes.c_void_p),
        ("table_scale", ctypes.c_float),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtq.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m compressed_decode_attention_tq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.tq_make_codebook_table.argtypes = [i32, i32, vp, vp]
        L.tq_value_table_scale.argtypes = [vp, i32]
        L.tq_value_table_scale.restype = f32
        L.tq_quantize_append.argtypes = [ctypes.POINTER(CacheStruct), vp, i32, i32, i32, vp]
        L.tq_quantize_append_kv.argtypes = [ctypes.POINTER(CacheStruct), ctypes.POINTER(CacheStruct), vp, vp,
                                            i32, i32, i32, vp]
        L.tq_decode_attn.argtypes = [ctypes.POINTER(CacheStruct), ctypes.POINTER(CacheStruct), vp, i32,
                                     i32, vp, i32, f32, f32, vp, vp, vp, vp, sz, vp]
        L.tq_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, f32]
        L.tq_decode_workspace_bytes.restype = sz
        L.tq_decode_attn_multi.argtypes = [ctypes.POINTER(CacheStruct), ctypes.POINTER(CacheStruct), vp, i32,
                                           i32, i32, vp, i32, f32, vp, vp, vp, sz, vp]
        L.tq_decode_attn_multi_append.argtypes = [ctypes.POINTER(CacheStruct), ctypes.POINTER(CacheStruct), vp, vp,
                                                  i32, vp, i32, i32, i32, vp, i32, f32, vp, vp, vp, sz, vp]
        L.tq_decode_attn_multi_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.tq_decode_attn_append.argtypes = [ctypes.POINTER(CacheStruct), ctypes.POINTER(CacheStruct), vp, vp, i32,
                                            vp, i32, i32, vp, i32, f32, vp, vp, vp, sz, vp]
        L.tq_decode_attn_append_sparse.argtypes = [ctypes.POINTER(CacheStruct), ctypes.POINTER(CacheStruct), vp, vp,
                                                   i32, vp, i32, i32, vp, i32, f32, f32, vp, vp, vp, sz, vp]
        L.tq_decode_attn_multi_workspace_bytes.restype = sz
        L.tq_decode_attn_append_noalloc.argtypes = [ctypes.POINTER(CacheStruct), ctypes.POINTER(CacheStruct), vp,
                                                    vp, i32, vp, i32, i32, vp, i32, f32, vp, vp, vp]
        L.tq_dequantize.argtypes = [ctypes.POINTER(CacheStruct), i32, i32, vp, i32, vp]
        PP = ctypes.POINTER(PagedCacheStruct)
        L.tq_paged_quantize_append_kv.argtypes = [PP, PP, vp, vp, i32, vp, i32, vp]
        L.tq_paged_decode_attn.argtypes = [PP, PP, vp, i32, i32, vp, i32, f32, vp, vp, vp, sz, vp]
        L.tq_paged_decode_attn_append.argtypes = [PP, PP, vp, vp, i32, vp, i32, i32, vp, i32, f32, vp, vp, vp, sz,
                                                  vp]
        L.tq_ip_search.argtypes = [ctypes.POINTER(CacheStruct), vp, i32, i32, i32, i32, vp, vp, vp, sz, vp]
        QP = ctypes.POINTER(QjlSketchStruct)
        L.tq_qjl_quantize_append.argtypes = [ctypes.POINTER(CacheStruct), QP, vp, i32, i32, i32, vp]
        L.tq_qjl_quantize_append_kv.argtypes = [ctypes.POINTER(CacheStruct), QP, ctypes.POINTER(CacheStruct), vp, vp,
                                                i32, i32, i32, vp]
        L.tq_qjl_decode_attn.argtypes = [ctypes.POINTER(CacheStruct), QP, ctypes.POINTER(CacheStruct), vp, i32, i32,
                                         vp, i32, f32, f32, vp, vp, vp, vp, sz, vp]
        L.tq_ip_search_workspace_bytes.argtypes = [i32, i32, i32]
        L.tq_ip_search_workspace_bytes.restype = sz
        L.tq_paged_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.tq_paged_decode_workspace_bytes.restype = sz
        L.tq_paged_decode_attn_ext.argtypes = [PP, PP, vp, i32, i32, i32, vp, i32, f32, f32, vp, vp, vp, sz, vp]
        L.tq_paged_decode_ext_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, f32]
        L.tq_paged_decode_ext_workspace_bytes.restype = sz
        L.tq_probe_stream_read.argtypes = [vp, sz, vp, vp]
        L.tq_code_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.tq_code_bytes.restype = sz
        L.tq_status_string.argtypes = [i32]
        L.tq_status_string.restype = ctypes.c_char_p
        for name in ("tq_make_codebook_table", "tq_quantize_append", "tq_quantize_append_kv", "tq_decode_attn",
                     "tq_decode_attn_multi", "tq_decode_attn_multi_append", "tq_decode_attn_append",
                     "tq_decode_attn_append_sparse",
                     "tq_decode_attn_append_noalloc", "tq_dequantize", "tq_probe_stream_read",
                     "tq_paged_quantize_append_kv", "tq_paged_decode_attn", "tq_paged_decode_attn_append", "tq_ip_search",
                     "tq_qjl_quantize_append", "tq_qjl_quantize_append_kv", "tq_qjl_decode_attn",
                     "tq_paged_decode_attn_ext"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().tq_status_string(status).decode()


def _check(status: int, what: str):
    if status != TQ_OK:
        raise TQError(status, what)


def make_codebook_table(d: int, bits: int):
    """Host call: fp32 (centroids[2^bits], boundaries[2^bits - 1]) as numpy arrays."""
    c, t = _codebook_table(d, bits)
    return c.copy(), t.copy()


@functools.lru_cache(maxsize=None)
def _codebook_table(d: int, bits: int):
    c = np.zeros(1 << bits, dtype=np.float32)
    t = np.zeros(max((1 << bits) - 1, 1), dtype=np.float32)
    _check(lib().tq_make_codebook_table(d, bits, c.ctypes.data, t.ctypes.data), "tq_make_codebook_table")
    return c, t[: (1 << bits) - 1]


def value_table_scale(centroids) -> float:
    """Host call: the table_scale for a cache with these fp32 centroids (1.0 when none applies)."""
    c = np.ascontiguousarray(centroids, dtype=np.float32)
    return float(lib().tq_value_table_scale(c.ctypes.data, int(c.size)))


def code_bytes(d: int, bits: int, batch: int, n_kv_heads: int, capacity: int) -> int:
    return int(lib().tq_code_bytes(d, bits, batch, n_kv_heads, capacity))


def decode_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, ctx_len: int, tau: float) -> int:
    return int(lib().tq_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, ctx_len, tau))


def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return TQ_F32
    if dt == torch.bfloat16:
        return TQ_BF16
    if dt == torch.float16:
        return TQ_F16
    raise TypeError(f"unsupported dtype {dt}")


def _stream_ptr(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, want, name):
    """Raise ValueError unless tensor t has exactly the shape `want` (checked before any launch:
    the kernels index caller buffers with the call's sizes, not the buffers')."""
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, the call needs {tuple(want)}")


def _check_query(q, cache, n_dims, what):
    if q.dim() != n_dims:
        raise ValueError(f"{what}: q must have {n_dims} dimensions, got shape {tuple(q.shape)}")
    if q.shape[0] != cache.batch:
        raise ValueError(f"{what}: q has batch {q.shape[0]}, the caches hold {cache.batch} sequences")
    if q.shape[-1] != cache.d:
        raise ValueError(f"{what}: q has head dim {q.shape[-1]}, the caches {cache.d}")
    if q.shape[-2] % cache.n_kv_heads != 0:
        raise ValueError(f"{what}: {q.shape[-2]} query heads is not a multiple of {cache.n_kv_heads} kv heads")


def _check_seq_lens(seq_lens, batch, what, required=False):
    if seq_lens is None:
        if required:
            raise ValueError(f"{what}: seq_lens is required")
        return
    torch = _torch()
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (batch,):
        raise ValueError(f"{what}: seq_lens must be int32 of shape ({batch},), got {seq_lens.dtype} "
                         f"{tuple(seq_lens.shape)}")


def _check_outputs(buffers, out_shape, lse_shape, what, scores_shape=None):
    torch = _torch()
    _shape(buffers.out, out_shape, f"{what}: out")
    if buffers.out.dtype != torch.float32:
        raise ValueError(f"{what}: out must be float32")
    lse = getattr(buffers, "lse", None)
    if lse is not None:
        _shape(lse, lse_shape, f"{what}: lse")
        if lse.dtype != torch.float32:
            raise ValueError(f"{what}: lse must be float32")
    scores = getattr(buffers, "scores", None)
    if scores is not None:
        if scores_shape is None:
            raise ValueError(f"{what}: this call writes no scores")
        _shape(scores, scores_shape, f"{what}: scores")
        if scores.dtype != torch.float32:
            raise ValueError(f"{what}: scores must be float32")


class PackedCache:
    """One K or V cache of one layer: packed codes + fp16 norms + codebook + signs (device)."""

    def __init__(self, batch: int, n_kv_heads: int, capacity: int, bits: int, layout: int,
                 signs, device="cuda", d: int = D):
        torch = _torch()
        self.d, self.bits, self.layout = d, bits, layout
        self.batch, self.n_kv_heads, self.capacity = batch, n_kv_heads, capacity
        nbytes = batch * n_kv_heads * capacity * d * bits // 8
        self.codes = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.norms = torch.zeros(batch * n_kv_heads * capacity, dtype=torch.float16, device=device)
        c, t = make_codebook_table(d, bits)
        self.centroids = torch.from_numpy(c).to(device)
        self.boundaries = torch.from_numpy(np.concatenate([t, [0.0]]).astype(np.float32)).to(device)
        self.table_scale = value_table_scale(c)
        if signs.is_cuda and signs.dtype == torch.int8 and signs.is_contiguous():
            self.signs = signs          # shared: the K and V caches of a layer use one sign vector
        else:
            self.signs = signs.to(device=device, dtype=torch.int8).contiguous()

    def struct(self) -> CacheStruct:
        return CacheStruct(self.d, self.bits, self.layout, self.batch, self.n_kv_heads, self.capacity,
                           self.codes.data_ptr(), self.norms.data_ptr(), self.centroids.data_ptr(),
                           self.boundaries.data_ptr(), self.signs.data_ptr(), self.table_scale)

    def plane_codes(self, b: int, h: int):
        per = self.capacity * self.d * self.bits // 8
        i = b * self.n_kv_heads + h
        return self.codes[i * per:(i + 1) * per]

    def plane_norms(self, b: int, h: int):
        i = b * self.n_kv_heads + h
        return self.norms[i * self.capacity:(i + 1) * self.capacity]


def quantize_append(cache: PackedCache, x, start_pos: int, stream=None):
    """Quantize x [batch, n_tokens, n_kv_heads, d] into positions start_pos .. start_pos+n_tokens."""
    if x.dim() != 4 or x.shape[0] != cache.batch or x.shape[2] != cache.n_kv_heads or x.shape[3] != cache.d:
        raise ValueError(f"x has shape {tuple(x.shape)}")
    st = cache.struct()
    _check(lib().tq_quantize_append(ctypes.byref(st), _dev(x, "x"), _dtype_code(x.dtype), start_pos,
                                    x.shape[1], _stream_ptr(stream)), "tq_quantize_append")


def quantize_append_kv(k_cache: PackedCache, v_cache: PackedCache, k, v, start_pos: int, stream=None):
    """quantize_append of k into k_cache and v into v_cache, one launch (row-layout keys,
    value-group values; same batch, kv heads and capacity)."""
    for name, cache, x in (("k", k_cache, k), ("v", v_cache, v)):
        if x.dim() != 4 or x.shape[0] != cache.batch or x.shape[2] != cache.n_kv_heads or x.shape[3] != cache.d:
            raise ValueError(f"{name} has shape {tuple(x.shape)}")
    if k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    ks, vs = k_cache.struct(), v_cache.struct()
    _check(lib().tq_quantize_append_kv(ctypes.byref(ks), ctypes.byref(vs), _dev(k, "k"), _dev(v, "v"),
                                       _dtype_code(k.dtype), start_pos, k.shape[1], _stream_ptr(stream)),
           "tq_quantize_append_kv")


def probe_stream_read(buf, sink, stream=None):
    """One launch of the streaming-read probe over the device tensor `buf` (measurement
    only); `sink` is a device int32 tensor of at least one element."""
    _check(lib().tq_probe_stream_read(_dev(buf, "buf"), buf.numel() * buf.element_size(), _dev(sink, "sink"),
                                      _stream_ptr(stream)), "tq_probe_stream_read")


def dequantize(cache: PackedCache, start_pos: int, n_tokens: int, dtype=None, stream=None):
    """x_hat [batch, n_tokens, n_kv_heads, d] for cache positions start_pos .. start_pos+n_tokens."""
    torch = _torch()
    dtype = torch.float32 if dtype is None else dtype
    out = torch.empty((cache.batch, n_tokens, cache.n_kv_heads, cache.d), dtype=dtype,
                      device=cache.codes.device)
    st = cache.struct()
    _check(lib().tq_dequantize(ctypes.byref(st), start_pos, n_tokens, _dev(out, "out"),
                               _dtype_code(dtype), _stream_ptr(stream)), "tq_dequantize")
    return out


class DecodeBuffers:
    """Caller-owned outputs and workspace of one decode problem shape."""

    def __init__(self, batch, n_q_heads, n_kv_heads, ctx_len, tau, device="cuda", d=D,
                 want_lse=True, want_scores=False):
        torch = _torch()
        self.out = torch.empty((batch, n_q_heads, d), dtype=torch.float32, device=device)
        self.lse = torch.empty((batch, n_q_heads), dtype=torch.float32, device=device) if want_lse else None
        self.scores = (torch.empty((batch, n_q_heads, ctx_len), dtype=torch.float32, device=device)
                       if want_scores else None)
        nbytes = decode_workspace_bytes(batch, n_q_heads, n_kv_heads, ctx_len, tau)
        if nbytes == 0:
            raise TQError(TQ_ERR_INVALID_ARG, "tq_decode_workspace_bytes")
        # zero once: the decode call's arrival counters live here and return to zero
        self.workspace = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.workspace.data_ptr()) % 256
        self.ws_ptr = self.workspace.data_ptr() + off
        self.ws_bytes = nbytes


def decode_attn(k_cache: PackedCache, v_cache: PackedCache, q, ctx_len: int, scale: float,
                tau: float = 0.0, seq_lens=None, buffers: DecodeBuffers | None = None,
                want_scores: bool = False, stream=None):
    """Decode attention; returns the DecodeBuffers holding out [B, Hq, d], lse and scores."""
    _check_query(q, k_cache, 3, "decode_attn")
    bsz, hq, d = q.shape
    _check_seq_lens(seq_lens, bsz, "decode_attn")
    if buffers is None:
        buffers = DecodeBuffers(bsz, hq, k_cache.n_kv_heads, ctx_len, tau, device=q.device,
                                d=d, want_scores=want_scores)
    _check_outputs(buffers, (bsz, hq, d), (bsz, hq), "decode_attn", scores_shape=(bsz, hq, ctx_len))
    ks, vs = k_cache.struct(), v_cache.struct()
    sl = _dev(seq_lens, "seq_lens") if seq_lens is not None else None
    _check(lib().tq_decode_attn(
        ctypes.byref(ks), ctypes.byref(vs), _dev(q, "q"), _dtype_code(q.dtype), hq, sl, ctx_len,
        float(scale), float(tau), _dev(buffers.out, "out"),
        _dev(buffers.lse, "lse") if buffers.lse is not None else None,
        _dev(buffers.scores, "scores") if buffers.scores is not None else None,
        ctypes.c_void_p(buffers.ws_ptr), buffers.ws_bytes, _stream_ptr(stream)), "tq_decode_attn")
    return buffers


def decode_attn_multi_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, n_q: int, ctx_len: int) -> int:
    return int(lib().tq_decode_attn_multi_workspace_bytes(batch, n_q_heads, n_kv_heads, n_q, ctx_len))


class MultiQueryBuffers:
    """Caller-owned outputs and workspace of one multi-query problem shape."""

    def __init__(self, batch, n_q, n_q_heads, n_kv_heads, ctx_len, device="cuda", d=D, want_lse=True):
        torch = _torch()
        self.out = torch.empty((batch, n_q, n_q_heads, d), dtype=torch.float32, device=device)
        self.lse = (torch.empty((batch, n_q, n_q_heads), dtype=torch.float32, device=device)
                    if want_lse else None)
        nbytes = decode_attn_multi_workspace_bytes(batch, n_q_heads, n_kv_heads, n_q, ctx_len)
        if nbytes == 0:
            raise TQError(TQ_ERR_INVALID_ARG, "tq_decode_attn_multi_workspace_bytes")
        # zero once: the arrival counters live here and every call leaves them at zero
        self.workspace = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.workspace.data_ptr()) % 256
        self.ws_ptr = self.workspace.data_ptr() + off
        self.ws_bytes = nbytes


def decode_attn_multi(k_cache: PackedCache, v_cache: PackedCache, q, ctx_len: int, scale: float,
                      seq_lens=None, buffers: MultiQueryBuffers | None = None, stream=None):
    """Attention of the last n_q positions of each sequence (q [B, n_q, Hq, d]) over the packed
    cache, causal; returns the MultiQueryBuffers holding out [B, n_q, Hq, d] and lse."""
    _check_query(q, k_cache, 4, "decode_attn_multi")
    bsz, n_q, hq, d = q.shape
    _check_seq_lens(seq_lens, bsz, "decode_attn_multi")
    if buffers is None:
        buffers = MultiQueryBuffers(bsz, n_q, hq, k_cache.n_kv_heads, ctx_len, device=q.device, d=d)
    _check_outputs(buffers, (bsz, n_q, hq, d), (bsz, n_q, hq), "decode_attn_multi")
    ks, vs = k_cache.struct(), v_cache.struct()
    sl = _dev(seq_lens, "seq_lens") if seq_lens is not None else None
    _check(lib().tq_decode_attn_multi(
        ctypes.byref(ks), ctypes.byref(vs), _dev(q, "q"), _dtype_code(q.dtype), hq, n_q, sl, ctx_len,
        float(scale), _dev(buffers.out, "out"),
        _dev(buffers.lse, "lse") if buffers.lse is not None else None,
        ctypes.c_void_p(buffers.ws_ptr), buffers.ws_bytes, _stream_ptr(stream)), "tq_decode_attn_multi")
    return buffers


def decode_attn_multi_append(k_cache: PackedCache, v_cache: PackedCache, k_new, v_new, q, ctx_len: int, scale: float,
                             seq_lens=None, buffers: MultiQueryBuffers | None = None, stream=None):
    """Quantize k_new, v_new [B, n_q, Hkv, d] into positions T_b - n_q .. T_b - 1, then
    decode_attn_multi for q [B, n_q, Hq, d] (one launch for up to 8 positions); returns the
    MultiQueryBuffers."""
    _check_query(q, k_cache, 4, "decode_attn_multi_append")
    bsz, n_q, hq, d = q.shape
    for name, cache, x in (("k_new", k_cache, k_new), ("v_new", v_cache, v_new)):
        if x.dim() != 4 or x.shape[0] != bsz or x.shape[1] != n_q or x.shape[2] != cache.n_kv_heads or x.shape[3] != d:
            raise ValueError(f"{name} has shape {tuple(x.shape)}")
    if k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same dtype")
    _check_seq_lens(seq_lens, bsz, "decode_attn_multi_append")
    if buffers is None:
        buffers = MultiQueryBuffers(bsz, n_q, hq, k_cache.n_kv_heads, ctx_len, device=q.device, d=d)
    _check_outputs(buffers, (bsz, n_q, hq, d), (bsz, n_q, hq), "decode_attn_multi_append")
    ks, vs = k_cache.struct(), v_cache.struct()
    sl = _dev(seq_lens, "seq_lens") if seq_lens is not None else None
    _check(lib().tq_decode_attn_multi_append(
        ctypes.byref(ks), ctypes.byref(vs), _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dtype_code(k_new.dtype),
        _dev(q, "q"), _dtype_code(q.dtype), hq, n_q, sl, ctx_len, float(scale), _dev(buffers.out, "out"),
        _dev(buffers.lse, "lse") if buffers.lse is not None else None,
        ctypes.c_void_p(buffers.ws_ptr), buffers.ws_bytes, _stream_ptr(stream)), "tq_decode_attn_multi_append")
    return buffers


def decode_attn_append(k_cache: PackedCache, v_cache: PackedCache, k_new, v_new, q, ctx_len: int,
                       scale: float, seq_lens=None, buffers: DecodeBuffers | None = None, stream=None,
                       tau: float = 0.0):
    """Quantize k_new, v_new [B, 1, Hkv, d] into position T_b - 1 of each sequence, then decode
    attention: dense (one launch where the fused kernel applies), or with Sparse V at tau > 0
    (the new token written by the key pass where it runs on matrix cores); returns the
    DecodeBuffers (sized for tau)."""
    _check_query(q, k_cache, 3, "decode_attn_append")
    bsz, hq, d = q.shape
    for name, cache, x in (("k_new", k_cache, k_new), ("v_new", v_cache, v_new)):
        if x.dim() != 4 or x.shape[0] != bsz or x.shape[1] != 1 or x.shape[2] != cache.n_kv_heads or x.shape[3] != d:
            raise ValueError(f"{name} has shape {tuple(x.shape)}")
    if k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same dtype")
    _check_seq_lens(seq_lens, bsz, "decode_attn_append")
    if buffers is None:
        buffers = DecodeBuffers(bsz, hq, k_cache.n_kv_heads, ctx_len, tau, device=q.device, d=d)
    _check_outputs(buffers, (bsz, hq, d), (bsz, hq), "decode_attn_append")
    ks, vs = k_cache.struct(), v_cache.struct()
    sl = _dev(seq_lens, "seq_lens") if seq_lens is not None else None
    head = (ctypes.byref(ks), ctypes.byref(vs), _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dtype_code(k_new.dtype),
            _dev(q, "q"), _dtype_code(q.dtype), hq, sl, ctx_len, float(scale))
    tail = (_dev(buffers.out, "out"), _dev(buffers.lse, "lse") if buffers.lse is not None else None,
            ctypes.c_void_p(buffers.ws_ptr), buffers.ws_bytes, _stream_ptr(stream))
    if tau == 0.0:
        _check(lib().tq_decode_attn_append(*head, *tail), "tq_decode_attn_append")
    else:
        _check(lib().tq_decode_attn_append_sparse(*head, float(tau), *tail), "tq_decode_attn_append_sparse")
    return buffers


def decode_attn_append_noalloc(k_cache: PackedCache, v_cache: PackedCache, k_new, v_new, q, ctx_len: int,
                               scale: float, seq_lens=None, out=None, lse=None, stream=None):
    """decode_attn_append through the allocation-free entry point: the library's static
    scratch replaces the workspace.  out [B, Hq, d] and lse [B, Hq] (float32, device) may be
    given by the caller; returns (out, lse)."""
    torch = _torch()
    _check_query(q, k_cache, 3, "decode_attn_append_noalloc")
    bsz, hq, d = q.shape
    for name, cache, x in (("k_new", k_cache, k_new), ("v_new", v_cache, v_new)):
        if x.dim() != 4 or x.shape[0] != bsz or x.shape[1] != 1 or x.shape[2] != cache.n_kv_heads or x.shape[3] != d:
            raise ValueError(f"{name} has shape {tuple(x.shape)}")
    if k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same dtype")
    _check_seq_lens(seq_lens, bsz, "decode_attn_append_noalloc")
    if out is None:
        out = torch.empty((bsz, hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((bsz, hq), dtype=torch.float32, device=q.device)
    _shape(out, (bsz, hq, d), "decode_attn_append_noalloc: out")
    _shape(lse, (bsz, hq), "decode_attn_append_noalloc: lse")
    ks, vs = k_cache.struct(), v_cache.struct()
    sl = _dev(seq_lens, "seq_lens") if seq_lens is not None else None
    _check(lib().tq_decode_attn_append_noalloc(
        ctypes.byref(ks), ctypes.byref(vs), _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dtype_code(k_new.dtype),
        _dev(q, "q"), _dtype_code(q.dtype), hq, sl, ctx_len, float(scale), _dev(out, "out"), _dev(lse, "lse"),
        _stream_ptr(stream)), "tq_decode_attn_append_noalloc")
    return out, lse


class QjlSketch:
    """The QJL sign sketch beside a key cache (device): bits [batch, n_kv_heads, capacity, m/8]
    uint8, residual norms [batch, n_kv_heads, capacity] fp16, and the sketch matrix S [m, d]
    fp32 (drawn by the caller)."""

    def __init__(self, key_cache: PackedCache, proj, device="cuda"):
        torch = _torch()
        self.m = int(proj.shape[0])
        c = key_cache
        self.bits = torch.zeros(c.batch * c.n_kv_heads * c.capacity * self.m // 8, dtype=torch.uint8, device=device)
        self.res_norms = torch.zeros(c.batch * c.n_kv_heads * c.capacity, dtype=torch.float16, device=device)
        self.proj = proj.to(device=device, dtype=torch.float32).contiguous()
        self.capacity, self.n_kv_heads = c.capacity, c.n_kv_heads

    def struct(self) -> QjlSketchStruct:
        return QjlSketchStruct(self.m, self.bits.data_ptr(), self.res_norms.data_ptr(), self.proj.data_ptr())

    def plane_bits(self, b: int, h: int):
        per = self.capacity * self.m // 8
        i = b * self.n_kv_heads + h
        return self.bits[i * per:(i + 1) * per]

    def plane_res_norms(self, b: int, h: int):
        i = b * self.n_kv_heads + h
        return self.res_norms[i * self.capacity:(i + 1) * self.capacity]


def qjl_quantize_append(k_cache: PackedCache, sketch: QjlSketch, x, start_pos: int, stream=None):
    """QJL keys: quantize x [batch, n_tokens, n_kv_heads, d] into the key cache (codes, norms)
    and the sketch (sign bits, residual norms) at positions start_pos .. start_pos+n_tokens."""
    if x.dim() != 4 or x.shape[0] != k_cache.batch or x.shape[2] != k_cache.n_kv_heads or x.shape[3] != k_cache.d:
        raise ValueError(f"x has shape {tuple(x.shape)}")
    st, ss = k_cache.struct(), sketch.struct()
    _check(lib().tq_qjl_quantize_append(ctypes.byref(st), ctypes.byref(ss), _dev(x, "x"), _dtype_code(x.dtype),
                                        start_pos, x.shape[1], _stream_ptr(stream)), "tq_qjl_quantize_append")


def qjl_quantize_append_kv(k_cache: PackedCache, sketch: QjlSketch, v_cache: PackedCache, xk, xv, start_pos: int,
                           stream=None):
    """QJL keys and plain values of one step: xk into the key cache and its sketch, xv
    [batch, n_tokens, n_kv_heads, d] into the value cache, positions start_pos .. +n_tokens (one
    launch for up to 8 tokens)."""
    for name, x in (("xk", xk), ("xv", xv)):
        if x.dim() != 4 or x.shape[0] != k_cache.batch or x.shape[2] != k_cache.n_kv_heads or x.shape[3] != k_cache.d:
            raise ValueError(f"{name} has shape {tuple(x.shape)}")
    if xk.shape != xv.shape or xk.dtype != xv.dtype:
        raise ValueError(f"xk {tuple(xk.shape)} {xk.dtype} and xv {tuple(xv.shape)} {xv.dtype} differ")
    ks, ss, vs = k_cache.struct(), sketch.struct(), v_cache.struct()
    _check(lib().tq_qjl_quantize_append_kv(ctypes.byref(ks), ctypes.byref(ss), ctypes.byref(vs), _dev(xk, "xk"),
                                           _dev(xv, "xv"), _dtype_code(xk.dtype), start_pos, xk.shape[1],
                                           _stream_ptr(stream)), "tq_qjl_quantize_append_kv")


def qjl_decode_attn(k_cache: PackedCache, sketch: QjlSketch, v_cache: PackedCache, q, ctx_len: int, scale: float,
                    tau: float = 0.0, seq_lens=None, buffers: DecodeBuffers | None = None, want_scores: bool = False,
                    stream=None):
    """Decode attention with QJL-corrected scores; returns the DecodeBuffers (out, lse, scores)."""
    _check_query(q, k_cache, 3, "qjl_decode_attn")
    bsz, hq, d = q.shape
    _check_seq_lens(seq_lens, bsz, "qjl_decode_attn")
    if buffers is None:
        buffers = DecodeBuffers(bsz, hq, k_cache.n_kv_heads, ctx_len, tau, device=q.device, d=d,
                                want_scores=want_scores)
    _check_outputs(buffers, (bsz, hq, d), (bsz, hq), "qjl_decode_attn", scores_shape=(bsz, hq, ctx_len))
    ks, ss, vs = k_cache.struct(), sketch.struct(), v_cache.struct()
    sl = _dev(seq_lens, "seq_lens") if seq_lens is not None else None
    _check(lib().tq_qjl_decode_attn(
        ctypes.byref(ks), ctypes.byref(ss), ctypes.byref(vs), _dev(q, "q"), _dtype_code(q.dtype), hq, sl, ctx_len,
        float(scale), float(tau), _dev(buffers.out, "out"),
        _dev(buffers.lse, "lse") if buffers.lse is not None else None,
        _dev(buffers.scores, "scores") if buffers.scores is not None else None,
        ctypes.c_void_p(buffers.ws_ptr), buffers.ws_bytes, _stream_ptr(stream)), "tq_qjl_decode_attn")
    return buffers


class PagedCache:
    """One paged K or V cache of one layer: a pool of pages (page_tokens positions of every kv
    head each) + the block table [batch, max_pages] (int32, -1 = no page) it is read through.
    The K and V caches of a layer share one block table (pass the K cache's `block_table`)."""

    def __init__(self, batch: int, n_kv_heads: int, page_tokens: int, n_pages: int, max_pages: int,
                 bits: int, layout: int, signs, block_table=None, device="cuda", d: int = D):
        torch = _torch()
        self.d, self.bits, self.layout = d, bits, layout
        self.batch, self.n_kv_heads, self.page_tokens = batch, n_kv_heads, page_tokens
        self.n_pages, self.max_pages = n_pages, max_pages
        self.codes = torch.zeros(n_pages * n_kv_heads * page_tokens * d * bits // 8, dtype=torch.uint8, device=device)
        self.norms = torch.zeros(n_pages * n_kv_heads * page_tokens, dtype=torch.float16, device=device)
        self.block_table = (torch.full((batch, max_pages), -1, dtype=torch.int32, device=device)
                            if block_table is None else block_table)
        c, t = make_codebook_table(d, bits)
        self.centroids = torch.from_numpy(c).to(device)
        self.boundaries = torch.from_numpy(np.concatenate([t, [0.0]]).astype(np.float32)).to(device)
        self.table_scale = value_table_scale(c)
        if signs.is_cuda and signs.dtype == torch.int8 and signs.is_contiguous():
            self.signs = signs
        else:
            self.signs = signs.to(device=device, dtype=torch.int8).contiguous()

    def struct(self) -> PagedCacheStruct:
        return PagedCacheStruct(self.d, self.bits, self.layout, self.batch, self.n_kv_heads, self.page_tokens,
                                self.n_pages, self.max_pages, self.codes.data_ptr(), self.norms.data_ptr(),
                                self.block_table.data_ptr(), self.centroids.data_ptr(),
                                self.boundaries.data_ptr(), self.signs.data_ptr(), self.table_scale)

    def page_codes(self, page: int, h: int):
        per = self.page_tokens * self.d * self.bits // 8
        i = page * self.n_kv_heads + h
        return self.codes[i * per:(i + 1) * per]

    def page_norms(self, page: int, h: int):
        i = page * self.n_kv_heads + h
        return self.norms[i * self.page_tokens:(i + 1) * self.page_tokens]


def paged_quantize_append_kv(k_cache: PagedCache, v_cache: PagedCache, xk, xv, start_pos, stream=None):
    """Quantize xk, xv [B, n, Hkv, d] into positions start_pos[b] + j of the paged caches."""
    for name, cache, x in (("xk", k_cache, xk), ("xv", v_cache, xv)):
        if x.dim() != 4 or x.shape[0] != cache.batch or x.shape[2] != cache.n_kv_heads or x.shape[3] != cache.d:
            raise ValueError(f"{name} has shape {tuple(x.shape)}")
    if xk.shape != xv.shape or xk.dtype != xv.dtype:
        raise ValueError("xk and xv must have the same shape and dtype")
    ks, vs = k_cache.struct(), v_cache.struct()
    _check(lib().tq_paged_quantize_append_kv(
        ctypes.byref(ks), ctypes.byref(vs), _dev(xk, "xk"), _dev(xv, "xv"), _dtype_code(xk.dtype),
        _dev(start_pos, "start_pos"), xk.shape[1], _stream_ptr(stream)), "tq_paged_quantize_append_kv")


def paged_decode_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, max_ctx_len: int) -> int:
    return int(lib().tq_paged_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, max_ctx_len))


def paged_decode_ext_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, n_q: int, max_ctx_len: int,
                                     tau: float = 0.0) -> int:
    return int(lib().tq_paged_decode_ext_workspace_bytes(batch, n_q_heads, n_kv_heads, n_q, max_ctx_len, tau))


class PagedDecodeBuffers:
    """Caller-owned outputs and workspace of one paged decode problem shape."""

    def __init__(self, batch, n_q_heads, n_kv_heads, max_ctx_len, device="cuda", d=D, want_lse=True):
        torch = _torch()
        self.out = torch.empty((batch, n_q_heads, d), dtype=torch.float32, device=device)
        self.lse = torch.empty((batch, n_q_heads), dtype=torch.float32, device=device) if want_lse else None
        nbytes = paged_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, max_ctx_len)
        if nbytes == 0:
            raise TQError(TQ_ERR_INVALID_ARG, "tq_paged_decode_workspace_bytes")
        # zero once: the arrival counters live here and every call leaves them at zero
        self.workspace = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.workspace.data_ptr()) % 256
        self.ws_ptr = self.workspace.data_ptr() + off
        self.ws_bytes = nbytes


def paged_decode_attn(k_cache: PagedCache, v_cache: PagedCache, q, seq_lens, max_ctx_len: int, scale: float,
                      buffers: PagedDecodeBuffers | None = None, stream=None):
    """Dense decode attention over paged caches; returns the PagedDecodeBuffers (out, lse)."""
    _check_query(q, k_cache, 3, "paged_decode_attn")
    bsz, hq, d = q.shape
    _check_seq_lens(seq_lens, bsz, "paged_decode_attn", required=True)
    if buffers is None:
        buffers = PagedDecodeBuffers(bsz, hq, k_cache.n_kv_heads, max_ctx_len, device=q.device, d=d)
    _check_outputs(buffers, (bsz, hq, d), (bsz, hq), "paged_decode_attn")
    ks, vs = k_cache.struct(), v_cache.struct()
    _check(lib().tq_paged_decode_attn(
        ctypes.byref(ks), ctypes.byref(vs), _dev(q, "q"), _dtype_code(q.dtype), hq, _dev(seq_lens, "seq_lens"),
        max_ctx_len, float(scale), _dev(buffers.out, "out"),
        _dev(buffers.lse, "lse") if buffers.lse is not None else None,
        ctypes.c_void_p(buffers.ws_ptr), buffers.ws_bytes, _stream_ptr(stream)), "tq_paged_decode_attn")
    return buffers


def paged_decode_attn_append(k_cache: PagedCache, v_cache: PagedCache, k_new, v_new, q, seq_lens, max_ctx_len: int,
                             scale: float, buffers: PagedDecodeBuffers | None = None, stream=None):
    """Quantize k_new, v_new [B, 1, Hkv, d] into position T_b - 1 of the paged caches and
    attend, in one launch; returns the PagedDecodeBuffers (out, lse)."""
    _check_query(q, k_cache, 3, "paged_decode_attn_append")
    bsz, hq, d = q.shape
    for name, cache, x in (("k_new", k_cache, k_new), ("v_new", v_cache, v_new)):
        if x.dim() != 4 or x.shape[0] != bsz or x.shape[1] != 1 or x.shape[2] != cache.n_kv_heads or x.shape[3] != d:
            raise ValueError(f"{name} has shape {tuple(x.shape)}")
    if k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must have the same dtype")
    _check_seq_lens(seq_lens, bsz, "paged_decode_attn_append", required=True)
    if buffers is None:
        buffers = PagedDecodeBuffers(bsz, hq, k_cache.n_kv_heads, max_ctx_len, device=q.device, d=d)
    _check_outputs(buffers, (bsz, hq, d), (bsz, hq), "paged_decode_attn_append")
    ks, vs = k_cache.struct(), v_cache.struct()
    _check(lib().tq_paged_decode_attn_append(
        ctypes.byref(ks), ctypes.byref(vs), _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dtype_code(k_new.dtype),
        _dev(q, "q"), _dtype_code(q.dtype), hq, _dev(seq_lens, "seq_lens"), max_ctx_len, float(scale),
        _dev(buffers.out, "out"), _dev(buffers.lse, "lse") if buffers.lse is not None else None,
        ctypes.c_void_p(buffers.ws_ptr), buffers.ws_bytes, _stream_ptr(stream)), "tq_paged_decode_attn_append")
    return buffers


class PagedExtBuffers:
    """Caller-owned outputs and workspace of tq_paged_decode_attn_ext: out [B, n_q, Hq, d] (or
    [B, Hq, d] for one position), lse, and the workspace."""

    def __init__(self, batch, n_q, n_q_heads, n_kv_heads, max_ctx_len, tau=0.0, device="cuda", d=D):
        torch = _torch()
        shape = (batch, n_q_heads) if n_q == 1 else (batch, n_q, n_q_heads)
        self.out = torch.empty(shape + (d,), dtype=torch.float32, device=device)
        self.lse = torch.empty(shape, dtype=torch.float32, device=device)
        nbytes = paged_decode_ext_workspace_bytes(batch, n_q_heads, n_kv_heads, n_q, max_ctx_len, tau)
        if nbytes == 0:
            raise TQError(TQ_ERR_INVALID_ARG, "tq_paged_decode_ext_workspace_bytes")
        # zero once: the arrival counters live here and every call leaves them at zero
        self.workspace = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.workspace.data_ptr()) % 256
        self.ws_ptr = self.workspace.data_ptr() + off
        self.ws_bytes = nbytes


def paged_decode_attn_ext(k_cache: PagedCache, v_cache: PagedCache, q, seq_lens, max_ctx_len: int, scale: float,
                          tau: float = 0.0, buffers: PagedExtBuffers | None = None, stream=None):
    """Paged attention of several query positions (q [B, n_q, Hq, d], causal) or Sparse V with one
    position (q [B, Hq, d], tau > 0); returns the PagedExtBuffers (out, lse)."""
    _check_query(q, k_cache, 3 if q.dim() == 3 else 4, "paged_decode_attn_ext")
    if q.dim() == 3:
        (bsz, hq, d), n_q = q.shape, 1
    else:
        bsz, n_q, hq, d = q.shape
    _check_seq_lens(seq_lens, bsz, "paged_decode_attn_ext", required=True)
    if buffers is None:
        buffers = PagedExtBuffers(bsz, n_q, hq, k_cache.n_kv_heads, max_ctx_len, tau, device=q.device, d=d)
    shape = (bsz, hq) if n_q == 1 else (bsz, n_q, hq)
    _check_outputs(buffers, shape + (d,), shape, "paged_decode_attn_ext")
    ks, vs = k_cache.struct(), v_cache.struct()
    _check(lib().tq_paged_decode_attn_ext(
        ctypes.byref(ks), ctypes.byref(vs), _dev(q, "q"), _dtype_code(q.dtype), hq, n_q, _dev(seq_lens, "seq_lens"),
        max_ctx_len, float(scale), float(tau), _dev(buffers.out, "out"), _dev(buffers.lse, "lse"),
        ctypes.c_void_p(buffers.ws_ptr), buffers.ws_bytes, _stream_ptr(stream)), "tq_paged_decode_attn_ext")
    return buffers


def ip_search_workspace_bytes(n_queries: int, n_vectors: int, top_k: int) -> int:
    return int(lib().tq_ip_search_workspace_bytes(n_queries, n_vectors, top_k))


class SearchBuffers:
    """Caller-owned outputs and workspace of one inner-product search shape."""

    def __init__(self, n_queries, n_vectors, top_k, device="cuda"):
        torch = _torch()
        self.idx = torch.empty((n_queries, top_k), dtype=torch.int32, device=device)
        self.score = torch.empty((n_queries, top_k), dtype=torch.float32, device=device)
        nbytes = ip_search_workspace_bytes(n_queries, n_vectors, top_k)
        if nbytes == 0:
            raise TQError(TQ_ERR_UNSUPPORTED, "tq_ip_search_workspace_bytes")
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.workspace.data_ptr()) % 256
        self.ws_ptr = self.workspace.data_ptr() + off
        self.ws_bytes = nbytes


def ip_search(db: PackedCache, q, n_vectors: int, top_k: int, buffers: SearchBuffers | None = None, stream=None):
    """Top-k inner-product search of q [Q, d] over vectors 0 .. n_vectors - 1 of the database
    cache (batch 1, one kv head, rows); returns the SearchBuffers (idx, score [Q, top_k])."""
    if q.dim() != 2 or q.shape[1] != db.d:
        raise ValueError(f"ip_search: q has shape {tuple(q.shape)}")
    nq, d = q.shape
    if buffers is None:
        buffers = SearchBuffers(nq, n_vectors, top_k, device=q.device)
    _shape(buffers.idx, (nq, top_k), "ip_search: idx")
    _shape(buffers.score, (nq, top_k), "ip_search: score")
    st = db.struct()
    _check(lib().tq_ip_search(ctypes.byref(st), _dev(q, "q"), _dtype_code(q.dtype), nq, n_vectors, top_k,
                              _dev(buffers.idx, "idx"), _dev(buffers.score, "score"), ctypes.c_void_p(buffers.ws_ptr),
                              buffers.ws_bytes, _stream_ptr(stream)), "tq_ip_search")
    return buffers

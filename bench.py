"""Benchmark of the TurboQuant compressed-KV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--tau T]

A step is one pass of the whole hot path over one batch of synthetic input:
  decode workloads: append-quantize one new token per (batch, kv head) into the K and V
                    caches (at the last position), then decode attention for every query
                    head over the full context;
  prefill:          quantize a 32-layer cache of 32768 tokens (K and V of every layer).
Inputs are resident in HBM before the timed region.  Decode workloads rotate over enough
copies of the cache (one per step, like the layers of a model) that the reads come from
HBM rather than the 256 MB Infinity Cache, and every timed batch starts cold: right
before it, a streaming read of 1 GiB of other data evicts the Infinity Cache and the L2s,
so no copy the timed steps read is still cached from the untimed replays.  The steps are
recorded once into a HIP graph and the graph is replayed, so the timed region holds GPU
work only (no Python launch overhead between kernels); --eager times plain launches
instead.  The default workload is the batched long-context decode (batch 16, 32 query
heads, 8 kv heads, 32768 tokens, K3/V2), the largest decode configuration.

Prints one JSON line: the throughput, the roofline of the dominant kernel (the single
decode-attention kernel, or quantize for prefill) timed with HIP events on the stream the
kernels run on, and the CPU oracle timed on this host.

Two helper modes turn rocprofv3 output into the short summaries kept under profiles/:
    python bench.py --summarize-stats DIR --name NAME --command "CMD"
    python bench.py --summarize-traffic --fetch DIR --write DIR --workload W --kernel K \
        --command "CMD"
(--calibrate-copy makes a timed run end with plain 512 MiB device copies: the FETCH_SIZE
and WRITE_SIZE they read scale the counters to bytes.)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "compressed-KV decode attention KV-tokens/s & HBM GB/s; quantize tokens/s"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense fp16 matrix peak of the MI355X
D = 128
COPY_BYTES = 512 << 20
STEADY_STEPS = 32  # back-to-back steps of the warm steady-state figure
MAX_COPIES = 256   # small workloads are launch-bound; more copies only lengthen the set-up
CALIBRATION_COPIES = 5
CALIBRATION_KERNEL = "copyBuffer"   # the HIP runtime's device-to-device copy kernel
DECODE_KERNEL = "decode_fused_kernel"
QUANTIZE_KERNEL = "quantize_kv_kernel"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="batch32k",
                   choices=["tiny", "llama8k", "batch32k", "prefill", "ctx131k", "verify8k", "paged32k", "search1m",
                            "qjl8k", "chunk8k"])
    p.add_argument("--tau", type=float, default=None, help="Sparse-V threshold (default: workload's)")
    p.add_argument("--copies", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--eager", action="store_true", help="time plain launches, no HIP graph")
    p.add_argument("--calibrate-copy", action="store_true")
    p.add_argument("--summarize-stats", default=None)
    p.add_argument("--summarize-traffic", action="store_true")
    p.add_argument("--summarize-instmix", default=None,
                   help="rocprofv3 --pmc directory with SQ_WAVES and SQ_INSTS_* counters")
    p.add_argument("--kernel-us", type=float, default=None, help="average launch time of --kernel")
    p.add_argument("--fetch", default=None)
    p.add_argument("--write", default=None)
    p.add_argument("--kernel", default=DECODE_KERNEL,
                   help="regular expression over the kernel names (template arguments included)")
    p.add_argument("--name", default=None)
    p.add_argument("--record", default=None,
                   help="traffic record name (profiles/traffic_<record>_<workload>.txt); default decode or quantize")
    p.add_argument("--sum-instances", action="store_true",
                   help="traffic per step = sum over the matching kernels (one dispatch each per step), "
                        "e.g. Sparse V's key pass and value pass")
    p.add_argument("--command", default="")
    return p.parse_args()


def kernel_sources_digest() -> str:
    """Digest of the kernel sources' code: comments and blank space are left out, so that a
    counter record stays valid across comment edits and goes stale on any code change."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "compressed_decode_attention_tq_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, kernel: str, digest: str):
    """Calibrated HBM bytes per launch from rocprofv3 counters, if taken on these sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("sources_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


def decode_bytes(w, bits_k, bits_v, hkv, batch, ctx):
    """Algorithmic bytes of one decode call: packed K and V codes + fp16 norms of every token."""
    per_token_head = (D * bits_k // 8 + 2) + (D * bits_v // 8 + 2)
    return batch * hkv * ctx * per_token_head


def append_bytes(w, bits_k, bits_v, hkv, batch):
    """Algorithmic bytes of appending one token per sequence: its K and V inputs read, packed
    codes + fp16 norms written."""
    in_bytes = w.dtype.itemsize
    return batch * hkv * (2 * D * in_bytes + (D * bits_k // 8 + 2) + (D * bits_v // 8 + 2))


def cpu_cores():
    """Host cores this process may run on (its affinity set)."""
    return len(os.sched_getaffinity(0))


def cpu_context():
    """The BLAS thread count (the oracle's dense-rotation matrix products may use that many
    threads; the rest of the oracle is single-threaded NumPy) and the CPU model string."""
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max((int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"),
                   default=None)
    except Exception:
        pass
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"blas_threads": blas, "cpu_model": model}


def with_cpu_context(rec):
    rec.update(cpu_context())
    return rec


def main():
    args = parse()
    if args.summarize_stats:
        summarize_stats(args)
        return
    if args.summarize_traffic:
        summarize_traffic(args)
        return
    if args.summarize_instmix:
        summarize_instmix(args)
        return
    try:  # the oracle's BLAS calls use at most the cores this process may run on
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=cpu_cores(), user_api="blas")
    except Exception:
        pass
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): it measures the single-GPU "
              "kernel; the path would shard by (batch, kv head) with no exchange.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import compressed_decode_attention_tq_amd as tq
    from compressed_decode_attention_tq_amd import inputs

    dev = "cuda:0"
    torch.cuda.set_device(0)

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    if args.workload in inputs.SEARCH:
        digest = kernel_sources_digest()
        result = bench_search(args, inputs.SEARCH[args.workload], inputs.rotation_signs().to(dev), dev, tq, inputs,
                              torch, np, log)
        stream = stream_read_gbs(torch, tq, log)
        result["roofline"]["stream_read_gbs"] = stream
        result["roofline"]["frac_of_stream_read"] = result["roofline"]["achieved"] / stream
        result["roofline"]["traffic"] = traffic_from_profiles(args.workload, result.pop("_kernel"), digest)
        result["sources_digest"] = digest
        if args.calibrate_copy:
            calibrate_copy(torch, log)
        print(json.dumps(result), flush=True)
        return
    w = inputs.WORKLOADS[args.workload]
    tau = w.tau if args.tau is None else args.tau
    if args.workload == "batch32k" and args.tau is None:
        tau = 0.0          # reported dense by default; pass --tau 1e-4 for Sparse V
    signs = inputs.rotation_signs().to(dev)
    digest = kernel_sources_digest()

    if args.workload == "prefill":
        result = bench_prefill(args, w, signs, dev, tq, inputs, torch, np, log)
    elif w.n_q > 1:
        result = bench_multi_query(args, w, signs, dev, tq, inputs, torch, np, log)
    elif w.page_tokens > 0:
        result = bench_paged(args, w, signs, dev, tq, inputs, torch, np, log)
    elif w.extra.get("qjl_m"):
        result = bench_qjl(args, w, signs, dev, tq, inputs, torch, np, log)
    else:
        result = bench_decode(args, w, tau, signs, dev, tq, inputs, torch, np, log)
    stream = stream_read_gbs(torch, tq, log)
    result["roofline"]["stream_read_gbs"] = stream
    if result["roofline"]["unit"] == "GB/s":
        result["roofline"]["frac_of_stream_read"] = result["roofline"]["achieved"] / stream
    traffic = traffic_from_profiles(args.workload, result.pop("_kernel"), digest)
    launches = result.pop("_launches", 1)  # traffic per step when a step is several launches
    result["roofline"]["traffic"] = None if traffic is None else traffic * launches
    result["sources_digest"] = digest
    if args.calibrate_copy:
        calibrate_copy(torch, log)
    print(json.dumps(result), flush=True)


class Timer:
    """Time of one iteration of a callable, with HIP events on the current stream.  Exactly
    `n` iterations are timed: they are recorded once into a HIP graph, the graph is replayed
    untimed (at least 3 times and 50 ms), then once between the events; or (eager) launched
    directly."""

    def __init__(self, torch, eager, flush=None):
        self.torch = torch
        self.eager = eager
        self.flush = flush  # run (untimed) before every timed batch: leaves the caches cold

    def per_iteration_ms(self, fn, n, warmup):
        return self.per_iteration_stats(fn, n, warmup, batches=1)[0]

    def per_iteration_stats(self, fn, n, warmup, batches):
        """(median, min, max) per-iteration ms over `batches` timed runs of the same n
        iterations (graph replays, or eager loops)."""
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream()
        times = []
        if self.eager:
            for _ in range(batches):
                self._cold()
                start.record(stream)
                for i in range(n):
                    fn(i)
                end.record(stream)
                torch.cuda.synchronize()
                times.append(start.elapsed_time(end) / n)
        else:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(n):
                    fn(i)
            # untimed replays first, at least 3 and 50 ms of work: the device idles while the
            # graph is captured, and the first replays after that run slower
            t_warm = 0.0
            for r in range(100):
                start.record(stream)
                graph.replay()
                end.record(stream)
                torch.cuda.synchronize()
                t_warm += start.elapsed_time(end)
                if r >= 2 and t_warm >= 50.0:
                    break
            for _ in range(batches):
                self._cold()
                start.record(stream)
                graph.replay()
                end.record(stream)
                torch.cuda.synchronize()
                times.append(start.elapsed_time(end) / n)
            del graph
        times.sort()
        return times[len(times) // 2], times[0], times[-1]

    def _cold(self):
        if self.flush is not None:
            self.flush()
        self.torch.cuda.synchronize()


def stream_read_gbs(torch, tq, log):
    """Streaming-read bandwidth of the device: the library's plain read kernel over three
    512 MiB buffers in turn (more than the 256 MB last-level cache), best of 5 rounds."""
    bufs = [torch.ones(512 << 20, dtype=torch.uint8, device="cuda") for _ in range(3)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for b in bufs:
        tq.probe_stream_read(b, sink)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    best = float("inf")
    for _ in range(5):
        start.record(stream)
        for b in bufs:
            tq.probe_stream_read(b, sink)
        end.record(stream)
        torch.cuda.synchronize()
        best = min(best, start.elapsed_time(end))
    gbs = 3 * (512 << 20) / (best * 1e-3) / 1e9
    log(f"[bench] streaming-read probe: {gbs:.0f} GB/s")
    del bufs
    return gbs


def cache_flush(torch, tq):
    """A callable that streams 1 GiB of unrelated data through the read path (the library's
    plain read kernel): more than the 256 MB Infinity Cache plus the 8 L2s, so whatever the
    benchmark read before is evicted and the next timed batch reads its inputs from HBM."""
    buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def flush():
        tq.probe_stream_read(buf, sink)

    return flush


def bench_decode(args, w, tau, signs, dev, tq, inputs, torch, np, log):
    batch, hq, hkv, ctx = w.batch, w.n_q_heads, w.n_kv_heads, w.ctx
    bk, bv = w.bits_k, w.bits_v
    cap = ctx
    per_copy = tq.code_bytes(D, bk, batch, hkv, cap) + tq.code_bytes(D, bv, batch, hkv, cap) + 4 * batch * hkv * cap
    copies = args.copies or min(MAX_COPIES, max(1, math.ceil(600e6 / per_copy)))
    log(f"[bench] workload={w.name} tau={tau} copies={copies} cache/copy={per_copy / 1e6:.1f} MB "
        f"({'eager launches' if args.eager else 'HIP graph replay'})")
    g = inputs.generate(w, device=dev)
    k_all, v_all, q = g["k"], g["v"], g["q"].contiguous()
    caches = []
    for c in range(copies):
        kc = tq.PackedCache(batch, hkv, cap, bk, tq.LAYOUT_ROWS, signs, device=dev)
        vc = tq.PackedCache(batch, hkv, cap, bv, tq.LAYOUT_GROUP8, signs, device=dev)
        tq.quantize_append(kc, k_all[:, : ctx - 1].contiguous(), 0)
        tq.quantize_append(vc, v_all[:, : ctx - 1].contiguous(), 0)
        caches.append((kc, vc))
    k_new = k_all[:, ctx - 1:ctx].contiguous()
    v_new = v_all[:, ctx - 1:ctx].contiguous()
    host_k = k_all[:1].cpu() if not args.no_cpu_baseline else None
    host_v = v_all[:1].cpu() if not args.no_cpu_baseline else None
    prefill = prefill_quantize_stats(args, w, caches, k_all, v_all, tq, torch, log)
    del k_all, v_all, g
    bufs = tq.DecodeBuffers(batch, hq, hkv, ctx, tau, device=dev, want_lse=True)
    scale = 1.0 / math.sqrt(D)
    torch.cuda.synchronize()

    def append(i):
        kc, vc = caches[i % copies]
        tq.quantize_append_kv(kc, vc, k_new, v_new, ctx - 1)

    def decode_only(i):
        kc, vc = caches[i % copies]
        tq.decode_attn(kc, vc, q, ctx, scale, tau=tau, buffers=bufs)

    # matrix-core widths: the step is one call that appends inside the attention: dense, one
    # launch; Sparse V, the key pass (which writes the new token first) and the value pass
    fused_step = bk in (3, 4) and bv == 2 and w.group <= 8
    dense_single = fused_step and tau == 0.0

    def append_and_decode(i):
        kc, vc = caches[i % copies]
        tq.decode_attn_append(kc, vc, k_new, v_new, q, ctx, scale, buffers=bufs, tau=tau)

    def two_launches(i):
        append(i)
        decode_only(i)

    step = append_and_decode if fused_step else two_launches
    timer = Timer(torch, args.eager, cache_flush(torch, tq))
    steps = args.steps
    ms_per_step = timer.per_iteration_ms(step, steps, args.warmup)
    kv_tokens = batch * ctx
    value = kv_tokens / (ms_per_step / 1e3)
    n_rep = max(args.steps, 2 * copies)
    # the roofline launches: the step's call when fused (dense: one launch; Sparse V: the key pass
    # with the append and the value pass), else the decode call
    ms_k, ms_k_min, ms_k_max = timer.per_iteration_stats(step if fused_step else decode_only, n_rep, 2, batches=5)
    ms_d = timer.per_iteration_ms(decode_only, n_rep, 2) if fused_step else ms_k
    ms_a = timer.per_iteration_ms(append, n_rep, 2)
    # steady state of a decode loop over a resident cache: 32 back-to-back steps on one copy,
    # caches warm (a small context stays in the L2s and the 256 MB last-level cache)
    ms_ss = Timer(torch, args.eager, None).per_iteration_ms(lambda i: step(0), STEADY_STEPS, 2)
    nbytes = decode_bytes(w, bk, bv, hkv, batch, ctx)
    sparse_info = None
    if dense_single:
        nbytes += append_bytes(w, bk, bv, hkv, batch)
    elif tau > 0:
        # Sparse V: the keys of every token plus the value rows that some head of the group
        # keeps (p = exp(s - LSE) >= tau), counted from this call's own scores and LSE
        kept, kept_tiles, n_tiles = sparse_kept_rows(tq, torch, caches[0], q, ctx, scale, tau, batch, hq, hkv, dev)
        k_bytes = batch * hkv * ctx * (D * bk // 8 + 2)
        nbytes = k_bytes + kept * (D * bv // 8 + 2)
        if fused_step:
            nbytes += append_bytes(w, bk, bv, hkv, batch)
        sparse_info = {"kept_value_rows": kept, "kept_value_rows_frac": kept / (batch * hkv * ctx),
                       "tiles_with_kept_row_frac": kept_tiles / n_tiles, "key_bytes": k_bytes,
                       "dense_bytes": decode_bytes(w, bk, bv, hkv, batch, ctx)}
        log(f"[bench] Sparse V: {kept} of {batch * hkv * ctx} value rows kept by a group "
            f"({100 * kept / (batch * hkv * ctx):.2f}%), {100 * kept_tiles / n_tiles:.1f}% of 64-token tiles hold one")
    achieved = nbytes / (ms_k / 1e3) / 1e9
    how = 'one fused launch' if dense_single else 'key pass with the append + value pass' if fused_step else 'append + decode'
    log(f"[bench] step {ms_per_step * 1e3:.1f} us ({how}), "
        f"decode-only call {ms_d * 1e3:.1f} us, standalone append (K+V) {ms_a * 1e3:.1f} us, "
        f"roofline launch {ms_k * 1e3:.1f} us = {achieved:.0f} GB/s algorithmic")
    result = {
        "metric": METRIC, "value": value, "unit": "KV-tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16+f32",
        "data": "synthetic (seeded; shapes and value distributions of the workload)",
        "config": {"workload": w.name, "batch": batch, "n_q_heads": hq, "n_kv_heads": hkv, "d": D,
                   "ctx": ctx, "bits_k": bk, "bits_v": bv, "sparse_v_tau": tau,
                   "step": ("append 1 token (K,V) + decode attention, one fused launch" if dense_single
                            else "append 1 token (K,V) in Sparse V's key pass, then the masked value pass"
                            if fused_step else "append 1 token (K,V) + decode attention"), "cache_copies": copies,
                   "timing": "eager" if args.eager else "hip graph replay"},
        "decode_call_us": ms_d * 1e3,
        "append_kv_us": ms_a * 1e3,
        "steady_state": {"us_per_step": ms_ss * 1e3, "kv_tokens_per_s": kv_tokens / (ms_ss / 1e3),
                         "note": f"{STEADY_STEPS} back-to-back steps on one cache copy, caches warm"},
        "prefill_quantize": prefill,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": f"{DECODE_KERNEL} (append + attend instance)" if dense_single
                     else f"{DECODE_KERNEL}: Sparse V's key pass (with the append) + masked value pass" if fused_step
                     else "decode attention call (Sparse V: key pass + masked value pass)",
                     "bytes_per_launch": nbytes, "launch_us": ms_k * 1e3,
                     "launch_us_min_max": [ms_k_min * 1e3, ms_k_max * 1e3]},
        "_kernel": "decode" if dense_single else "decode_sparse",
    }
    if sparse_info is not None:
        result["roofline"]["bytes_note"] = ("algorithmic bytes: every key (codes + norm) plus the value rows "
                                            "kept by the union of the group's heads"
                                            + (", plus the appended token's input and codes" if fused_step else ""))
        result["sparse_v"] = sparse_info
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_decode(w, tau, caches[0], host_k, host_v, q, signs, np, torch, log)
    return result


def prefill_quantize_stats(args, w, caches, k_all, v_all, tq, torch, log):
    """The whole context of every sequence quantized into the caches in one K-and-V call
    (tq_quantize_append_kv at position 0): HBM-cold, rotated over the cache copies."""
    batch, hkv, ctx, bk, bv = w.batch, w.n_kv_heads, w.ctx, w.bits_k, w.bits_v
    k_all, v_all = k_all.contiguous(), v_all.contiguous()

    def fill(i):
        kc, vc = caches[i % len(caches)]
        tq.quantize_append_kv(kc, vc, k_all, v_all, 0)

    timer = Timer(torch, args.eager, cache_flush(torch, tq))
    ms = timer.per_iteration_ms(fill, max(4, 2 * len(caches)), 1)
    vectors = 2 * batch * ctx * hkv
    nbytes = vectors * D * k_all.element_size() + batch * ctx * hkv * ((D * bk // 8 + 2) + (D * bv // 8 + 2))
    log(f"[bench] prefill quantize of the whole cache: {ms * 1e3:.1f} us for {vectors} vectors "
        f"({nbytes / (ms / 1e3) / 1e9:.0f} GB/s)")
    return {"us": ms * 1e3, "tokens_per_s": batch * ctx / (ms / 1e3), "vectors_per_s": vectors / (ms / 1e3),
            "vectors": vectors, "bytes": nbytes, "gbs": nbytes / (ms / 1e3) / 1e9,
            "frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
            "note": "every sequence's whole context, K and V of all kv heads, one tq_quantize_append_kv call"}


def sparse_kept_rows(tq, torch, cache_pair, q, ctx, scale, tau, batch, hq, hkv, dev):
    """Value rows a Sparse-V call must read: (batch, kv head, position) triples that some
    query head of the group keeps (p = exp(s - LSE) >= tau), and the 64-token tiles that
    hold at least one of them, from one call's score and LSE outputs (measurement only)."""
    kc, vc = cache_pair
    b2 = tq.DecodeBuffers(batch, hq, hkv, ctx, tau, device=dev, want_scores=True)
    tq.decode_attn(kc, vc, q, ctx, scale, tau=tau, buffers=b2)
    torch.cuda.synchronize()
    g = hq // hkv
    keep = (torch.exp(b2.scores - b2.lse[..., None]) >= tau).view(batch, hkv, g, ctx).any(dim=2)
    n_tiles = batch * hkv * ((ctx + 63) // 64)
    pad = (-ctx) % 64
    tiles = torch.nn.functional.pad(keep, (0, pad)).view(batch, hkv, -1, 64).any(dim=-1)
    kept, kept_tiles = int(keep.sum()), int(tiles.sum())
    del b2
    return kept, kept_tiles, n_tiles


def cpu_baseline_decode(w, tau, cache_pair, host_k, host_v, q, signs, np, torch, log):
    """The CPU oracle on a bounded sample: batch element 0, every kv head, the whole context:
    quantize + pack the appended token, then unpack, dequantize and attend."""
    from oracle import tq_oracle as o

    kc, vc = cache_pair
    ctx, hkv, g = w.ctx, w.n_kv_heads, w.group
    s64 = signs.cpu().numpy().astype(np.float64)
    tabk = o.make_codebook(D, w.bits_k)[:2]
    tabv = o.make_codebook(D, w.bits_v)[:2]
    raw_k = [kc.plane_codes(0, h).cpu().numpy() for h in range(hkv)]
    raw_v = [vc.plane_codes(0, h).cpu().numpy() for h in range(hkv)]
    nk = [kc.plane_norms(0, h).cpu().numpy() for h in range(hkv)]
    nv = [vc.plane_norms(0, h).cpu().numpy() for h in range(hkv)]
    q64 = q[:1].double().cpu().numpy()
    xk = host_k[0, ctx - 1].double().numpy()
    xv = host_v[0, ctx - 1].double().numpy()
    reps, t0 = 0, time.perf_counter()
    while True:
        o.quantize(xk, s64, *tabk)
        o.quantize(xv, s64, *tabv)
        kh = np.stack([o.dequantize(o.unpack(raw_k[h], ctx, D, w.bits_k, 0), nk[h], s64, tabk[0])
                       for h in range(hkv)])[None]
        vh = np.stack([o.dequantize(o.unpack(raw_v[h], ctx, D, w.bits_v, 1), nv[h], s64, tabv[0])
                       for h in range(hkv)])[None]
        o.decode_attention(q64, kh, vh, 1.0 / math.sqrt(D), tau=tau)
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or reps >= 50:
            break
    value = reps * ctx / el
    log(f"[bench] cpu oracle: {reps} sample steps in {el:.1f} s")
    return with_cpu_context({"value": value, "unit": "KV-tokens/s", "cores": cpu_cores(), "kind": "oracle",
            "sample": f"batch element 0 of {w.batch}, all {hkv} kv heads / {hkv * g} query heads, "
                      f"{ctx} tokens: quantize+pack the appended token, unpack+dequantize+attend; "
                      f"{reps} repetitions"})


class _GatheredPlanes:
    """Batch element 0 of a paged cache as the planes the CPU baseline reads (host-side
    gather through the block table; not timed)."""

    def __init__(self, cache, table_row, torch):
        self.cache, self.row, self.torch = cache, [int(p) for p in table_row], torch

    def plane_codes(self, b, h):
        return self.torch.cat([self.cache.page_codes(p, h) for p in self.row])

    def plane_norms(self, b, h):
        return self.torch.cat([self.cache.page_norms(p, h) for p in self.row])


def bench_paged(args, w, signs, dev, tq, inputs, torch, np, log):
    """Decode over paged caches: the batched long-context shape with each sequence's positions
    in pages of w.page_tokens scattered over the pool in a seeded random order.  A step
    appends one token per sequence (K and V) through the block table, then paged decode."""
    batch, hq, hkv, ctx, P = w.batch, w.n_q_heads, w.n_kv_heads, w.ctx, w.page_tokens
    bk, bv = w.bits_k, w.bits_v
    max_pages = (ctx + P - 1) // P
    n_pages = batch * max_pages
    per_copy = tq.code_bytes(D, bk, n_pages, hkv, P) + tq.code_bytes(D, bv, n_pages, hkv, P) + 4 * n_pages * hkv * P
    copies = args.copies or min(MAX_COPIES, max(1, math.ceil(600e6 / per_copy)))
    log(f"[bench] workload={w.name} pages of {P} tokens, {n_pages} pages, copies={copies} "
        f"cache/copy={per_copy / 1e6:.1f} MB ({'eager launches' if args.eager else 'HIP graph replay'})")
    g = inputs.generate(w, device=dev)
    k_all, v_all, q = g["k"], g["v"], g["q"].contiguous()
    rng = np.random.default_rng(w.seed)
    caches = []
    zeros = torch.zeros(batch, dtype=torch.int32, device=dev)
    for c in range(copies):
        table = torch.tensor(rng.permutation(n_pages).reshape(batch, max_pages), dtype=torch.int32, device=dev)
        kc = tq.PagedCache(batch, hkv, P, n_pages, max_pages, bk, tq.LAYOUT_ROWS, signs, block_table=table, device=dev)
        vc = tq.PagedCache(batch, hkv, P, n_pages, max_pages, bv, tq.LAYOUT_GROUP8, kc.signs, block_table=table,
                           device=dev)
        tq.paged_quantize_append_kv(kc, vc, k_all[:, : ctx - 1].contiguous(), v_all[:, : ctx - 1].contiguous(), zeros)
        caches.append((kc, vc))
    k_new = k_all[:, ctx - 1:ctx].contiguous()
    v_new = v_all[:, ctx - 1:ctx].contiguous()
    host_k = k_all[:1].cpu() if not args.no_cpu_baseline else None
    host_v = v_all[:1].cpu() if not args.no_cpu_baseline else None
    del k_all, v_all, g
    start = torch.full((batch,), ctx - 1, dtype=torch.int32, device=dev)
    lens = torch.full((batch,), ctx, dtype=torch.int32, device=dev)
    bufs = tq.PagedDecodeBuffers(batch, hq, hkv, ctx, device=dev)
    scale = 1.0 / math.sqrt(D)
    torch.cuda.synchronize()

    def append(i):
        kc, vc = caches[i % copies]
        tq.paged_quantize_append_kv(kc, vc, k_new, v_new, start)

    def decode_only(i):
        kc, vc = caches[i % copies]
        tq.paged_decode_attn(kc, vc, q, lens, ctx, scale, buffers=bufs)

    def step(i):  # one launch: the fused kernel writes the new token into its page, then attends
        kc, vc = caches[i % copies]
        tq.paged_decode_attn_append(kc, vc, k_new, v_new, q, lens, ctx, scale, buffers=bufs)

    timer = Timer(torch, args.eager, cache_flush(torch, tq))
    ms_per_step = timer.per_iteration_ms(step, args.steps, args.warmup)
    value = batch * ctx / (ms_per_step / 1e3)
    n_rep = max(args.steps, 2 * copies)
    ms_k, ms_k_min, ms_k_max = timer.per_iteration_stats(step, n_rep, 2, batches=5)
    ms_d = timer.per_iteration_ms(decode_only, n_rep, 2)
    ms_a = timer.per_iteration_ms(append, n_rep, 2)
    nbytes = decode_bytes(w, bk, bv, hkv, batch, ctx) + append_bytes(w, bk, bv, hkv, batch)
    achieved = nbytes / (ms_k / 1e3) / 1e9
    log(f"[bench] step {ms_per_step * 1e3:.1f} us (one fused paged launch), paged decode-only call "
        f"{ms_d * 1e3:.1f} us, paged append (K+V) alone {ms_a * 1e3:.1f} us, roofline launch {ms_k * 1e3:.1f} us "
        f"= {achieved:.0f} GB/s algorithmic")
    result = {
        "metric": METRIC, "value": value, "unit": "KV-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16+f32",
        "data": "synthetic (seeded; shapes and value distributions of the workload; pages in seeded random order)",
        "config": {"workload": w.name, "batch": batch, "n_q_heads": hq, "n_kv_heads": hkv, "d": D,
                   "ctx": ctx, "bits_k": bk, "bits_v": bv, "sparse_v_tau": 0.0, "page_tokens": P,
                   "step": "append 1 token (K,V) + decode attention over paged caches, one fused launch",
                   "cache_copies": copies,
                   "timing": "eager" if args.eager else "hip graph replay"},
        "decode_call_us": ms_d * 1e3,
        "append_kv_us": ms_a * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": f"{DECODE_KERNEL} (paged append + attend instance)",
                     "bytes_per_launch": nbytes, "launch_us": ms_k * 1e3,
                     "launch_us_min_max": [ms_k_min * 1e3, ms_k_max * 1e3]},
        "_kernel": "decode",
    }
    if not args.no_cpu_baseline:
        kc, vc = caches[0]
        row = kc.block_table[0].cpu().numpy()
        gathered = (_GatheredPlanes(kc, row, torch), _GatheredPlanes(vc, row, torch))
        result["cpu_baseline"] = cpu_baseline_decode(w, 0.0, gathered, host_k, host_v, q, signs, np, torch, log)
    return result


def bench_qjl(args, w, signs, dev, tq, inputs, torch, np, log):
    """QJL keys: a step appends one token per (batch, kv head), the key with its sign sketch and
    the value as usual, then decode attention with QJL-corrected scores (one launch of the fused
    kernel: the query's sketch and the sign products on matrix cores)."""
    batch, hq, hkv, ctx = w.batch, w.n_q_heads, w.n_kv_heads, w.ctx
    bk, bv, m = w.bits_k, w.bits_v, w.extra["qjl_m"]
    k_row = D * bk // 8 + 2 + m // 8 + 2       # codes + norm + sign bits + residual norm
    v_row = D * bv // 8 + 2
    per_copy = batch * hkv * ctx * (k_row + v_row)
    copies = args.copies or min(MAX_COPIES, max(1, math.ceil(600e6 / per_copy)))
    log(f"[bench] workload={w.name} QJL keys ({bk}-bit codes + {m} sign bits) copies={copies} "
        f"cache/copy={per_copy / 1e6:.1f} MB ({'eager launches' if args.eager else 'HIP graph replay'})")
    g = inputs.generate(w, device=dev)
    k_all, v_all, q = g["k"], g["v"], g["q"].contiguous()
    proj = inputs.qjl_projection(m)
    caches = []
    for c in range(copies):
        kc = tq.PackedCache(batch, hkv, ctx, bk, tq.LAYOUT_ROWS, signs, device=dev)
        vc = tq.PackedCache(batch, hkv, ctx, bv, tq.LAYOUT_GROUP8, signs, device=dev)
        sk = tq.QjlSketch(kc, proj, device=dev)
        tq.qjl_quantize_append(kc, sk, k_all[:, : ctx - 1].contiguous(), 0)
        tq.quantize_append(vc, v_all[:, : ctx - 1].contiguous(), 0)
        caches.append((kc, sk, vc))
    k_new = k_all[:, ctx - 1:ctx].contiguous()
    v_new = v_all[:, ctx - 1:ctx].contiguous()
    host_k = k_all[:1, ctx - 1].cpu() if not args.no_cpu_baseline else None
    del k_all, v_all, g
    bufs = tq.DecodeBuffers(batch, hq, hkv, ctx, 0.0, device=dev)
    scale = 1.0 / math.sqrt(D)
    torch.cuda.synchronize()

    def append(i):  # keys (codes and sketch) and values in one launch
        kc, sk, vc = caches[i % copies]
        tq.qjl_quantize_append_kv(kc, sk, vc, k_new, v_new, ctx - 1)

    def attend(i):
        kc, sk, vc = caches[i % copies]
        tq.qjl_decode_attn(kc, sk, vc, q, ctx, scale, buffers=bufs)

    def step(i):
        append(i)
        attend(i)

    timer = Timer(torch, args.eager, cache_flush(torch, tq))
    ms_per_step = timer.per_iteration_ms(step, args.steps, args.warmup)
    n_rep = max(args.steps, 2 * copies)
    ms_k, ms_k_min, ms_k_max = timer.per_iteration_stats(attend, n_rep, 2, batches=5)
    ms_a = timer.per_iteration_ms(append, n_rep, 2)
    nbytes = batch * hkv * ctx * (k_row + v_row)
    achieved = nbytes / (ms_k / 1e3) / 1e9
    log(f"[bench] step {ms_per_step * 1e3:.1f} us, QJL decode call {ms_k * 1e3:.1f} us = {achieved:.0f} GB/s, "
        f"append (QJL key + value) {ms_a * 1e3:.1f} us")
    result = {
        "metric": METRIC, "value": batch * ctx / (ms_per_step / 1e3), "unit": "KV-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16+f32",
        "data": "synthetic (seeded; shapes and value distributions of the workload; seeded Gaussian sketch)",
        "config": {"workload": w.name, "batch": batch, "n_q_heads": hq, "n_kv_heads": hkv, "d": D, "ctx": ctx,
                   "bits_k": bk, "qjl_sketch_rows": m, "bits_v": bv,
                   "step": "QJL key + value append (1 token, one launch) + decode attention with QJL-corrected "
                           "scores",
                   "cache_copies": copies, "timing": "eager" if args.eager else "hip graph replay"},
        "decode_call_us": ms_k * 1e3, "append_us": ms_a * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "decode_fused_kernel (QJL: sign products against the query's sketch)",
                     "bytes_per_launch": nbytes, "launch_us": ms_k * 1e3,
                     "launch_us_min_max": [ms_k_min * 1e3, ms_k_max * 1e3],
                     "bytes_note": f"per (token, kv head): key {k_row} B (codes, norm, sign bits, residual norm), "
                                   f"value {v_row} B"},
        "_kernel": "decode_qjl",
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_qjl(w, caches[0], host_k, q, signs, proj, np, log)
    return result


def cpu_baseline_qjl(w, cache, host_k, q, signs, proj, np, log):
    """The CPU oracle on a bounded sample: batch element 0, every kv head, the whole context:
    QJL-quantize the appended key, then unpack the codes and sign bits, form the effective keys
    and attend."""
    from oracle import tq_oracle as o

    kc, sk, vc = cache
    ctx, hkv, g, m = w.ctx, w.n_kv_heads, w.group, w.extra["qjl_m"]
    s64 = signs.cpu().numpy().astype(np.float64)
    p64 = proj.numpy().astype(np.float64)
    tabk = o.make_codebook(D, w.bits_k)[:2]
    tabv = o.make_codebook(D, w.bits_v)[:2]
    raw_k = [kc.plane_codes(0, h).cpu().numpy() for h in range(hkv)]
    raw_s = [sk.plane_bits(0, h).cpu().numpy() for h in range(hkv)]
    raw_v = [vc.plane_codes(0, h).cpu().numpy() for h in range(hkv)]
    nk = [kc.plane_norms(0, h).cpu().numpy() for h in range(hkv)]
    rk = [sk.plane_res_norms(0, h).cpu().numpy() for h in range(hkv)]
    nv = [vc.plane_norms(0, h).cpu().numpy() for h in range(hkv)]
    q64 = q[:1].double().cpu().numpy()
    xk = host_k[0].double().numpy()
    reps, t0 = 0, time.perf_counter()
    while True:
        o.qjl_quantize(xk, s64, *tabk, p64)
        kh = np.stack([o.qjl_dequantize(o.unpack(raw_k[h], ctx, D, w.bits_k, 0), nk[h],
                                        o.unpack(raw_s[h], ctx, m, 1, 0).astype(bool), rk[h], s64, tabk[0], p64)
                       for h in range(hkv)])[None]
        vh = np.stack([o.dequantize(o.unpack(raw_v[h], ctx, D, w.bits_v, 1), nv[h], s64, tabv[0])
                       for h in range(hkv)])[None]
        o.decode_attention(q64, kh, vh, 1.0 / math.sqrt(D))
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or reps >= 50:
            break
    log(f"[bench] cpu oracle: {reps} sample steps in {el:.1f} s")
    return with_cpu_context({"value": reps * ctx / el, "unit": "KV-tokens/s", "cores": cpu_cores(), "kind": "oracle",
                             "sample": f"batch element 0 of {w.batch}, all {hkv} kv heads / {hkv * g} query heads, "
                                       f"{ctx} tokens: QJL-quantize the appended key, unpack codes and sign bits, "
                                       f"effective keys, attend; {reps} repetitions"})


def bench_search(args, spec, signs, dev, tq, inputs, torch, np, log):
    """Inner-product nearest-neighbour search: a step is one tq_ip_search call for the
    queries over the whole quantized database (scores with block top-k, then the final top-k)."""
    n, nq, k, bits = spec["n"], spec["n_queries"], spec["top_k"], spec["bits"]
    per_copy = tq.code_bytes(D, bits, 1, 1, n) + 2 * n
    copies = args.copies or min(MAX_COPIES, max(1, math.ceil(600e6 / per_copy)))
    log(f"[bench] search n={n} queries={nq} top_k={k} bits={bits} copies={copies} db/copy={per_copy / 1e6:.1f} MB "
        f"({'eager launches' if args.eager else 'HIP graph replay'})")
    g = inputs.generate_search(spec, device=dev)
    x, q = g["x"], g["q"].contiguous()
    dbs = []
    for c in range(copies):
        db = tq.PackedCache(1, 1, n, bits, tq.LAYOUT_ROWS, signs, device=dev)
        tq.quantize_append(db, x[None, :, None, :].contiguous(), 0)
        dbs.append(db)
    bufs = tq.SearchBuffers(nq, n, k, device=dev)
    torch.cuda.synchronize()

    def step(i):
        tq.ip_search(dbs[i % copies], q, n, k, buffers=bufs)

    timer = Timer(torch, args.eager, cache_flush(torch, tq))
    ms_per_step = timer.per_iteration_ms(step, args.steps, args.warmup)
    ms_k, ms_k_min, ms_k_max = timer.per_iteration_stats(step, max(args.steps, 2 * copies), 2, batches=5)
    nbytes = per_copy  # the packed database, read once per call
    achieved = nbytes / (ms_k / 1e3) / 1e9
    # recall@k against exact inner-product search over the unquantized vectors (measurement only)
    step(0)
    exact = torch.topk(q.float() @ x.float().T, k, dim=1).indices
    got = bufs.idx.long()
    recall = float(sum(len(set(got[j].tolist()) & set(exact[j].tolist())) for j in range(nq)) / (nq * k))
    log(f"[bench] step {ms_per_step * 1e3:.1f} us ({nq} queries over {n} vectors), {achieved:.0f} GB/s of packed "
        f"database, recall@{k} vs exact search {recall:.3f}")
    result = {
        "metric": METRIC, "value": nq / (ms_per_step / 1e3), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16+f32",
        "data": "synthetic (seeded clustered vectors standing in for a search benchmark)",
        "config": {"workload": "search1m", "n_vectors": n, "n_queries": nq, "top_k": k, "bits": bits, "d": D,
                   "step": "inner-product search: scores + top-k per query", "cache_copies": copies,
                   "timing": "eager" if args.eager else "hip graph replay"},
        "recall_at_k_vs_exact": recall,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "search call (ip_score_kernel, topk_final_kernel)",
                     "bytes_per_launch": nbytes, "launch_us": ms_k * 1e3,
                     "launch_us_min_max": [ms_k_min * 1e3, ms_k_max * 1e3]},
        "_kernel": "ip_search",
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_search(spec, dbs[0], q, signs, np, torch, log)
    return result


def cpu_baseline_search(spec, db, q, signs, np, torch, log):
    """The CPU oracle on a bounded sample: one query over the first 65536 database vectors,
    scaled to queries/s over the whole database (the work is linear in its size)."""
    from oracle import tq_oracle as o

    n, bits, sample = spec["n"], spec["bits"], 65536
    s64 = signs.cpu().numpy().astype(np.float64)
    c, _, _ = o.make_codebook(D, bits)[:3]
    codes = o.unpack(db.plane_codes(0, 0)[: sample * 16 * bits].cpu().numpy(), sample, D, bits, 0)
    n16 = db.plane_norms(0, 0)[:sample].cpu().numpy().astype(np.float16)
    q64 = q[:1].double().cpu().numpy()
    reps, t0 = 0, time.perf_counter()
    while True:
        o.ip_search(q64, codes, n16, s64, c, spec["top_k"])
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or reps >= 1000:  # about 10 s of CPU work
            break
    value = reps * sample / n / el
    log(f"[bench] cpu oracle: {reps} sample searches in {el:.1f} s")
    return with_cpu_context({"value": value, "unit": "queries/s", "cores": cpu_cores(), "kind": "oracle",
            "sample": f"1 query over the first {sample} of {n} vectors, scaled to the whole database; "
                      f"{reps} repetitions"})


def bench_multi_query(args, w, signs, dev, tq, inputs, torch, np, log):
    """Speculative verification: a step appends n_q tokens (K and V of every kv head) at the
    end of each sequence and attends from those n_q positions, causally, over the cache."""
    batch, hq, hkv, ctx, n_q = w.batch, w.n_q_heads, w.n_kv_heads, w.ctx, w.n_q
    bk, bv = w.bits_k, w.bits_v
    per_copy = tq.code_bytes(D, bk, batch, hkv, ctx) + tq.code_bytes(D, bv, batch, hkv, ctx) + 4 * batch * hkv * ctx
    copies = args.copies or min(MAX_COPIES, max(1, math.ceil(600e6 / per_copy)))
    rows = n_q * w.group
    vgroups = (rows + 7) // 8
    log(f"[bench] workload={w.name} n_q={n_q} ({rows} query rows per kv head in {vgroups} groups) "
        f"copies={copies} cache/copy={per_copy / 1e6:.1f} MB ({'eager launches' if args.eager else 'HIP graph replay'})")
    g = inputs.generate(w, device=dev)
    k_all, v_all, q = g["k"], g["v"], g["q"].contiguous()
    caches = []
    for c in range(copies):
        kc = tq.PackedCache(batch, hkv, ctx, bk, tq.LAYOUT_ROWS, signs, device=dev)
        vc = tq.PackedCache(batch, hkv, ctx, bv, tq.LAYOUT_GROUP8, signs, device=dev)
        tq.quantize_append(kc, k_all[:, : ctx - n_q].contiguous(), 0)
        tq.quantize_append(vc, v_all[:, : ctx - n_q].contiguous(), 0)
        caches.append((kc, vc))
    k_new = k_all[:, ctx - n_q:].contiguous()
    v_new = v_all[:, ctx - n_q:].contiguous()
    host_k = k_all[:1].cpu() if not args.no_cpu_baseline else None
    host_v = v_all[:1].cpu() if not args.no_cpu_baseline else None
    del k_all, v_all, g
    bufs = tq.MultiQueryBuffers(batch, n_q, hq, hkv, ctx, device=dev)
    scale = 1.0 / math.sqrt(D)
    for kc, vc in caches:
        tq.quantize_append_kv(kc, vc, k_new, v_new, ctx - n_q)
    torch.cuda.synchronize()

    def append(i):
        kc, vc = caches[i % copies]
        tq.quantize_append_kv(kc, vc, k_new, v_new, ctx - n_q)

    def attend(i):
        kc, vc = caches[i % copies]
        tq.decode_attn_multi(kc, vc, q, ctx, scale, buffers=bufs)

    # up to 8 positions (outside the prefill mode): one launch writes the tokens, then attends
    one_launch = n_q <= 8 and vgroups < 8

    def step(i):
        if one_launch:
            kc, vc = caches[i % copies]
            tq.decode_attn_multi_append(kc, vc, k_new, v_new, q, ctx, scale, buffers=bufs)
            return
        append(i)
        attend(i)

    timer = Timer(torch, args.eager, cache_flush(torch, tq))
    steps = args.steps
    ms_per_step = timer.per_iteration_ms(step, steps, args.warmup)
    value = batch * ctx / (ms_per_step / 1e3)
    # the roofline launch: the attention call alone (the append's few kilobytes aside)
    ms_k, ms_k_min, ms_k_max = timer.per_iteration_stats(attend, max(args.steps, 2 * copies), 2, batches=5)
    ms_a = timer.per_iteration_ms(append, max(args.steps, 2 * copies), 2)
    nbytes = decode_bytes(w, bk, bv, hkv, batch, ctx)
    achieved = nbytes / (ms_k / 1e3) / 1e9
    # causal (query row, visible token) pairs: QK and PV take 2 d multiply-adds per pair
    pairs = batch * hq * sum(max(ctx - n_q + i + 1, 0) for i in range(n_q))
    flops = 4 * D * pairs
    tflops = flops / (ms_k / 1e3) / 1e12
    prefill = vgroups >= 8
    log(f"[bench] step {ms_per_step * 1e3:.1f} us, attention call {ms_k * 1e3:.1f} us "
        f"({n_q} positions), append {n_q} tokens (K+V) {ms_a * 1e3:.1f} us, {achieved:.0f} GB/s algorithmic, "
        f"{tflops:.1f} TFLOP/s algorithmic")
    result = {
        "metric": METRIC, "value": value, "unit": "KV-tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16+f32",
        "data": "synthetic (seeded; shapes and value distributions of the workload)",
        "config": {"workload": w.name, "batch": batch, "n_q_heads": hq, "n_kv_heads": hkv, "d": D,
                   "ctx": ctx, "bits_k": bk, "bits_v": bv, "n_q": n_q, "row_groups": vgroups,
                   "step": (f"append {n_q} tokens (K,V) and causal attention of the {n_q} positions, one launch"
                            if one_launch else
                            f"append {n_q} tokens (K,V) + causal attention of the {n_q} positions"),
                   "cache_copies": copies, "timing": "eager" if args.eager else "hip graph replay"},
        "attention_call_us": ms_k * 1e3,
        "attention_call_us_min_max": [ms_k_min * 1e3, ms_k_max * 1e3],
        "query_positions_per_s": batch * n_q / (ms_per_step / 1e3),
        "append_kv_us": ms_a * 1e3,
        "roofline": ({"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": tflops / MFMA_F16_PEAK_TFLOPS, "traffic": None,
                      "kernel": DECODE_KERNEL + " (prefill: 8 row groups per workgroup)",
                      "flops_per_launch": flops, "bytes_per_launch": nbytes, "launch_us": ms_k * 1e3,
                      "hbm_gbs": achieved,
                      "note": f"algorithmic flops: 4 d per causal (query row, token) pair; the products run on "
                              f"fp16 matrix cores with hi/lo operand splits (about 4x the algorithmic products); "
                              f"the cache is read from memory once per workgroup of 8 row groups "
                              f"({(vgroups + 7) // 8} per kv head here)"}
                     if prefill else
                     {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": DECODE_KERNEL,
                      "bytes_per_launch": nbytes, "launch_us": ms_k * 1e3, "tflops": tflops,
                      "note": f"algorithmic bytes read the cache once; the kernel reads it once per "
                              f"group of up to 8 query rows ({vgroups} here)"}),
        "_kernel": "decode_multi",
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_multi(w, caches[0], host_k, host_v, q, signs, np, torch, log)
    return result


def cpu_baseline_multi(w, cache_pair, host_k, host_v, q, signs, np, torch, log):
    """The CPU oracle on a bounded sample: batch element 0, every kv head, the whole context:
    quantize + pack the n_q appended tokens, then unpack, dequantize and attend causally."""
    from oracle import tq_oracle as o

    kc, vc = cache_pair
    ctx, hkv, g, n_q = w.ctx, w.n_kv_heads, w.group, w.n_q
    s64 = signs.cpu().numpy().astype(np.float64)
    tabk = o.make_codebook(D, w.bits_k)[:2]
    tabv = o.make_codebook(D, w.bits_v)[:2]
    raw_k = [kc.plane_codes(0, h).cpu().numpy() for h in range(hkv)]
    raw_v = [vc.plane_codes(0, h).cpu().numpy() for h in range(hkv)]
    nk = [kc.plane_norms(0, h).cpu().numpy() for h in range(hkv)]
    nv = [vc.plane_norms(0, h).cpu().numpy() for h in range(hkv)]
    q64 = q[:1].double().cpu().numpy()
    xk = host_k[0, ctx - n_q:].double().numpy()
    xv = host_v[0, ctx - n_q:].double().numpy()
    reps, t0 = 0, time.perf_counter()
    while True:
        o.quantize(xk, s64, *tabk)
        o.quantize(xv, s64, *tabv)
        kh = np.stack([o.dequantize(o.unpack(raw_k[h], ctx, D, w.bits_k, 0), nk[h], s64, tabk[0])
                       for h in range(hkv)])[None]
        vh = np.stack([o.dequantize(o.unpack(raw_v[h], ctx, D, w.bits_v, 1), nv[h], s64, tabv[0])
                       for h in range(hkv)])[None]
        o.multi_query_attention(q64, kh, vh, 1.0 / math.sqrt(D))
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or reps >= 50:
            break
    value = reps * ctx / el
    log(f"[bench] cpu oracle: {reps} sample steps in {el:.1f} s")
    return with_cpu_context({"value": value, "unit": "KV-tokens/s", "cores": cpu_cores(), "kind": "oracle",
            "sample": f"batch element 0 of {w.batch}, all {hkv} kv heads / {hkv * g} query heads, "
                      f"{ctx} tokens, {n_q} query positions: quantize+pack the appended tokens, "
                      f"unpack+dequantize+attend; {reps} repetitions"})


def bench_prefill(args, w, signs, dev, tq, inputs, torch, np, log):
    hkv, ctx, layers = w.n_kv_heads, w.ctx, w.layers
    xs, caches = [], []
    in_bytes = out_bytes = 0
    for layer in range(layers):
        g = inputs.generate(w, device=dev, layer=layer, with_query=False)
        bk, bv = inputs.layer_bits(w, layer)
        kc = tq.PackedCache(1, hkv, ctx, bk, tq.LAYOUT_ROWS, signs, device=dev)
        vc = tq.PackedCache(1, hkv, ctx, bv, tq.LAYOUT_GROUP8, signs, device=dev)
        xs.append((g["k"].contiguous(), g["v"].contiguous()))
        caches.append((kc, vc))
        in_bytes += 2 * hkv * ctx * D * 2
        out_bytes += hkv * ctx * ((D * bk // 8 + 2) + (D * bv // 8 + 2))
    torch.cuda.synchronize()
    log(f"[bench] prefill: {layers} layers, in {in_bytes / 1e9:.3f} GB, out {out_bytes / 1e9:.3f} GB "
        f"({in_bytes / out_bytes:.2f}x smaller)")

    def step(i):
        for (kc, vc), (k, v) in zip(caches, xs):
            tq.quantize_append_kv(kc, vc, k, v, 0)

    timer = Timer(torch, args.eager, cache_flush(torch, tq))
    steps = max(1, args.steps // 20)
    ms_per_step = timer.per_iteration_ms(step, steps, max(1, args.warmup // 20))
    tokens = layers * ctx
    value = tokens / (ms_per_step / 1e3)
    achieved = (in_bytes + out_bytes) / (ms_per_step / 1e3) / 1e9
    result = {
        "metric": METRIC, "value": value, "unit": "tokens/s (layer x position, K and V of all kv heads)",
        "n_gpus": 1, "steps": steps, "warmup": max(1, args.warmup // 20), "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; shapes and value distributions of the workload)",
        "config": {"workload": w.name, "layers": layers, "n_kv_heads": hkv, "d": D, "tokens": ctx,
                   "bits": "K4/V3, layers 0,1,30,31 at 8/8", "packed_vs_bf16": in_bytes / out_bytes,
                   "timing": "eager" if args.eager else "hip graph replay"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": QUANTIZE_KERNEL + " (32 launches per step, K and V of one layer each)",
                     "bytes_per_launch": (in_bytes + out_bytes) / layers},
        "_kernel": "quantize",
        "_launches": layers,
    }
    mix = recorded_instmix("quantize_kv_kernel", w.name)
    if mix is not None:
        result["roofline"]["valu_issue_fraction"] = {
            "value": mix.get("valu_issue_fraction"), "per_wave": mix.get("per_wave"),
            "record": f"profiles/instmix_quantize_kv_kernel_{w.name}.txt",
            "note": "vector-instruction issue cycles (4 per wave64 instruction) over the recorded launch time"}
    if not args.no_cpu_baseline:
        from oracle import tq_oracle as o
        s64 = signs.cpu().numpy().astype(np.float64)
        tab4, tab3 = o.make_codebook(D, 4)[:2], o.make_codebook(D, 3)[:2]
        xk = xs[5][0][0, :1024].double().cpu().numpy()
        xv = xs[5][1][0, :1024].double().cpu().numpy()
        reps, t0 = 0, time.perf_counter()
        while True:
            ck, _, _ = o.quantize(xk, s64, *tab4)
            cv, _, _ = o.quantize(xv, s64, *tab3)
            for h in range(hkv):
                o.pack(ck[:, h], 4, 0)
                o.pack(cv[:, h], 3, 1)
            reps += 1
            el = time.perf_counter() - t0
            if el > 10.0 or reps >= 100:
                break
        result["cpu_baseline"] = with_cpu_context({
            "value": reps * 1024 / el, "unit": result["unit"], "cores": cpu_cores(), "kind": "oracle",
            "sample": f"layer 5, 1024 positions x {hkv} kv heads, K4/V3, quantize+pack, {reps} reps"})
    return result


def recorded_instmix(kernel, workload):
    """The committed instruction-mix record of a kernel (rocprofv3 counters), or None."""
    path = os.path.join(ROOT, "profiles", f"instmix_{kernel}_{workload}.txt")
    try:
        with open(path) as fh:
            return json.load(fh)
    except (OSError, ValueError):
        return None


def calibrate_copy(torch, log):
    """Plain device-to-device copies of COPY_BYTES each (read COPY_BYTES, write COPY_BYTES)."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    for _ in range(CALIBRATION_COPIES):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] calibration: 5 copies of {COPY_BYTES} bytes")


# ---- rocprofv3 summaries -------------------------------------------------------------------

def _short(name: str) -> str:
    n = name.replace("void ", "").replace("tq::(anonymous namespace)::", "")
    return n.split("(")[0][:90]


def _trace_medians(d):
    """Median duration (ns) per kernel from the run's kernel trace (csv, or csv.gz), if kept."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv*"), recursive=True)
    if not files:
        return {}
    import gzip
    opener = gzip.open if files[0].endswith(".gz") else open
    durs = {}
    with opener(files[0], "rt") as fh:
        for r in csv.DictReader(fh):
            durs.setdefault(_short(r["Kernel_Name"]), []).append(
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = {}
    for k, v in durs.items():
        v.sort()
        out[k] = v[len(v) // 2]
    return out


def summarize_stats(args):
    """Kernel table of a `rocprofv3 --kernel-trace --stats --output-format csv` run: calls, mean,
    median (from the kernel trace: the mean also counts the slower first replays after a graph
    capture or a cache flush), min, max and share of the time."""
    files = glob.glob(os.path.join(args.summarize_stats, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        sys.exit(f"no kernel_stats.csv under {args.summarize_stats}")
    rows = list(csv.DictReader(open(files[0])))
    med = _trace_medians(args.summarize_stats)
    lines = [f"# {args.name}", "", f"command: {args.command}", "",
             f"{'kernel':90s} {'calls':>7s} {'avg us':>10s} {'median us':>10s} {'min us':>10s} {'max us':>10s} "
             f"{'total %':>8s}"]
    for r in rows:
        m = med.get(_short(r["Name"]))
        ms = f"{m / 1e3:10.2f}" if m is not None else f"{'-':>10s}"
        lines.append(f"{_short(r['Name']):90s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.2f} {ms} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):8.2f}")
    out = "\n".join(lines) + "\n"
    with open(os.path.join(ROOT, "profiles", f"{args.name}.txt"), "w") as fh:
        fh.write(out)
    print(out)


def _counter_means(d, counter):
    """Mean per-dispatch value of `counter` per kernel (short name) in a rocprofv3 --pmc run."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    acc = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (_short(r["Kernel_Name"]), r.get("Dispatch_Id", ""))
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    per_kernel = {}
    for (name, _), v in acc.items():
        per_kernel.setdefault(name, []).append(v)
    means = {k: sum(v) / len(v) for k, v in per_kernel.items()}
    # the calibration copies are the largest dispatches of the runtime's copy kernel (it also
    # serves the small host-to-device uploads of the run)
    for k, v in per_kernel.items():
        if CALIBRATION_KERNEL in k:
            top = sorted(v)[-CALIBRATION_COPIES:]
            means[k] = sum(top) / len(top)
    return means, {k: len(v) for k, v in per_kernel.items()}


def summarize_traffic(args):
    """HBM bytes per launch of `--kernel`: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
    scaled by bytes / counter of the calibration copies of the same runs."""
    fetch, nf = _counter_means(args.fetch, "FETCH_SIZE")
    write, nw = _counter_means(args.write, "WRITE_SIZE")

    def pick(table, pat):
        keys = [k for k in table if pat in k]
        if not keys:
            sys.exit(f"no kernel matching {pat!r} in {sorted(table)}")
        return keys[0]

    def weighted(table, counts):
        # every instance of the kernel (e.g. the bit widths of the prefill layers), weighted
        # by its number of dispatches
        keys = sorted(k for k in table if re.search(args.kernel, k) and CALIBRATION_KERNEL not in k)
        if not keys:
            sys.exit(f"no kernel matching {args.kernel!r} in {sorted(table)}")
        n = sum(counts[k] for k in keys)
        return keys, sum(table[k] * counts[k] for k in keys) / n, {k: counts[k] for k in keys}

    def summed(table, counts):
        keys = sorted(k for k in table if re.search(args.kernel, k) and CALIBRATION_KERNEL not in k)
        if not keys:
            sys.exit(f"no kernel matching {args.kernel!r} in {sorted(table)}")
        return keys, sum(table[k] for k in keys), {k: counts[k] for k in keys}

    agg = summed if args.sum_instances else weighted
    kf, mf, df = agg(fetch, nf)
    kw, mw, dw = agg(write, nw)
    cf, cw = pick(fetch, CALIBRATION_KERNEL), pick(write, CALIBRATION_KERNEL)
    scale_f = COPY_BYTES / (fetch[cf] * 1024.0)
    scale_w = COPY_BYTES / (write[cw] * 1024.0)
    fb = mf * 1024.0 * scale_f
    wb = mw * 1024.0 * scale_w
    rec = {"kernel": kf, "workload": args.workload, "fetch_kib_per_dispatch": mf,
           "write_kib_per_dispatch": mw,
           "per_instance_kib": {k: {"fetch": fetch[k], "write": write.get(k)} for k in kf},
           "copy_fetch_kib": fetch[cf], "copy_write_kib": write[cw],
           "copy_bytes": COPY_BYTES, "fetch_scale": scale_f, "write_scale": scale_w,
           "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb, "bytes_per_launch": fb + wb,
           "dispatches": {"fetch": df, "write": dw}, "sources_digest": kernel_sources_digest(),
           "per_step": "sum of the matching kernels" if args.sum_instances else "dispatch-weighted mean",
           "command": args.command}
    kname = args.record or ("decode" if args.kernel.startswith(DECODE_KERNEL) else "quantize")
    with open(os.path.join(ROOT, "profiles", f"traffic_{kname}_{args.workload}.txt"), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def summarize_instmix(args):
    """Instructions per wave of `--kernel` (all its instances, dispatch-weighted) from
    SQ_WAVES and SQ_INSTS_{VALU,MFMA,LDS,SALU,VMEM}, and the vector-ALU issue fraction: a wave64
    VALU instruction occupies a 16-lane SIMD for 4 cycles, so the fraction is
    4 x (VALU - MFMA instructions) / (SIMDs x clock x launch time) (256 CUs x 4 SIMDs, 2.4 GHz)."""
    names = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM"]
    got = {}
    for n in names:
        means, counts = _counter_means(args.summarize_instmix, n)
        keys = [k for k in means if re.search(args.kernel, k)]
        if keys:
            tot = sum(counts[k] for k in keys)
            got[n] = sum(means[k] * counts[k] for k in keys) / tot
    if "SQ_WAVES" not in got or "SQ_INSTS_VALU" not in got:
        sys.exit(f"no SQ_WAVES / SQ_INSTS_VALU for {args.kernel!r}")
    waves = got["SQ_WAVES"]
    rec = {"kernel": args.kernel, "workload": args.workload, "waves_per_launch": waves,
           "per_wave": {n[9:].lower(): got[n] / waves for n in names[1:] if n in got},
           "command": args.command}
    if args.kernel_us:
        cycles = args.kernel_us * 1e-6 * 2.4e9
        rec["launch_us"] = args.kernel_us
        # SQ_INSTS_VALU includes the matrix instructions, which run on their own unit
        rec["valu_issue_fraction"] = 4.0 * (got["SQ_INSTS_VALU"] - got.get("SQ_INSTS_MFMA", 0.0)) / (1024 * cycles)
    base = DECODE_KERNEL if args.kernel.startswith(DECODE_KERNEL) else QUANTIZE_KERNEL
    with open(os.path.join(ROOT, "profiles", f"instmix_{base}_{args.workload}.txt"), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()

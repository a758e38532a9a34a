"""The hot path recorded into a HIP graph gives, on every replay, what eager launches give.

The decode kernel keeps per-(batch, kv head) arrival counters in the caller's workspace and
clears them itself, and no call of the path records a memset, so a graph of append + decode
steps can be replayed any number of times.  The search keeps only per-block candidates in its
workspace, rewritten by every call.  Each replay is checked against the eager result with eager
work and synchronisations in between.
"""
import math
import sys

import pytest

torch = pytest.importorskip("torch")

import compressed_decode_attention_tq_amd as tq  # noqa: E402
from compressed_decode_attention_tq_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("workload,tau,batch,ctx,fused", [
    ("llama8k", 0.0, 2, 2048 + 37, False), ("ctx131k", 0.0, 2, 2048 + 37, False),
    ("batch32k", 1e-4, 2, 2048 + 37, False),
    # splits of 3072+ tokens: 12 waves per workgroup (dense), 16 and 12 in the key pass
    ("batch32k", 0.0, 32, 3100, False), ("batch32k", 1e-4, 32, 3100, False), ("ctx131k", 1e-4, 64, 6200, False),
    # the decode step as one call: append inside the dense launch, or inside Sparse V's key pass
    ("llama8k", 0.0, 2, 2048 + 37, True), ("ctx131k", 1e-4, 2, 2048 + 37, True), ("batch32k", 1e-4, 32, 3100, True),
])
def test_graph_replays_match_eager(workload, tau, batch, ctx, fused):
    print("graph", workload, tau, batch, ctx, fused, flush=True)
    sys.stdout.flush()
    w = inputs.WORKLOADS[workload]
    hkv = w.n_kv_heads
    hq = hkv * w.group
    g = inputs.generate(w, device=DEV, batch=batch, ctx=ctx, n_kv_heads=hkv, n_q_heads=hq)
    signs = inputs.rotation_signs().to(DEV)
    cap = (ctx + 63) // 64 * 64 + 64
    caches = []
    for _ in range(2):
        kc = tq.PackedCache(batch, hkv, cap, w.bits_k, tq.LAYOUT_ROWS, signs, device=DEV)
        vc = tq.PackedCache(batch, hkv, cap, w.bits_v, tq.LAYOUT_GROUP8, signs, device=DEV)
        tq.quantize_append(kc, g["k"][:, : ctx - 1].contiguous(), 0)
        tq.quantize_append(vc, g["v"][:, : ctx - 1].contiguous(), 0)
        caches.append((kc, vc))
    k_new = g["k"][:, ctx - 1:].contiguous()
    v_new = g["v"][:, ctx - 1:].contiguous()
    q = g["q"].contiguous()
    bufs = [tq.DecodeBuffers(batch, hq, hkv, ctx, tau, device=DEV) for _ in caches]
    scale = 1.0 / math.sqrt(128)

    def step(i):
        kc, vc = caches[i]
        if fused:
            tq.decode_attn_append(kc, vc, k_new, v_new, q, ctx, scale, buffers=bufs[i], tau=tau)
            return
        tq.quantize_append(kc, k_new, ctx - 1)
        tq.quantize_append(vc, v_new, ctx - 1)
        tq.decode_attn(kc, vc, q, ctx, scale, tau=tau, buffers=bufs[i])

    for i in range(2):
        step(i)
    torch.cuda.synchronize()
    eager = [(b.out.clone(), b.lse.clone()) for b in bufs]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(2):
            step(i)
    for rep in range(3):
        for b in bufs:
            b.out.fill_(float("nan"))
            b.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, b in enumerate(bufs):
            assert torch.equal(b.out, eager[i][0]), f"replay {rep}, step {i}: out differs"
            assert torch.equal(b.lse, eager[i][1]), f"replay {rep}, step {i}: lse differs"
        step(0)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(bufs[0].out, eager[0][0])


@pytest.mark.parametrize("n,nq,k", [(300000, 11, 10), (70000, 8, 64)])
def test_search_graph_replays_match_eager(n, nq, k):
    """Inner-product search (score kernel, then the final ranking) recorded into a graph over
    two databases, replayed with eager searches of a third in between."""
    print("graph search", n, nq, k, flush=True)
    spec = dict(inputs.SEARCH["search1m"])
    g = inputs.generate_search(spec, device=DEV, n=n, n_queries=nq)
    signs = inputs.rotation_signs().to(DEV)
    cap = (n + 63) // 64 * 64
    dbs = []
    for c in range(3):
        db = tq.PackedCache(1, 1, cap, 4, tq.LAYOUT_ROWS, signs, device=DEV)
        x = g["x"] if c == 0 else g["x"].flip(0).contiguous() if c == 1 else (g["x"] * 0.5).contiguous()
        tq.quantize_append(db, x[None, :, None, :].contiguous(), 0)
        dbs.append(db)
    q = g["q"].contiguous()
    bufs = [tq.SearchBuffers(nq, n, k, device=DEV) for _ in range(2)]
    extra = tq.SearchBuffers(nq, n, k, device=DEV)
    for i in range(2):
        tq.ip_search(dbs[i], q, n, k, buffers=bufs[i])
    tq.ip_search(dbs[2], q, n, k, buffers=extra)
    torch.cuda.synchronize()
    eager = [(b.idx.clone(), b.score.clone()) for b in bufs]
    eager_extra = extra.idx.clone()
    assert not torch.equal(eager[0][0], eager[1][0])  # the two databases rank differently

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(2):
            tq.ip_search(dbs[i], q, n, k, buffers=bufs[i])
    for rep in range(3):
        for b in bufs:
            b.idx.fill_(-7)
            b.score.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, b in enumerate(bufs):
            assert torch.equal(b.idx, eager[i][0]), f"replay {rep}, database {i}: idx differs"
            assert torch.equal(b.score, eager[i][1]), f"replay {rep}, database {i}: score differs"
        tq.ip_search(dbs[2], q, n, k, buffers=extra)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(extra.idx, eager_extra)


@pytest.mark.parametrize("tau,hq", [(0.0, 16), (1e-4, 16), (1e-3, 8)])
def test_qjl_graph_replays_match_eager(tau, hq):
    """The QJL decode step (the key-and-value append in one launch, then the decode: one launch,
    or Sparse V's key pass and masked value pass) recorded into a graph over two caches,
    replayed with eager calls in between."""
    print("graph qjl", tau, hq, flush=True)
    w = inputs.WORKLOADS["qjl8k"]
    batch, hkv, ctx = 2, 2, 3000
    g = inputs.generate(w, device=DEV, batch=batch, ctx=ctx, n_kv_heads=hkv, n_q_heads=hq)
    signs = inputs.rotation_signs().to(DEV)
    proj = inputs.qjl_projection()
    cap = (ctx + 63) // 64 * 64
    caches = []
    for c in range(2):
        kc = tq.PackedCache(batch, hkv, cap, 3, tq.LAYOUT_ROWS, signs, device=DEV)
        vc = tq.PackedCache(batch, hkv, cap, 2, tq.LAYOUT_GROUP8, signs, device=DEV)
        sk = tq.QjlSketch(kc, proj, device=DEV)
        k = g["k"] if c == 0 else g["k"].flip(1).contiguous()
        tq.qjl_quantize_append(kc, sk, k.contiguous(), 0)
        tq.quantize_append(vc, g["v"].contiguous(), 0)
        caches.append((kc, sk, vc))
    q = g["q"].contiguous()
    sl = torch.tensor([ctx, ctx - 777], dtype=torch.int32, device=DEV)
    scale = 1.0 / math.sqrt(128)
    bufs = [tq.DecodeBuffers(batch, hq, hkv, ctx, tau, device=DEV) for _ in caches]

    k_new = g["k"][:, ctx - 1:].contiguous()
    v_new = g["v"][:, ctx - 1:].contiguous()

    def step(i):  # the decode step: keys (with their sketch) and values in one launch, then attend
        kc, sk, vc = caches[i]
        tq.qjl_quantize_append_kv(kc, sk, vc, k_new, v_new, ctx - 1)
        tq.qjl_decode_attn(kc, sk, vc, q, ctx, scale, tau=tau, seq_lens=sl, buffers=bufs[i])

    for i in range(2):
        step(i)
    torch.cuda.synchronize()
    eager = [(b.out.clone(), b.lse.clone()) for b in bufs]
    assert not torch.equal(eager[0][0], eager[1][0])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(2):
            step(i)
    for rep in range(3):
        for b in bufs:
            b.out.fill_(float("nan"))
            b.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, b in enumerate(bufs):
            assert torch.equal(b.out, eager[i][0]), f"replay {rep}, cache {i}: out differs"
            assert torch.equal(b.lse, eager[i][1]), f"replay {rep}, cache {i}: lse differs"
        step(0)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(bufs[0].out, eager[0][0])

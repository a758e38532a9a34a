"""The hot path recorded into a HIP graph gives, on every replay, what eager launches give.

The decode kernel keeps per-(batch, kv head) arrival counters in the caller's workspace and
clears them itself, and no call of the path records a memset, so a graph of append + decode
steps can be replayed any number of times.  Each replay is checked against the eager result
with eager work and synchronisations in between.
"""
import math
import sys

import pytest

torch = pytest.importorskip("torch")

import compressed_decode_attention_tq_amd as tq  # noqa: E402
from compressed_decode_attention_tq_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("workload,tau", [("llama8k", 0.0), ("ctx131k", 0.0), ("batch32k", 1e-4)])
def test_graph_replays_match_eager(workload, tau):
    print("graph", workload, tau, flush=True)
    sys.stdout.flush()
    w = inputs.WORKLOADS[workload]
    batch, hkv, ctx = 2, w.n_kv_heads, 2048 + 37
    hq = hkv * w.group
    g = inputs.generate(w, device=DEV, batch=batch, ctx=ctx, n_kv_heads=hkv, n_q_heads=hq)
    signs = inputs.rotation_signs().to(DEV)
    cap = 2112
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

"""Seeded synthetic inputs shaped like the workloads the TurboQuant pages describe.

This module only draws random numbers; it holds none of the method's arithmetic,
so both the HIP path and the CPU oracle may use it.  Every draw goes through a
`torch.Generator` seeded from the workload's seed; streams drawn on a CPU
generator and on a GPU generator differ, so a test that compares the two sides
draws once and hands the same tensors to both.

Workloads (d = 128 everywhere):
  tiny    1 kv head, 1 query head, 1024 tokens, fp32 N(0,1) K/V from seed 0,
          4 random channels x10, K 4-bit / V 2-bit, fp32 query.
  llama8k batch 1, 32 query heads, 8 kv heads, 8192 tokens, bf16 N(0,1) times
          per-(kv head, channel) scales log-uniform in [0.5, 20] (separate for
          K and V), seed 2, K 4-bit / V 2-bit; 8191 tokens prefilled, 1 appended.
  batch32k batch 16, 32/8 heads, 32768 tokens, bf16 Student-t(5) with 8 random
          channels x4, seed 3, K 3-bit / V 2-bit, Sparse V tau 1e-4 (and 0).
  prefill 32 layers, 8 kv heads, 32768 tokens, bf16 N(0,1) times a per-layer std
          uniform in [0.5, 3] (shared by K and V), seed 4; K 4-bit / V 3-bit,
          layers 0, 1, 30, 31 at 8/8 bits.
  ctx131k batch 4, 16/2 heads (group 8), 131072 tokens, bf16 N(0,1), 2% of the
          token positions of each sequence x8 in K and V (attention sinks),
          seed 5, K 4-bit / V 2-bit, Sparse V tau 1e-4.
  qjl8k   as llama8k (seed 9) with QJL keys: 3-bit codes plus a 128-row Gaussian sign
          sketch of the residual (sketch matrix from seed 10), V 2-bit.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

D = 128
SIGN_SEED = 1


def rotation_signs(d: int = D, seed: int = SIGN_SEED) -> torch.Tensor:
    """Random +/-1 vector (int8, CPU) for the random-sign Hadamard rotation."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    bits = torch.randint(0, 2, (d,), generator=g)
    return (1 - 2 * bits).to(torch.int8)


QJL_SEED = 10


def qjl_projection(m: int = D, d: int = D, seed: int = QJL_SEED) -> torch.Tensor:
    """Gaussian sketch matrix S [m, d] (fp32, CPU) with i.i.d. N(0, 1) entries, for the QJL
    residual variant; drawn here and passed in (the library has no random generator)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn((m, d), generator=g, dtype=torch.float32)


@dataclass
class Workload:
    name: str
    seed: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    ctx: int
    bits_k: int
    bits_v: int
    dtype: torch.dtype
    dist: str                      # "normal" | "student5"
    tau: float = 0.0
    outlier_channels: int = 0
    outlier_scale: float = 1.0
    head_channel_scales: tuple | None = None   # (lo, hi) log-uniform, per kv head+channel
    sink_fraction: float = 0.0
    sink_scale: float = 1.0
    layers: int = 1
    layer_std: tuple | None = None             # (lo, hi) uniform, per layer
    boundary_layers: tuple = ()
    boundary_bits: int = 8
    append: int = 0                            # tokens appended after the prefill
    n_q: int = 1                               # query positions per sequence (multi-query)
    page_tokens: int = 0                       # paged cache: positions per page (0 = contiguous)
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 1, 1, 1024, 4, 2, torch.float32, "normal",
                     outlier_channels=4, outlier_scale=10.0),
    "llama8k": Workload("llama8k", 2, 1, 32, 8, 8192, 4, 2, torch.bfloat16, "normal",
                        head_channel_scales=(0.5, 20.0), append=1),
    "batch32k": Workload("batch32k", 3, 16, 32, 8, 32768, 3, 2, torch.bfloat16, "student5",
                         tau=1e-4, outlier_channels=8, outlier_scale=4.0),
    "prefill": Workload("prefill", 4, 1, 8, 8, 32768, 4, 3, torch.bfloat16, "normal",
                        layers=32, layer_std=(0.5, 3.0), boundary_layers=(0, 1, 30, 31)),
    "ctx131k": Workload("ctx131k", 5, 4, 16, 2, 131072, 4, 2, torch.bfloat16, "normal",
                        tau=1e-4, sink_fraction=0.02, sink_scale=8.0),
    # speculative verification on the Llama-3-8B-shaped layer: 4 new positions per step
    "verify8k": Workload("verify8k", 6, 1, 32, 8, 8192, 4, 2, torch.bfloat16, "normal",
                         head_channel_scales=(0.5, 20.0), append=4, n_q=4),
    # a prefill chunk on the Llama-3-8B-shaped layer: 512 new positions at the end of 8192
    "chunk8k": Workload("chunk8k", 11, 1, 32, 8, 8192, 4, 2, torch.bfloat16, "normal",
                        head_channel_scales=(0.5, 20.0), append=512, n_q=512),
    # the batched long-context shape in a paged cache: 256-token pages, shuffled in the pool
    "paged32k": Workload("paged32k", 7, 16, 32, 8, 32768, 3, 2, torch.bfloat16, "student5",
                         outlier_channels=8, outlier_scale=4.0, append=1, page_tokens=256),
    # the Llama-3-8B-shaped layer with QJL keys: 3-bit codes plus a 128-bit sign sketch of the
    # residual (4 bits per coordinate in all), 2-bit values
    "qjl8k": Workload("qjl8k", 9, 1, 32, 8, 8192, 3, 2, torch.bfloat16, "normal",
                      head_channel_scales=(0.5, 20.0), append=1, extra={"qjl_m": 128}),
}


def _draw(dist: str, shape, g: torch.Generator, device) -> torch.Tensor:
    if dist == "normal":
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if dist == "student5":
        # t_5 = Z / sqrt(chi2_5 / 5); chi2_5 = sum of 5 squared normals.
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        chi = torch.zeros(shape, device=device, dtype=torch.float32)
        for _ in range(5):
            e = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            chi.addcmul_(e, e)
        return z / torch.sqrt(chi / 5.0)
    raise ValueError(dist)


def generate(w: Workload, device="cpu", batch=None, ctx=None, n_kv_heads=None,
             n_q_heads=None, layer: int = 0, with_query: bool = True, n_q=None) -> dict:
    """Draw K, V [batch, ctx, n_kv_heads, d] and q [batch, n_q_heads, d] for one layer
    (q [batch, n_q, n_q_heads, d] for a workload or call with n_q > 1).

    Shapes default to the workload's; smaller shapes keep the same recipe.
    Draw order: special channels / positions, K, V, scales, q.  Values are
    drawn in fp32 and rounded (round to nearest even) to the workload dtype.
    """
    batch = w.batch if batch is None else batch
    ctx = w.ctx if ctx is None else ctx
    hkv = w.n_kv_heads if n_kv_heads is None else n_kv_heads
    hq = w.n_q_heads if n_q_heads is None else n_q_heads
    g = torch.Generator(device=device).manual_seed(w.seed * 1000 + layer)
    info = {}
    ch = None
    if w.outlier_channels:
        ch = torch.randperm(D, generator=g, device=device)[: w.outlier_channels]
        info["outlier_channels"] = ch.cpu().tolist()
    sinks = None
    if w.sink_fraction:
        n_sink = int(round(w.sink_fraction * ctx))
        sinks = torch.stack([torch.randperm(ctx, generator=g, device=device)[:n_sink]
                             for _ in range(batch)])
        info["sinks"] = sinks.cpu()
    k = _draw(w.dist, (batch, ctx, hkv, D), g, device)
    v = _draw(w.dist, (batch, ctx, hkv, D), g, device)
    if ch is not None:
        k[..., ch] *= w.outlier_scale
        v[..., ch] *= w.outlier_scale
    if w.head_channel_scales is not None:
        lo, hi = (math.log(x) for x in w.head_channel_scales)
        sk = torch.exp(lo + (hi - lo) * torch.rand((hkv, D), generator=g, device=device))
        sv = torch.exp(lo + (hi - lo) * torch.rand((hkv, D), generator=g, device=device))
        k *= sk
        v *= sv
    if w.layer_std is not None:
        lo, hi = w.layer_std
        std = lo + (hi - lo) * torch.rand((), generator=g, device=device)
        k *= std
        v *= std
        info["layer_std"] = float(std)
    if sinks is not None:
        for b in range(batch):
            k[b, sinks[b]] *= w.sink_scale
            v[b, sinks[b]] *= w.sink_scale
    out = {"k": k.to(w.dtype), "v": v.to(w.dtype), "info": info}
    n_q = w.n_q if n_q is None else n_q
    if with_query:
        shape = (batch, hq, D) if n_q == 1 else (batch, n_q, hq, D)
        out["q"] = torch.randn(shape, generator=g, device=device).to(w.dtype)
    return out


def layer_bits(w: Workload, layer: int) -> tuple:
    """(bits_k, bits_v) of a layer; boundary layers keep the higher width."""
    if layer in w.boundary_layers:
        return w.boundary_bits, w.boundary_bits
    return w.bits_k, w.bits_v


# Inner-product search: a database of n vectors drawn around `centers` cluster centres
# (centre N(0, 1) plus N(0, spread^2) noise, the shape of an embedding collection) and
# queries drawn the same way around random centres.  No public search benchmark is
# available offline; this stands in for one.
SEARCH = {
    "search1m": dict(seed=8, n=1 << 20, n_queries=8, top_k=10, bits=4, centers=1024, spread=0.5,
                     dtype=torch.bfloat16),
}


def generate_search(spec: dict, device="cpu", n=None, n_queries=None) -> dict:
    """Database x [n, d] and queries [n_queries, d] (fp32 drawn, rounded to spec dtype)."""
    n = spec["n"] if n is None else n
    nq = spec["n_queries"] if n_queries is None else n_queries
    g = torch.Generator(device=device).manual_seed(spec["seed"] * 1000)
    centers = torch.randn((spec["centers"], D), generator=g, device=device)
    which = torch.randint(0, spec["centers"], (n,), generator=g, device=device)
    x = centers[which] + spec["spread"] * torch.randn((n, D), generator=g, device=device)
    qc = torch.randint(0, spec["centers"], (nq,), generator=g, device=device)
    q = centers[qc] + spec["spread"] * torch.randn((nq, D), generator=g, device=device)
    return {"x": x.to(spec["dtype"]), "q": q.to(spec["dtype"])}

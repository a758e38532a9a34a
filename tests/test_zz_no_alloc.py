"""The allocation-free decode step (tq_decode_attn_append_noalloc) against the workspace entry
point it varies (tq_decode_attn_append): same caches, same inputs, calls in a row on one GPU, a
smaller problem after a larger one (the static scratch keeps the last call's contents), then the
larger one again.  Outputs must be bit-identical (the same kernel and split plan), the caches
must hold the same appended token, and the output must meet the oracle's tolerance."""
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


def _pair(batch, hkv, cap, bits_k, signs_dev):
    kc = tq.PackedCache(batch, hkv, cap, bits_k, tq.LAYOUT_ROWS, signs_dev, device=DEV)
    vc = tq.PackedCache(batch, hkv, cap, 2, tq.LAYOUT_GROUP8, signs_dev, device=DEV)
    return kc, vc


def _case(name, batch, hq, hkv, ctx, cap, bits_k, seq_lens, golden):
    _say("noalloc", name, batch, hq, hkv, ctx, bits_k, seq_lens)
    w = inputs.WORKLOADS[name]
    signs = inputs.rotation_signs()
    sd = signs.to(DEV)
    g = inputs.generate(w, device="cpu", batch=batch, ctx=ctx, n_kv_heads=hkv, n_q_heads=hq)
    k, v = g["k"], g["v"]
    lens = [ctx] * batch if seq_lens is None else list(seq_lens)
    a, b = _pair(batch, hkv, cap, bits_k, sd), _pair(batch, hkv, cap, bits_k, sd)
    for kc, vc in (a, b):
        tq.quantize_append(kc, k.to(DEV), 0)
        tq.quantize_append(vc, v.to(DEV), 0)
    k_new = torch.zeros((batch, 1, hkv, 128), dtype=k.dtype)
    v_new = torch.zeros((batch, 1, hkv, 128), dtype=v.dtype)
    for i, tb in enumerate(lens):
        if tb >= 1:  # the new token is each sequence's last position, overwritten by the call
            k_new[i, 0] = k[i, tb - 1] * -1.5
            v_new[i, 0] = v[i, tb - 1] * 0.75
    k_new, v_new = k_new.to(DEV), v_new.to(DEV)
    q = g["q"].to(DEV).contiguous()
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    scale = 1.0 / math.sqrt(128)
    ref = tq.decode_attn_append(a[0], a[1], k_new, v_new, q, ctx, scale, seq_lens=sl)
    out, lse = tq.decode_attn_append_noalloc(b[0], b[1], k_new, v_new, q, ctx, scale, seq_lens=sl)
    torch.cuda.synchronize()
    assert torch.equal(out, ref.out) and torch.equal(lse, ref.lse)
    for ca, cb in zip(a, b):
        assert torch.equal(ca.codes, cb.codes) and torch.equal(ca.norms, cb.norms)
    s64 = signs.numpy().astype(np.float64)
    kh = parity.oracle_cache_view(b[0], s64, golden[bits_k], ctx)
    vh = parity.oracle_cache_view(b[1], s64, golden[2], ctx)
    ref_o, ref_lse, _ = o.decode_attention(parity.to_f64(g["q"]), kh, vh, scale, seq_lens=lens)
    fin = np.isfinite(ref_lse)
    got_lse = lse.cpu().numpy()
    assert np.all(np.isneginf(got_lse[~fin]))
    assert np.allclose(got_lse[fin], ref_lse[fin], rtol=0, atol=1e-3 * np.maximum(1, np.abs(ref_lse[fin])))
    worst = parity.check_rows(out.cpu().numpy(), ref_o, "noalloc decode out")
    _say(f"  bit-identical to the workspace call; worst rel err vs oracle {worst:.2e}")


def test_noalloc_decode_step_matches_workspace_entry_point(golden_codebooks):
    # a larger call, a smaller one after it (fewer (batch, kv head) counters, fewer splits,
    # other widths), then the larger one again: counters and partials reused each time
    _case("llama8k", 3, 32, 8, 3000, 3008, 4, None, golden_codebooks)
    _case("batch32k", 1, 8, 2, 700, 704, 3, [700], golden_codebooks)
    _case("ctx131k", 2, 16, 2, 4000, 4032, 4, [4000, 1], golden_codebooks)

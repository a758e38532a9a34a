"""Build libtq.so (HIP kernels for gfx950 + the C-ABI) in place, next to this file.

    python -m compressed_decode_attention_tq_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtq.so")

SOURCES = ["api.hip", "quantize.hip", "quantize_kv.hip", "append_small.hip", "ip_search.hip", "decode_generic.hip", "decode_mfma.hip", "decode_fused.hip",
           "noalloc.hip", "qjl.hip", "probe.hip", "codebook.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-fPIC", "-std=c++17",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # packed-fp32 instructions stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in p.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if p.returncode != 0:
        raise RuntimeError(f"build step failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(OUT_DIR, src + ".o")
        objs.append(obj)
        cmd = [HIPCC, f"--offload-arch={ARCH}", *COMMON, "-c", path, "-o", obj]
        if src.endswith(".cpp"):
            cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    for cmd, p in procs:
        out, _ = p.communicate()
        out = "\n".join(ln for ln in out.splitlines() if "packed-fp32-ops" not in ln)
        if p.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

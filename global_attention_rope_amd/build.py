"""Build ``libmimo_attn.so`` (gfx950) in-tree with hipcc.

Usage: ``python -m global_attention_rope_amd.build`` (or ``build()`` from Python).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmimo_attn.so")
SOURCES = ["abi.hip", "prefill_bf16.hip", "decode_bf16.hip", "rope_kv.hip", "attn_f32.hip",
           "layer.hip", "router.hip", "verify_bf16.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def command(out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 VALU ops stay disabled in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            # the LDS-DMA wrapper clobbers m0 on purpose (no other m0 user in these kernels)
            "-Wno-inline-asm",
            "-I", os.path.join(ROOT, "include"),
            *[os.path.join(CSRC, s) for s in SOURCES], "-lhipblaslt", "-o", out]


def build(verbose: bool = False) -> str:
    """Compile every source (always) and atomically replace the library."""
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

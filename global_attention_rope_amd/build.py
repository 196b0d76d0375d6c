"""Build ``libmimo_attn.so`` (gfx950) in-tree with hipcc.

Usage: ``python -m global_attention_rope_amd.build`` (or ``build()`` from Python).

Each source is compiled to an object of its own, in parallel, then the objects are linked; every
call recompiles every source.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmimo_attn.so")
PROBE_LIB = os.path.join(PKG, "libmimo_probe.so")   # latency references (measurement aid)
PROBE_SOURCES = ["probe.hip"]
OBJ_DIR = os.path.join(ROOT, "_build")
SOURCES = ["abi.hip", "prefill_bf16.hip", "decode_bf16.hip", "rope_kv.hip", "attn_f32.hip",
           "layer.hip", "router.hip", "verify_bf16.hip", "gemm_bf16.hip"]
ARCH = "gfx950"
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def compile_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed fp32 VALU ops stay disabled in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            # the LDS-DMA wrapper clobbers m0 on purpose (no other m0 user in these kernels)
            "-Wno-inline-asm",
            "-I", os.path.join(ROOT, "include")]


# Per-source code generation options.  The decode kernels are short, latency-bound launches whose
# code is fetched cold on every call: accumulating the matrix products in ordinary vector
# registers (not the accumulation registers, which the rescale and merge code would otherwise copy
# in and out) keeps their code about 12% smaller.
SOURCE_FLAGS = {"decode_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def flags_for(source: str) -> list[str]:
    return compile_flags() + SOURCE_FLAGS.get(source, [])


def command(out: str) -> list[str]:
    """One-shot command that compiles and links every source (kept for reference builds)."""
    return [hipcc(), *compile_flags(), "-shared",
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def _run(cmd: list[str]) -> tuple[int, str]:
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    return res.returncode, err


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source (always) and atomically replace the libraries."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    tag = f"{os.getpid()}"
    every = SOURCES + PROBE_SOURCES
    objs_all = [os.path.join(OBJ_DIR, s.replace(".hip", f".{tag}.o")) for s in every]
    objs = objs_all[:len(SOURCES)]
    cmds = [[hipcc(), *flags_for(s), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(every, objs_all)]
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    try:
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for s, (rc, err) in zip(every, results):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {s} ({rc}):\n{err}")
            if verbose and err.strip():
                print(err, file=sys.stderr)
        tmp = LIB + f".tmp{tag}"
        rc, err = _run([hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o", tmp])
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{err}")
        os.replace(tmp, LIB)
        tmp = PROBE_LIB + f".tmp{tag}"
        rc, err = _run([hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared",
                        *objs_all[len(SOURCES):], "-o", tmp])
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{err}")
        os.replace(tmp, PROBE_LIB)
    finally:
        for o in objs_all:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

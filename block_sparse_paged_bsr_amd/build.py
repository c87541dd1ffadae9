"""Build libbsr_attn.so (the attention path) and libbsr_probe.so (the HBM read probe that
bench.py prices the decode path against) in-tree with hipcc for gfx950.

Usage: ``python -m block_sparse_paged_bsr_amd.build`` (or ``build()`` from Python).
Every call recompiles every source; objects go to ``_build/`` next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libbsr_attn.so")
PROBE_OUT = os.path.join(HERE, "libbsr_probe.so")
BUILD = os.path.join(HERE, "_build")

SOURCES = [
    os.path.join(CSRC, "plan.cpp"),
    os.path.join(CSRC, "compose.cpp"),
    os.path.join(CSRC, "api.hip"),
    os.path.join(CSRC, "kernels", "attn_f32.hip"),
    os.path.join(CSRC, "kernels", "attn_prefill_bf16.hip"),
    os.path.join(CSRC, "kernels", "attn_decode_bf16.hip"),
    os.path.join(CSRC, "kernels", "merge.hip"),
]
PROBE_SOURCES = [os.path.join(CSRC, "hbm_probe.hip"), os.path.join(CSRC, "isa_probes.hip")]

ARCH = os.environ.get("BSR_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]
# Packed fp32 (v_pk_*_f32) code generation is switched off for every HIP source.
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The prefill kernel runs with the IEEE mode bit off: scores are never NaN (masked ones are
# -inf), and with the bit on every maximum over matrix-core results needs an extra NaN-quieting
# v_max_f32 per operand.
# The MFMA accumulators that the vector ALUs read (scores) stay in VGPRs; the 128-row shape
# places its output accumulators in AGPRs itself (inline asm), so the compiler's heuristic
# never moves scores into AGPRs and back.
EXTRA_FLAGS = {"attn_prefill_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + COMMON
    if src.endswith(".hip"):
        cmd += HIP_FLAGS + EXTRA_FLAGS.get(os.path.basename(src), []) + ["-x", "hip"]
    cmd += ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(out, objs):
    tmp = out + ".tmp"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(OUT, objs[:len(SOURCES)])
    _link(PROBE_OUT, objs[len(SOURCES):])
    if verbose:
        print(f"built {OUT} and {PROBE_OUT}")
    return OUT


if __name__ == "__main__":
    build()

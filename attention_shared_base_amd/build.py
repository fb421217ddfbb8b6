"""Build liblra_attn.so (all HIP sources, gfx950) in-tree with hipcc.

Usage: ``python -m attention_shared_base_amd.build`` or ``build()`` from Python.
Every call recompiles (the driver's "does it build" check relies on that).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "liblra_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["api.hip", "decode_bf16.hip", "decode_pa_bf16.hip", "decode_rope_bf16.hip",
           "decode_rope_pa_bf16.hip", "prefill_bf16.hip", "attn_f32.hip", "lr_build.hip",
           "naive_expand.hip", "paged.hip", "ceiling.hip"]
# per-source extra flags: the RoPE decodes keep MFMA results in VGPRs (their rotation
# reads them on the VALU)
EXTRA_FLAGS = {"decode_rope_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "decode_rope_pa_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build liblra_attn.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source for gfx950 and link the shared library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *CFLAGS, *EXTRA_FLAGS.get(src, []), f"-I{INCLUDE}", f"-I{CSRC}", "-c",
                     os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)

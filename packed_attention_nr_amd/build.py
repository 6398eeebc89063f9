"""Build libmmdit.so in-tree with hipcc for gfx950.

    python -m packed_attention_nr_amd.build        # or packed_attention_nr_amd.build.build()

Every source is compiled for gfx950 only (no CUDA or other targets), with the
packed-fp32 feature switched off, and linked into one shared library next to
this file. Objects go to _build/ at the repository root.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmmdit.so")

SOURCES = ["plan.cpp", "api.cpp", "prologue.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_f32.hip",
           "adaln.hip", "noalloc.hip", "probe.hip", "status.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmmdit.so)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


def compile_one(src: str, verbose: bool = False) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc()] + common_flags()
    if src.endswith(".hip"):
        cmd += ["-x", "hip", f"--offload-arch={ARCH}",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-fgpu-flush-denormals-to-zero", "-munsafe-fp-atomics"]
    else:
        cmd += ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: compile_one(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libqknr.so in-tree with hipcc for gfx950.

Every source is compiled for gfx950 only, with packed-fp32 instructions
disabled (the feature flag is device-side; hipcc's host pass warns that it
does not know it, which is harmless).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libqknr.so")
SOURCES = ["api.cpp", "plan.cpp", "qk_across_heads.hip", "qk_per_head.hip", "qk_split.hip", "permute.hip",
           "qkv_proj.hip", "kv_rmsnorm_rope_cache.hip",
           "kv_rmsnorm_rope_cache_f16.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _check_launch_stubs(lib: str) -> None:
    """Refuse a library that references a kernel's host launch stub without
    defining it. The host pass of a kernel template can fail to instantiate
    (for instance when a lambda in it calls a device-only function) without an
    error; the shared library then links with the stub undefined and fails
    only when it is loaded."""
    r = subprocess.run(["nm", "-u", lib], capture_output=True, text=True)
    if r.returncode != 0:
        return                                   # no nm: nothing to check with
    missing = [ln.split()[-1] for ln in r.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        os.remove(lib)
        raise RuntimeError("kernel launch stubs left undefined (host pass of the kernel failed): "
                           + ", ".join(missing))


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libqknr.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    _check_launch_stubs(tmp)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

"""Builds libattnqat.so (HIP C++ for gfx950) next to the Python package.

Usage: ``python nvfp4_fake_quantized_amd/csrc/build.py`` (run it by path: the
package itself loads the library on import) or ``build()``.
Each translation unit is compiled in parallel, then linked into one shared
library whose only exported symbols are the C ABI of include/attnqat.h.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libattnqat.so"
SOURCES = ["api.hip", "quant_kernels.hip", "fwd_kernel.hip", "fwd_out_kernel.hip", "bwd_kernels.hip", "dkdv_kernel.hip",
           "probe_kernels.hip", "probe_mix_kernels.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    # no packed-fp32 instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{HERE}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libattnqat.so)")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=(), out_dir: str | None = None) -> str:
    """Compiles every HIP source and links ``libattnqat.so`` into the package
    directory (or ``out_dir``); returns its path.  Always rebuilds.
    ``extra_flags`` are passed to every compile (e.g. -DATTNQAT_DQ_AHEAD=3)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), SOURCES))
    out = os.path.join(out_dir or PKG, LIB_NAME)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])

"""Build libattn71.so (HIP kernels for gfx950 + the C ABI) in place.

    python -m exact_attention_71_amd.build         # or build() from Python

Each source compiles to an object in parallel, then hipcc links the shared
library next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libattn71.so")
BUILD = os.path.join(HERE, "_build")

SOURCES = ["api.cpp", "fwd.hip", "bwd.hip", "bwd_dkdv.hip", "bwd_dq.hip", "bwd_dq_ds.hip", "varlen.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off: the compiler may not form v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPR form: avoids AGPR<->VGPR copies of live tiles
    # (long-lived accumulators are pinned to AGPRs by inline asm instead)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # fully unrolled hand-scheduled steps exceed the default #pragma unroll size
    # limit; a partial unroll would index register arrays dynamically
    "-mllvm", "-pragma-unroll-threshold=65536",
    # fp32 atomics as global_atomic_add_f32 (no compare-and-swap loops)
    "-munsafe-fp-atomics",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str, csrc: str = CSRC, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *FLAGS, *extra, "-I", os.path.join(HERE, "..", "include"), "-c",
           os.path.join(csrc, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False, csrc: str = CSRC, out: str = OUT, extra=()) -> str:
    """Compile every source in `csrc` and link `out` (defaults: this package)."""
    build_dir = BUILD if out == OUT else out + ".build"
    os.makedirs(build_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, csrc, build_dir, tuple(extra)), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

"""Build libpav2.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each source is compiled to an object in parallel, then linked into one shared
library next to this file.  ``python -m decode_attention_paged_v2_amd.build``
runs it from the command line.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpav2.so")
# phase 1's kernel variants are split by (query dtype, cache dtype) pair so they compile in parallel
PHASE1_PAIRS = ["f32_f32", "f16_f16", "bf16_bf16", "f32_fp8", "f16_fp8", "bf16_fp8"]
SOURCES = (["api.hip", "phase1.hip"] + [f"phase1_{p}.hip" for p in PHASE1_PAIRS] +
           [f"phase1_sparse_{p}.hip" for p in PHASE1_PAIRS] + ["phase2.hip", "check.hip", "cache.hip", "stream.hip", "prefix.hip"])
HEADERS = [os.path.join(CSRC, h) for h in ("pav2_internal.h", "phase1_kernel.h", "cache.h", "prefix.h")] + \
    [os.path.join(ROOT, "include", "pav2.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off; the kernels' fp32 work is scalar per lane
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, extra=(), build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile and link; ``extra`` adds hipcc flags (e.g. -DPAV2_PHASE1_WAVES=8)."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), max(1, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), SOURCES))
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + HEADERS
    return any(os.path.getmtime(s) > t for s in srcs if os.path.exists(s))


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])

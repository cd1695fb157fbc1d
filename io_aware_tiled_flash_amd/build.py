"""Build the gfx950 shared library `libflashattn.so` in-tree with hipcc.

    python -m io_aware_tiled_flash_amd.build        (or build() from Python)

The library holds the HIP kernels and the C ABI declared in include/flash_attn.h;
it links only the HIP runtime (no torch). Each source compiles to its own
object in parallel (the kernel files dominate the build time), then one hipcc
call links them.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libflashattn.so")
SOURCES = [os.path.join(CSRC, "fa_fwd_kernel.hip"), os.path.join(CSRC, "fa_fwd_fast.hip"),
           os.path.join(CSRC, "fa_merge.hip"), os.path.join(CSRC, "fa_bwd.hip"),
           os.path.join(CSRC, "fa_validate.cpp"), os.path.join(CSRC, "fa_api.cpp")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the gfx950 library)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # Keep the compiler from forming packed-fp32 VALU instructions.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-Wall", "-Wno-unused-command-line-argument",
    ]


def _run(cmd: list[str], verbose: bool):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd)}")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    cc = hipcc()
    jobs = jobs or min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in SOURCES]
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            futs = [ex.submit(_run, [cc, *flags(), "-c", s, "-o", o], verbose)
                    for s, o in zip(SOURCES, objs)]
            for f in futs:
                f.result()
        tmp = LIB + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libparallax.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m parallax_local_linear_amd.build          # compile in place

The library is written next to this file so that it travels with the source
tree.  Every HIP file is compiled with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libparallax.so")
SOURCES = ["api.hip", "prefill_bf16.hip", "prefill_f32.hip", "decode.hip", "backward.hip",
           "noalloc_scratch.hip"]
ARCH = os.environ.get("PLX_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
              shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: set ROCM_PATH")


def command(out: str = LIB):
    return [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", os.path.join(os.path.dirname(HERE), "include"),
            "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = True) -> str:
    """Compile every source into libparallax.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    t0 = time.time()
    res = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libparallax.so")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build()

"""Build libkamera.so in-tree for gfx950 with hipcc.

Usage: python -m position_invariant_kv_kamera_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libkamera.so"
SOURCES = [CSRC / "kamera_host.cpp", CSRC / "kamera_api.cpp", CSRC / "kamera_kernels.hip",
           CSRC / "kamera_noalloc.hip", CSRC / "kamera_compile.hip", CSRC / "kamera_attention.hip"]
ARCH = os.environ.get("KAMERA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 VALU ops (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, out: Path | None = None, defines: dict | None = None) -> Path:
    """Compile the library to `out` (default: the in-tree libkamera.so). `defines` sets the
    kernels' build-time knobs, e.g. {"KAMERA_PREFETCH_TILES": 3, "KAMERA_NONTEMPORAL": 0}."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    target = Path(out) if out else LIB
    tmp = target.with_suffix(f".so.tmp{os.getpid()}")
    macro = [f"-D{k}={v}" for k, v in (defines or {}).items()]
    cmd = [hipcc, *FLAGS, *macro, "-o", str(tmp), *map(str, SOURCES)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    print(build(verbose=True))

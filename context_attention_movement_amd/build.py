"""Build libcam.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

    python -m context_attention_movement_amd.build

Compiles every source under csrc/ with hipcc for gfx950 only.  Packed-FP32
instruction selection is disabled for device code; no fast-math, so fp32
denormals are kept.
"""

from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libcam.so"
SOURCES = ["cam_api.cpp", "thd_planner.cpp", "relayout.hip", "lse.hip", "proj.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return str(Path(rocm) / "bin" / "hipcc")


def build(out: Path | None = None, defines: list[str] | None = None, verbose: bool = False) -> Path:
    out = Path(out) if out else LIB
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-command-line-argument",
           "-I", str(PKG.parent / "include")]
    cmd += [f"-D{d}" for d in (defines or [])]
    cmd += ["-o", str(out) + ".tmp"] + [str(CSRC / s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    os.replace(str(out) + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libsparse_mla.so (the attention library) and libsmla_probe.so (the
benchmark's attainable-peak probe) in-tree with hipcc for gfx950.

    python -m sparse_top_mla_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SOURCES = [PKG / "csrc" / "sparse_mla.hip", PKG / "csrc" / "sparse_mla_bwd.hip",
           PKG / "csrc" / "block_sparse_fwd.hip"]
OUTPUT = PKG / "libsparse_mla.so"
PROBE_SOURCES = [PKG / "csrc" / "peak_probe.hip"]
PROBE_OUTPUT = PKG / "libsmla_probe.so"

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    f"-I{ROOT / 'include'}",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = Path(rocm) / "bin" / "hipcc"
    return str(path) if path.exists() else "hipcc"


def _compile(sources, output: Path, verbose: bool, extra=()) -> Path:
    tmp = output.with_suffix(".so.tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, *map(str, sources), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed")
    os.replace(tmp, output)
    return output


def build(verbose: bool = False, extra=()) -> Path:
    """Compiles both libraries; returns the attention library's path."""
    _compile(PROBE_SOURCES, PROBE_OUTPUT, verbose, extra)
    return _compile(SOURCES, OUTPUT, verbose, extra)


if __name__ == "__main__":
    print(build(verbose=True))

"""Build the gfx950 shared library ``libfa_mi355x.so`` in-tree with hipcc.

Usage: ``python -m exact_io_aware_09_amd.build [--verbose] [--resource-usage]``.
Cross-compiles without a GPU.  The library links only the HIP runtime.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG_DIR = Path(__file__).resolve().parent
REPO_DIR = PKG_DIR.parent
CSRC = PKG_DIR / "csrc"
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = PKG_DIR / LIB_NAME
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip", "fa_fp8.hip", "fa_f32.hip"]
ARCH = "gfx950"


def hipcc_path() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = Path(rocm) / "bin" / "hipcc"
    if cand.exists():
        return str(cand)
    found = shutil.which("hipcc")
    if not found:
        raise RuntimeError("hipcc not found (set ROCM_PATH)")
    return found


def compile_flags(resource_usage: bool = False):
    flags = [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        # packed fp32 VALU forms are disabled for all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        f"-I{REPO_DIR / 'include'}",
    ]
    if resource_usage:
        flags.append("-Rpass-analysis=kernel-resource-usage")
    return flags


def build(verbose: bool = False, resource_usage: bool = False) -> Path:
    """Compile every source into LIB_PATH (always rebuilds)."""
    srcs = [str(CSRC / s) for s in SOURCES]
    tmp = LIB_PATH.with_name(LIB_NAME + ".tmp")
    cmd = [hipcc_path(), *compile_flags(resource_usage), *srcs, "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = res.stdout + res.stderr
    # hipcc's host pass does not know the device-only feature; that note is noise
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose or resource_usage:
        print("\n".join(lines))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    a = ap.parse_args(argv)
    path = build(verbose=a.verbose, resource_usage=a.resource_usage)
    print(f"built {path}")


if __name__ == "__main__":
    main()

"""Build the gfx950 shared library ``libfa_mi355x.so`` in-tree with hipcc.

Usage: ``python -m exact_io_aware_09_amd.build [--verbose] [--resource-usage]
[--out PATH] [-D NAME=VALUE ...]``.  Cross-compiles without a GPU.  Every
unit is compiled to an object of its own (in parallel, under ``_build/``),
with the flags the unit needs, and the objects are linked into one library
that depends only on the HIP runtime.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG_DIR = Path(__file__).resolve().parent
REPO_DIR = PKG_DIR.parent
CSRC = PKG_DIR / "csrc"
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = PKG_DIR / LIB_NAME
BUILD_DIR = REPO_DIR / "_build"
ARCH = "gfx950"
# Matrix instructions with their accumulators in VGPRs: for the head-dim-256
# backward and FP8 units and the non-causal head-dim-128 backward, whose
# kernels run one wavefront per SIMD (see fa_bwd_d256.hip, fa_bwd_d128nc.hip;
# the head-dim-256 forward keeps its accumulator in AGPRs, fa_fwd_d256.hip).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# (unit, extra flags)
UNITS = [
    ("fa_api.hip", []),
    ("fa_fwd.hip", []),
    ("fa_fwd_d256.hip", []),
    ("fa_bwd.hip", []),
    ("fa_bwd_d256.hip", VGPR_FORM),
    ("fa_bwd_d128nc.hip", VGPR_FORM),
    ("fa_fp8.hip", []),
    ("fa_fp8_d256.hip", VGPR_FORM),
    ("fa_f32.hip", []),
    ("fa_sched.hip", []),
]
SOURCES = [u for u, _ in UNITS]


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
        # packed fp32 VALU forms are disabled for all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        f"-I{REPO_DIR / 'include'}",
    ]
    if resource_usage:
        flags.append("-Rpass-analysis=kernel-resource-usage")
    return flags


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature; that note is noise
    lines = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
    return res.returncode, lines


def build(verbose: bool = False, resource_usage: bool = False, out: Path | None = None,
          defines=()) -> Path:
    """Compile every unit and link them into ``out`` (default LIB_PATH); always rebuilds."""
    out = Path(out) if out is not None else LIB_PATH
    tag = out.stem
    objdir = BUILD_DIR / tag
    objdir.mkdir(parents=True, exist_ok=True)
    hipcc = hipcc_path()
    base = compile_flags(resource_usage) + [f"-D{d}" for d in defines]

    def compile_unit(unit):
        name, extra = unit
        obj = objdir / (Path(name).stem + ".o")
        rc, lines = _run([hipcc, *base, *extra, "-c", str(CSRC / name), "-o", str(obj)], verbose)
        return name, obj, rc, lines

    with ThreadPoolExecutor(max_workers=min(len(UNITS), os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_unit, UNITS))
    failed = False
    for name, _, rc, lines in results:
        if rc != 0:
            sys.stderr.write(f"--- {name}\n" + "\n".join(lines) + "\n")
            failed = True
        elif (verbose or resource_usage) and lines:
            print(f"--- {name}\n" + "\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = out.with_name(out.name + ".tmp")
    rc, lines = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC",
                      *[str(o) for _, o, _, _ in results], "-o", str(tmp)], verbose)
    if rc != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"link failed with exit code {rc}")
    os.replace(tmp, out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    ap.add_argument("--out", type=Path, default=None, help="library path (default: in the package)")
    ap.add_argument("-D", dest="defines", action="append", default=[],
                    help="preprocessor definition for every unit (launch-configuration sweeps)")
    a = ap.parse_args(argv)
    path = build(verbose=a.verbose, resource_usage=a.resource_usage, out=a.out, defines=a.defines)
    print(f"built {path}")


if __name__ == "__main__":
    main()

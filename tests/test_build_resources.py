"""Register budget of the one-wavefront-per-SIMD kernels (compile-only, no GPU).

The head-dim-256 kernels, and the non-causal head-dim-128 dK/dV kernels, run
one wavefront per SIMD; their speed depends on the matrix instructions
keeping their accumulators in VGPRs (the units fa_*_d256.hip and
fa_bwd_d128nc.hip are built that way) and on no register being spilled to
scratch memory.  This compiles those units for gfx950 with the compiler's
resource-usage remarks and checks their kernels: scratch 0 bytes per lane.
A toolchain or source change that brings spills back fails here.
"""
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_io_aware_09_amd import build as B

D256_UNITS = [(n, f) for n, f in B.UNITS if n.endswith("_d256.hip")]
D128NC_UNIT = [(n, f) for n, f in B.UNITS if n == "fa_bwd_d128nc.hip"]
FWD_UNIT = [(n, f) for n, f in B.UNITS if n == "fa_fwd.hip"]


def resource_remarks(name, extra):
    cmd = [B.hipcc_path(), *B.compile_flags(resource_usage=True), *extra, "--cuda-device-only",
           "-c", str(B.CSRC / name), "-o", "/dev/null"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1)] = int(m.group(2))
    return kernels


@pytest.mark.skipif(shutil.which("hipcc") is None and not (B.Path("/opt/rocm/bin/hipcc").exists()),
                    reason="hipcc not available")
def test_head_dim_256_kernels_do_not_spill():
    with ThreadPoolExecutor(max_workers=len(D256_UNITS)) as ex:
        results = list(ex.map(lambda u: (u[0], resource_remarks(*u)), D256_UNITS))
    for name, kernels in results:
        assert kernels, f"{name}: no kernels reported"
        for k, r in kernels.items():
            if "ILi256E" not in k:
                continue
            assert r.get("ScratchSize [bytes/lane]") == 0, f"{name}: {k} spills ({r})"
            assert r["VGPRs"] + r.get("AGPRs", 0) <= 512, f"{name}: {k} {r}"


@pytest.mark.skipif(shutil.which("hipcc") is None and not (B.Path("/opt/rocm/bin/hipcc").exists()),
                    reason="hipcc not available")
def test_head_dim_128_noncausal_unit():
    # the unit holds only non-causal kernels (its launcher refuses causal
    # problems); its dK/dV kernels -- plain, dropout and block-sparse -- and
    # its plain dQ kernel spill nothing; the dropout and block-sparse dQ keep
    # a few bytes (at most 32 per lane; not on a measured path)
    (name, extra), = D128NC_UNIT
    kernels = resource_remarks(name, extra)
    assert kernels, f"{name}: no kernels reported"
    dkdv = [k for k in kernels if "bwd_dkdv_bf16_kernelILi128E" in k]
    dq = [k for k in kernels if "bwd_dq_bf16_kernelILi128E" in k]
    assert len(dkdv) == 3 and len(dq) == 3, sorted(kernels)
    for k in dkdv + dq:
        # template arguments after the launch configuration: causal, sparse, dropout
        flags = re.search(r"ELb([01])ELb([01])ELb([01])E", k)
        assert flags and flags.group(1) == "0", f"causal kernel compiled in {name}: {k}"
        scratch = kernels[k].get("ScratchSize [bytes/lane]")
        if k in dq and "1" in (flags.group(2), flags.group(3)):
            assert scratch <= 32, f"{name}: {k} spills ({kernels[k]})"
        else:
            assert scratch == 0, f"{name}: {k} spills ({kernels[k]})"


@pytest.mark.skipif(shutil.which("hipcc") is None and not (B.Path("/opt/rocm/bin/hipcc").exists()),
                    reason="hipcc not available")
def test_head_dim_64_forward_kernels_fit_four_waves():
    # every head-dim-64 forward (plain, split, block-sparse, dropout; causal
    # or not) keeps four wavefronts per SIMD, and all but three without
    # scratch: the non-causal ones run the software-pipelined loop, whose
    # read-ahead is sized for that.  The causal long-row kernels (causal and
    # the last template flag set: pipelined loop left of the diagonal, plain
    # loop on it; plain, split and dropout) keep both loops' state and spill
    # a few bytes per lane; they are still the faster ones from N = 2048 on,
    # so they may use at most 40.
    (name, extra), = FWD_UNIT
    kernels = resource_remarks(name, extra)
    fwd = [k for k in kernels if "fwd_bf16_kernelILi64E" in k]
    assert len(fwd) >= 8, sorted(kernels)
    # template flags after OCC: CAUSAL, SPLIT, SPARSE, DROPOUT, and the last one
    longc = [k for k in fwd if re.search(r"ELb1ELb[01]ELb0ELb[01]ELb1E", k)]
    assert len(longc) == 3, fwd
    for k in fwd:
        r = kernels[k]
        limit = 40 if k in longc else 0
        assert r.get("ScratchSize [bytes/lane]") <= limit, f"{name}: {k} spills ({r})"
        assert r["VGPRs"] + r.get("AGPRs", 0) <= 128, f"{name}: {k} {r}"

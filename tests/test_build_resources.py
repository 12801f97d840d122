"""Register budget of the head-dim-256 kernels (compile-only, no GPU).

The head-dim-256 kernels run one wavefront per SIMD; their speed depends on
the matrix instructions keeping their accumulators in VGPRs (the units
fa_*_d256.hip are built that way) and on no register being spilled to
scratch memory.  This compiles those units for gfx950 with the compiler's
resource-usage remarks and checks every kernel in them: scratch 0 bytes per
lane.  A toolchain or source change that brings spills back fails here.
"""
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_io_aware_09_amd import build as B

D256_UNITS = [(n, f) for n, f in B.UNITS if n.endswith("_d256.hip")]


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

"""Host-side helpers of bench.py (no GPU): FLOP and pair counts of the measured workloads."""
import torch

import bench
from exact_io_aware_09_amd.workloads import WORKLOADS, Workload
from oracle import attention as A


def test_credited_flops_of_the_headline_workload():
    fwd, bwd = bench.credited_flops(WORKLOADS["gpt2_medium"])
    assert fwd == 4 * 64 * 16 * 1024 * 1024 * 64 // 2
    assert bwd == fwd * 5 // 2


def test_band_mask_pairs_equal_the_oracle_element_count():
    for N in (1, 130, 300, 1000):
        m = bench.band_mask(N)
        nb = -(-N // 128)
        assert m.shape == (nb, nb) and m.dtype == torch.int32
        for causal in (False, True):
            w = Workload("x", 2, 3, N, 64, torch.bfloat16, causal, 0.1, 0)
            vis = A.visible_from_blocks(m, N, 128)
            if causal:
                vis = vis & torch.ones(N, N, dtype=torch.bool).tril()
            assert bench.mask_pairs(w, m) == int(vis.sum()) * 6

"""IO / FLOP models against the counts printed in the CS324 Lecture 8 notes."""
import math

import pytest
import torch

from oracle import io_model as IO
from oracle import tiled as T
from tests.conftest import read_golden


def golden_rows(tag):
    return [r for r in read_golden("io_counts.txt") if r[0] == tag]


def kv(row):
    return {row[i]: row[i + 1] for i in range(0, len(row) - 1, 2)}


def test_exercise4_d64_ratio():
    r = golden_rows("ex4")[0]
    d, n, m = int(r[1]), int(r[2]), int(r[3])
    ratio = IO.standard_io(n, d) / IO.flash_io(n, d, m)
    assert round(ratio, 2) == float(kv(r[4:])["ratio"])


def test_exercise4_d128_exact_counts():
    r = golden_rows("ex4")[1]
    d, n, m = int(r[1]), int(r[2]), int(r[3])
    want = kv(r[4:])
    br, bc = T.block_sizes(m, d)
    assert (br, bc) == (int(want["br"]), int(want["bc"]))
    assert math.ceil(n / bc) == int(want["tc"])
    assert IO.standard_io(n, d) == int(want["standard"])
    assert IO.flash_io(n, d, m) == int(want["flash"])
    assert round(IO.standard_io(n, d) / IO.flash_io(n, d, m), 2) == float(want["ratio"])


def test_ratio_trend_small_and_large_n():
    # about 8x asymptotically at d = 64, only about 4x at small N (section 5.5)
    m = 98304
    small = IO.standard_io(512, 64) / IO.flash_io(512, 64, m)
    large = IO.standard_io(65536, 64) / IO.flash_io(65536, 64, m)
    assert 3.5 < small < 4.5
    assert 7.5 < large < 8.5
    # the leading coefficient: 32 d^2 / M N^2 against 11 N^2
    assert 11 / (32 * 64 * 64 / m) == pytest.approx(8.25)


def test_exercise1_qkt_intensity():
    r = golden_rows("ex1")[0]
    n, d = int(r[1]), int(r[2])
    want = kv(r[3:])
    flops, nbytes, inten = IO.intensity_qkt(n, d)
    assert flops == int(want["flops"]) and nbytes == int(want["bytes"])
    assert round(inten, 1) == float(want["intensity"])


def test_causal_forward_traffic_ratio():
    r = golden_rows("causal_blocks")[0]
    nblk = int(r[1])
    n, d = 256, 32
    blk = n // nblk
    causal = IO.flash_io_causal_forward(n, d, blk, blk)
    noncausal = sum(3 * blk * d + 4 * blk for _ in range(nblk * nblk)) + 3 * n * d + 2 * n
    assert round(causal / noncausal, 3) == float(r[4])


def test_p_matrix_size_exercise10():
    r = golden_rows("p_size")[0]
    heads, ctx, nbytes, want = (int(x) for x in r[1:])
    assert heads * ctx * ctx * nbytes == want


def test_recompute_flop_overhead():
    r = golden_rows("flop_ratio")[0]
    n, d = int(r[1]), int(r[2])
    extra = IO.matmul_flops_recompute(n, d) / IO.matmul_flops_standard(n, d) - 1
    assert round(extra, 2) == float(r[3])


@pytest.mark.parametrize("n", [256, 300, 1000])
@pytest.mark.parametrize("d", [16, 32])
def test_counted_tiled_io_equals_closed_form(n, d):
    """The counting tiled model and the closed form agree, ragged N included."""
    m = 4 * d * 40  # small on-chip size: B_c = 40, B_r = min(40, d)
    br, bc = T.block_sizes(m, d)
    g = torch.Generator().manual_seed(n + d)
    q, k, v, do = (torch.randn(n, d, generator=g, dtype=torch.float64) for _ in range(4))
    io = T.IOCount()
    o, mm, ll = T.forward_outer_kv(q, k, v, 0.3, False, br, bc, io)
    assert io.total == IO.flash_io(n, d, m, backward=False)
    T.backward_recompute(q, k, v, o, do, mm + torch.log(ll), 0.3, False, br, bc, io)
    assert io.total == IO.flash_io(n, d, m)


def test_credited_flops():
    fwd, bwd = IO.credited_flops(64, 16, 1024, 64, True)
    assert fwd == 4 * 64 * 16 * 1024 * 1024 * 64 // 2
    assert bwd == fwd * 5 // 2


@pytest.mark.parametrize("n,d,br,bc", [(256, 16, 64, 16), (200, 8, 64, 32), (97, 4, 32, 32),
                                        (130, 8, 128, 64), (64, 4, 64, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_second_version_traffic_model_counts_the_tiled_loop(n, d, br, bc, causal):
    # The lab-bench model ("FlashAttention and GPU memory", section 14) against
    # an independent count: the elements the Q-outer tiled forward actually
    # slices out of Q, K, V and writes to O, block by block.  K/V block widths
    # divide the query block, so a causal query block ending at row i1 reads
    # exactly the key rows [0, i1); N is ragged in several cases.
    g = torch.Generator().manual_seed(n * 131 + d)
    q, k, v = (torch.randn(n, d, generator=g, dtype=torch.float64) for _ in range(3))
    io = T.IOCount()
    T.forward_outer_q(q, k, v, 0.5, causal, br, bc, io=io)
    assert io.total == IO.second_version_uncached(n, d, br, causal=causal)
    # every visited (i, j) pair read its K and V blocks exactly once
    nq = -(-n // br)
    full = nq * (-(-n // bc))
    assert io.pairs == (full if not causal else
                        sum(-(-min(n, (i + 1) * br) // bc) for i in range(nq)))

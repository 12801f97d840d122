"""Pins of the dropout oracle: the generator, the draws and dropout attention.

The generator is checked against rocRAND's Philox4x32-10 (an independent
implementation of the same published algorithm, compiled here as a host
program from its header), its key increments against their closed forms, the
draws against uniformity and keep-rate statistics, and dropout attention
against plain attention (nothing dropped), its expectation over seeds, and
finite differences of the forward (the backward formulas).
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from oracle.attention import attention_forward_backward
from oracle.dropout import attention_forward_backward_dropout, draws, keep_masks, keep_threshold
from oracle.philox import MULT, WEYL, philox4x32_10

_HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
_ROCRAND_HDR = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"

# Host program: rocRAND's engine started at subsequence s, offset 4c returns
# the block of counter (c mod 2^32, c div 2^32, s mod 2^32, s div 2^32)
# under key (seed mod 2^32, seed div 2^32); the offset is a 64-bit count of
# words, so word 1 of the counter must stay below 2^30.
_ROCRAND_PROG = r"""
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    unsigned long long seed = ((unsigned long long)k1 << 32) | k0;
    unsigned long long sub = ((unsigned long long)c3 << 32) | c2;
    unsigned long long ctr = ((unsigned long long)c1 << 32) | c0;
    rocrand_device::philox4x32_10_engine e(seed, sub, 4ull * ctr);
    uint4 r = e.next4();
    printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    if not (shutil.which(_HIPCC) or os.path.exists(_HIPCC)) or not os.path.exists(_ROCRAND_HDR):
        pytest.skip("hipcc or the rocRAND headers are not available")
    d = tmp_path_factory.mktemp("rocrand")
    src, exe = d / "philox_ref.cpp", d / "philox_ref"
    src.write_text(_ROCRAND_PROG)
    res = subprocess.run([_HIPCC, "-x", "c++", "-O1", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                          str(src), "-o", str(exe)], capture_output=True, text=True, timeout=300)
    if res.returncode != 0:
        pytest.skip("could not build the rocRAND reference program: " + res.stderr[-300:])

    def run(ctr, key):
        rows = np.concatenate([ctr, key], axis=1).astype(np.uint64)
        text = "\n".join(" ".join(str(int(x)) for x in r) for r in rows) + "\n"
        out = subprocess.run([str(exe)], input=text, capture_output=True, text=True, check=True,
                             timeout=120).stdout
        return np.array([[int(x) for x in ln.split()] for ln in out.splitlines()], dtype=np.uint64)

    return run


def test_philox_matches_rocrand(rocrand_philox):
    rng = np.random.default_rng(11)
    ctr = rng.integers(0, 2**32, size=(200, 4), dtype=np.uint64)
    ctr[:, 1] >>= 2
    key = rng.integers(0, 2**32, size=(200, 2), dtype=np.uint64)
    # edge words: all zero, all ones, and the counters dropout uses
    ctr[:4] = [[0, 0, 0, 0], [2**32 - 1, 2**30 - 1, 2**32 - 1, 2**32 - 1], [5, 7, 3, 0],
               [16383, 16383, 2**31 - 1, 0]]
    key[:4] = [[0, 0], [2**32 - 1] * 2, [0x89ABCDEF, 0x01234567], [1, 0]]
    want = rocrand_philox(ctr, key)
    got = philox4x32_10(ctr, key).astype(np.uint64)
    np.testing.assert_array_equal(got, want)


def test_philox_weyl_increments_closed_form():
    # leading 32 fraction bits of the golden ratio and of sqrt(3) - 1
    golden = (math.isqrt(5 << 64) - (1 << 32)) // 2
    sqrt3m1 = math.isqrt(3 << 64) - (1 << 32)
    assert WEYL == (golden, sqrt3m1)
    assert all(m % 2 == 1 for m in MULT)  # odd multipliers: each round is a bijection


def test_philox_is_keyed_bijection_on_a_sample():
    # distinct counters give distinct blocks; the key changes every block
    ctr = np.stack([np.arange(4096), np.zeros(4096), np.zeros(4096), np.zeros(4096)], 1)
    a = philox4x32_10(ctr, [1, 2])
    b = philox4x32_10(ctr, [1, 3])
    assert len({tuple(r) for r in a}) == 4096
    assert not np.any(np.all(a == b, axis=1))


def test_draws_uniform_bytes_and_bits():
    idx = np.arange(1024)
    u = draws(0x5EED5EED5EED, 7, idx, idx).ravel()
    counts = np.bincount(u, minlength=256)
    exp = u.size / 256
    chi2 = ((counts - exp) ** 2 / exp).sum()
    # 255 degrees of freedom: mean 255, sd ~22.6; 7 sd either side
    assert 255 - 7 * 22.6 < chi2 < 255 + 7 * 22.6
    for bit in range(8):
        frac = ((u >> bit) & 1).mean()
        assert abs(frac - 0.5) < 7 * 0.5 / math.sqrt(u.size)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_rate(p):
    t = keep_threshold(p)
    z = keep_masks(2024, 1, 2, 512, t).numpy()
    rate, n = z.mean(), z.size
    want = t / 256
    assert abs(rate - want) < 6 * math.sqrt(want * (1 - want) / n)


def test_keep_threshold_values():
    assert keep_threshold(0.0) == 256
    assert keep_threshold(0.5) == 128
    assert keep_threshold(0.1) == 230      # (1 - 0.1) * 256 = 230.4
    assert keep_threshold(0.25) == 192
    assert keep_threshold(0.998) == 1      # 0.512 rounds to 1
    for bad in (-0.1, 1.0, 0.999):
        with pytest.raises(ValueError):
            keep_threshold(bad)


def test_draws_depend_only_on_element():
    full = draws(99, 3, np.arange(64), np.arange(64))
    rows, cols = np.array([63, 5, 17, 0]), np.array([2, 61, 30, 33, 7])
    np.testing.assert_array_equal(draws(99, 3, rows, cols), full[np.ix_(rows, cols)])
    assert not np.array_equal(draws(99, 4, np.arange(64), np.arange(64)), full)
    assert not np.array_equal(draws(100, 3, np.arange(64), np.arange(64)), full)
    assert not np.array_equal(draws(99 + (1 << 32), 3, np.arange(64), np.arange(64)), full)


def test_draws_element_by_element():
    # implementation check of the vectorised indexing: one block per element
    seed, bh = 0x0123456789ABCDEF, 5
    full = draws(seed, bh, np.arange(9), np.arange(11))
    for i in range(9):
        for j in range(11):
            blk = philox4x32_10([j // 4, i // 4, bh, 0], [seed & 0xFFFFFFFF, seed >> 32])
            assert full[i, j] == (int(blk[i % 4]) >> (8 * (j % 4))) & 0xFF


def _inputs(n, d, seed, heads=2):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(1, heads, n, d, generator=g, dtype=torch.float64) for _ in range(4)]


@pytest.mark.parametrize("causal", [False, True])
def test_nothing_dropped_is_attention(causal):
    q, k, v, do = _inputs(37, 8, 1)
    keep = keep_masks(7, 1, 2, 37, 256)
    assert bool(keep.all())
    got = attention_forward_backward_dropout(q, k, v, do, 0.3, causal, keep, 256)
    want = attention_forward_backward(q, k, v, do, 0.3, causal)
    for a, b in zip(got, want):
        torch.testing.assert_close(a, b, rtol=0, atol=1e-13)


def test_expectation_over_seeds_is_attention():
    # E[Z] * 256/t = 1 elementwise, so the mean output over many masks is P V
    q, k, v, do = _inputs(12, 4, 2, heads=1)
    t = keep_threshold(0.3)
    o_ref, _ = attention_forward_backward(q, k, v, do, 0.5, False)[:2]
    acc = torch.zeros_like(o_ref)
    n = 3000
    for s in range(n):
        acc += attention_forward_backward_dropout(q, k, v, do, 0.5, False, keep_masks(s, 1, 1, 12, t), t)[0]
    mean = acc / n
    # per-element sd of one sample is below max|V| * sqrt(p/(1-p)) * max P; 6 sd of the mean
    bound = 6 * float(v.abs().max()) * math.sqrt(0.3 / 0.7) / math.sqrt(n)
    assert float((mean - o_ref).abs().max()) < bound


@pytest.mark.parametrize("causal", [False, True])
def test_backward_is_gradient_of_forward(causal):
    # central differences of L = sum(dO * O) with the keep mask fixed
    q, k, v, do = (x[:, :1] for x in _inputs(6, 3, 3))
    t = keep_threshold(0.4)
    keep = keep_masks(31, 1, 1, 6, t)
    assert 0 < int(keep.sum()) < 36
    scale = 0.7
    _, _, dq, dk, dv = attention_forward_backward_dropout(q, k, v, do, scale, causal, keep, t)

    def loss(q_, k_, v_):
        o = attention_forward_backward_dropout(q_, k_, v_, do, scale, causal, keep, t)[0]
        return float((o * do).sum())

    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = torch.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args = [q.clone(), k.clone(), v.clone()]
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            num[idx] = (up - loss(*args)) / (2 * eps)
        torch.testing.assert_close(grad, num, rtol=1e-6, atol=1e-8)


def test_d_identity_with_dropout():
    # sum_j P_ij dP_ij = sum_k dO_ik O_ik: the backward's D needs only O, dO
    q, k, v, do = _inputs(20, 5, 4, heads=1)
    t = keep_threshold(0.2)
    keep = keep_masks(8, 1, 1, 20, t)
    o = attention_forward_backward_dropout(q, k, v, do, 0.4, True, keep, t)[0]
    from oracle.attention import scores, softmax_rows
    p = softmax_rows(scores(q, k, 0.4, True))[0]
    dp = (do @ v.transpose(-1, -2)) * keep.double() * (256.0 / t)
    torch.testing.assert_close((p * dp).sum(-1), (do * o).sum(-1), rtol=1e-12, atol=1e-12)

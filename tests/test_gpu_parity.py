"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Tolerances (max-abs unless stated):
  float32 inputs : O <= 1e-5, LSE <= 1e-5, dQ/dK/dV <= 1e-4
  bfloat16 inputs: O <= 2e-2, LSE <= 1e-3, dQ/dK/dV relative Frobenius <= 5e-2
The float32 LSE bound is derived (the target states none): LSE is a sum of a
max and a log of a float32 sum, |LSE| < 20 here, so float32 rounding leaves
it within a few 1e-6.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_09_amd as fa
from exact_io_aware_09_amd import _lib
from exact_io_aware_09_amd.workloads import WORKLOADS, make_inputs, sample_rows, workload_inputs
from oracle import attention as A
from oracle import sampled as SM

pytestmark = pytest.mark.gpu

TOL = {
    torch.float32: dict(o=1e-5, lse=1e-5, grad_abs=1e-4),
    torch.bfloat16: dict(o=2e-2, lse=1e-3, grad_relf=5e-2),
}


def dev():
    return torch.device("cuda:0")


def run_gpu(q, k, v, do, scale, causal):
    """fa_forward + fa_backward on cuda:0; CPU copies of (O, LSE, dQ, dK, dV)."""
    qd, kd, vd, dod = (t.to(dev()) for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, scale, causal)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, scale, causal)
    torch.cuda.synchronize()
    out = tuple(t.cpu() for t in (o, lse, dq, dk, dv))
    del qd, kd, vd, dod, o, lse, dq, dk, dv
    return out


def max_abs(a, b):
    return float((a.double() - b.double()).abs().max()) if a.numel() else 0.0


def rel_frob(a, b):
    num = float(torch.linalg.vector_norm(a.double() - b.double()))
    den = float(torch.linalg.vector_norm(b.double()))
    return num / den if den > 0 else num


def check(dtype, got, ref, what):
    """Compare GPU outputs with oracle outputs; `what` names the case."""
    tol = TOL[dtype]
    names = ("O", "LSE", "dQ", "dK", "dV")
    for name, g, r in zip(names, got, ref):
        if g is None:
            continue
        assert torch.isfinite(g.double()).all(), f"{what}: {name} not finite"
        if name == "O":
            err = max_abs(g, r)
            assert err <= tol["o"], f"{what}: O max-abs {err}"
        elif name == "LSE":
            err = max_abs(g, r)
            assert err <= tol["lse"], f"{what}: LSE max-abs {err}"
        elif dtype == torch.float32:
            err = max_abs(g, r)
            assert err <= tol["grad_abs"], f"{what}: {name} max-abs {err}"
        else:
            err = rel_frob(g, r)
            assert err <= tol["grad_relf"], f"{what}: {name} relF {err}"


def oracle_full(q, k, v, do, scale, causal, heads_per_chunk=16):
    return A.per_head(A.attention_forward_backward, (q, k, v, do), scale, causal,
                      heads_per_chunk=heads_per_chunk)


def full_case(shape, dtype, causal, seed, scale=None, mult=1.0):
    B, H, N, d = shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    q, k, v, do = make_inputs(shape, dtype, seed, mult)
    got = run_gpu(q, k, v, do, scale, causal)
    ref = oracle_full(q, k, v, do, scale, causal)
    check(dtype, got, ref, f"{shape} {dtype} causal={causal}")


# --------------------------------------------------------------------------
# small shapes: several tiles and ragged tails, full tensors
def test_tiny_workload_fp32():
    w = WORKLOADS["tiny"]
    q, k, v, do = workload_inputs(w)
    got = run_gpu(q, k, v, do, w.scale, w.causal)
    check(w.dtype, got, oracle_full(q, k, v, do, w.scale, w.causal), "tiny")


FP32_SHAPES = [(1, 1, 1, 64), (2, 3, 7, 64), (1, 2, 63, 64), (2, 1, 129, 128), (1, 1, 200, 256),
               (1, 2, 1000, 64), (1, 1, 300, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", FP32_SHAPES)
def test_fp32_shapes(shape, causal):
    full_case(shape, torch.float32, causal, seed=7 * sum(shape) + shape[3])


BF16_SHAPES = [(1, 1, 1, 64), (3, 5, 7, 64), (1, 2, 63, 64), (2, 2, 127, 64), (1, 3, 129, 64),
               (1, 2, 257, 64), (2, 1, 1000, 64), (1, 1, 513, 64),
               (1, 1, 1, 128), (1, 2, 65, 128), (2, 1, 300, 128), (1, 1, 1024, 128),
               (1, 1, 1, 256), (1, 2, 33, 256), (1, 1, 200, 256), (1, 1, 520, 256)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", BF16_SHAPES)
def test_bf16_shapes(shape, causal):
    full_case(shape, torch.bfloat16, causal, seed=sum(shape) + 17, mult=0.5 if shape[3] == 256 else 1.0)


# Causal rows long enough for the two-loop head-dim-64 forward (pipelined
# left of each query block's diagonal, plain on it; N >= 2048), with an odd
# and an even number of blocks before the diagonal and ragged tails.
@pytest.mark.parametrize("shape", [(1, 2, 2048, 64), (1, 1, 2100, 64), (1, 1, 3000, 64)])
def test_bf16_long_causal_rows(shape):
    full_case(shape, torch.bfloat16, True, seed=sum(shape) + 19, mult=1.0)


# No causal mask and N a multiple of the key-block size (32 keys at head dim
# 64, 64 at head dim 256): the forward's pipelined loop without mask code.
@pytest.mark.parametrize("shape", [(1, 2, 256, 64), (2, 1, 1024, 64), (1, 1, 512, 256), (1, 1, 1024, 256)])
def test_bf16_unmasked_blocks(shape):
    full_case(shape, torch.bfloat16, False, seed=sum(shape) + 23, mult=0.5 if shape[3] == 256 else 1.0)


# --------------------------------------------------------------------------
# GPT-2-medium attention shape, full tensors, checked 8 batches at a time
@pytest.fixture(scope="module")
def gpt2_run():
    w = WORKLOADS["gpt2_medium"]
    inp = workload_inputs(w)
    return w, inp, run_gpu(*inp, w.scale, w.causal)


@pytest.mark.parametrize("b0", list(range(0, 64, 8)))
def test_gpt2_medium_full(gpt2_run, b0):
    w, inp, got = gpt2_run
    sl = slice(b0, b0 + 8)
    ref = oracle_full(*(t[sl] for t in inp), w.scale, w.causal, heads_per_chunk=32)
    check(w.dtype, tuple(t[sl] for t in got), ref, f"gpt2_medium batches {b0}..{b0 + 7}")


# --------------------------------------------------------------------------
# memory-footprint shape, full tensors per head, batch-sliced
@pytest.fixture(scope="module")
def memory_run():
    w = WORKLOADS["memory"]
    inp = workload_inputs(w)
    return w, inp, run_gpu(*inp, w.scale, w.causal)


@pytest.mark.parametrize("b0", list(range(0, 16, 2)))
def test_memory_shape_full(memory_run, b0):
    w, inp, got = memory_run
    sl = slice(b0, b0 + 2)
    ref = oracle_full(*(t[sl] for t in inp), w.scale, w.causal, heads_per_chunk=2)
    check(w.dtype, tuple(t[sl] for t in got), ref, f"memory batches {b0}..{b0 + 1}")


# --------------------------------------------------------------------------
# sampled rows at the full long-sequence and large-head-dim shapes
def sampled_check(w, inp, got, b, h, keys: bool):
    q, k, v, do = (t[b, h] for t in inp)
    o, lse, dq, dk, dv = (t[b, h] for t in got)
    qi, ki = sample_rows(w.seed, b, h, w.H, w.N)
    ro, rl, rdq = SM.query_rows(q, k, v, do, qi, w.scale, w.causal)
    what = f"{w.name} b={b} h={h}"
    check(w.dtype, (o[qi], lse[qi], dq[qi], None, None), (ro, rl, rdq, None, None), what + " rows")
    if keys:
        rdk, rdv = SM.key_rows(q, k, v, do, ki, w.scale, w.causal, chunk=1024)
        check(w.dtype, (None, None, None, dk[ki], dv[ki]), (None, None, None, rdk, rdv),
              what + " key rows")


@pytest.fixture(scope="module")
def long_run():
    w = WORKLOADS["long"]
    inp = workload_inputs(w)
    return w, inp, run_gpu(*inp, w.scale, w.causal)


@pytest.mark.parametrize("h", list(range(8)))
def test_long_sequence_sampled(long_run, h):
    # query rows and key rows (dK, dV) on every head
    w, inp, got = long_run
    sampled_check(w, inp, got, 0, h, keys=True)


@pytest.fixture(scope="module")
def big_d_run():
    w = WORKLOADS["big_d"]
    inp = workload_inputs(w)
    return w, inp, run_gpu(*inp, w.scale, w.causal)


@pytest.mark.parametrize("bh", [(0, 0), (0, 5), (0, 7), (0, 12), (1, 0), (1, 3), (1, 9), (1, 15)])
def test_big_head_dim_sampled(big_d_run, bh):
    # query rows on 8 heads of both batches, key rows (dK, dV) on 4 of them
    w, inp, got = big_d_run
    b, h = bh
    sampled_check(w, inp, got, b, h, keys=bh in ((0, 0), (0, 12), (1, 3), (1, 15)))


# --------------------------------------------------------------------------
# properties of the GPU path itself
def test_bitwise_deterministic():
    w = WORKLOADS["gpt2_medium"]
    inp = make_inputs((8, 16, 1024, 64), torch.bfloat16, 11)
    a = run_gpu(*inp, w.scale, True)
    b = run_gpu(*inp, w.scale, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("shape,causal", [((1, 4, 4096, 64), True), ((1, 2, 2048, 256), False)])
def test_bitwise_deterministic_other_forward_loops(shape, causal):
    # the two-loop causal forward for long rows, the head-dim-256 forward
    # without mask code: the same bits on every run
    B, H, N, d = shape
    inp = make_inputs(shape, torch.bfloat16, 12, 0.5 if d == 256 else 1.0)
    a = run_gpu(*inp, d ** -0.5, causal)
    b = run_gpu(*inp, d ** -0.5, causal)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_causal_rows_ignore_future_on_gpu(dtype):
    q, k, v, do = make_inputs((2, 2, 700, 64), dtype, 21)
    i0 = 300
    k2, v2 = k.clone(), v.clone()
    k2[:, :, i0 + 1:] = -k2[:, :, i0 + 1:] * 3
    v2[:, :, i0 + 1:] = v2[:, :, i0 + 1:] + 5
    o1, l1, *_ = run_gpu(q, k, v, do, 0.125, True)
    o2, l2, *_ = run_gpu(q, k2, v2, do, 0.125, True)
    assert torch.equal(o1[:, :, : i0 + 1], o2[:, :, : i0 + 1])
    assert torch.equal(l1[:, :, : i0 + 1], l2[:, :, : i0 + 1])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_every_output_written_and_nothing_else(dtype, causal, d):
    """NaN-poisoned outputs are fully overwritten; guard bands stay intact."""
    B, H, N = 2, 3, 197
    q, k, v, do = (t.to(dev()) for t in make_inputs((B, H, N, d), dtype, 5, 0.5))
    G = 64  # guard elements on each side (keeps 16-byte alignment)
    n = B * H * N * d

    def guarded(numel, dt):
        buf = torch.full((numel + 2 * G,), float("nan"), dtype=dt, device=dev())
        buf[:G] = 7.0
        buf[-G:] = 7.0
        return buf

    ob, lb = guarded(n, dtype), guarded(B * H * N, torch.float32)
    o = ob[G:G + n].view(B, H, N, d)
    lse = lb[G:G + B * H * N].view(B, H, N)
    fa.forward(q, k, v, 0.1, causal, out=o, lse=lse)
    grads = [guarded(n, dtype) for _ in range(3)]
    views = [g[G:G + n].view(B, H, N, d) for g in grads]
    wsb = fa.workspace_bytes(B, H, N, d, dtype)
    ws = torch.full((wsb + 512,), 255, dtype=torch.uint8, device=dev())
    fa.backward(q, k, v, o, do, lse, 0.1, causal, workspace=ws[256:256 + wsb], dq=views[0],
                dk=views[1], dv=views[2])
    torch.cuda.synchronize()
    for buf in (ob, lb, *grads):
        inner = buf[G:-G]
        assert not torch.isnan(inner.float()).any()
        assert (buf[:G].float() == 7.0).all() and (buf[-G:].float() == 7.0).all()
    assert (ws[:256] == 255).all() and (ws[256 + wsb:] == 255).all()


def test_non_default_stream_gives_identical_results():
    q, k, v, do = (t.to(dev()) for t in make_inputs((2, 4, 333, 64), torch.bfloat16, 8))
    o1, l1 = fa.forward(q, k, v, 0.125, True)
    g1 = fa.backward(q, k, v, o1, do, l1, 0.125, True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o2, l2 = fa.forward(q, k, v, 0.125, True)
        g2 = fa.backward(q, k, v, o2, do, l2, 0.125, True)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_errors_reported_before_launch_on_device_pointers():
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device=dev())
    o = torch.full_like(q, 3.0)
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device=dev())
    rc = _lib.fa_forward(q.data_ptr() + 2, q.data_ptr(), q.data_ptr(), o.data_ptr(),
                         lse.data_ptr(), 1, 1, 64, 64, 0.125, 0, _lib.FA_BF16, None)
    assert rc == _lib.FA_ERR_MISALIGNED
    rc = _lib.fa_forward(q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(),
                         lse.data_ptr(), 1, 1, 64, 96, 0.125, 0, _lib.FA_BF16, None)
    assert rc == _lib.FA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (o == 3.0).all()  # nothing was launched
    with pytest.raises(fa.FAError):
        fa.forward(q, q, q, -1.0, False)


def test_long_sequence_allocates_nothing_quadratic():
    """At N = 65,536 the library adds no device memory beyond caller buffers."""
    w = WORKLOADS["long"]
    q, k, v, do = (t.to(dev()) for t in make_inputs(w.shape, w.dtype, 99))
    o = torch.empty_like(q)
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device=dev())
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.workspace_bytes(*w.shape, w.dtype), dtype=torch.uint8, device=dev())
    fa.forward(q, k, v, w.scale, True, out=o, lse=lse)  # warm-up: code objects loaded
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    free0, _ = torch.cuda.mem_get_info()
    base = torch.cuda.memory_allocated()
    fa.forward(q, k, v, w.scale, True, out=o, lse=lse)
    fa.backward(q, k, v, o, do, lse, w.scale, True, workspace=ws, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.max_memory_allocated() == base
    assert free0 - free1 < 64 << 20  # device-level: far below one N x N bf16 buffer (8 GiB)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_stage_calls_reproduce_fa_backward(dtype, d):
    """fa_backward_dq then fa_backward_dkdv == fa_backward, bit for bit; the
    standalone D preprocess agrees with the D that the dQ stage leaves."""
    B, H, N, scale = 2, 3, 301, 0.11
    q, k, v, do = (t.to(dev()) for t in make_inputs((B, H, N, d), dtype, 31))
    o, lse = fa.forward(q, k, v, scale, True)
    dq1, dk1, dv1 = fa.backward(q, k, v, o, do, lse, scale, True)
    dt = _lib.FA_BF16 if dtype == torch.bfloat16 else _lib.FA_F32
    wsb = fa.workspace_bytes(B, H, N, d, dtype)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev())
    dq2, dk2, dv2 = (torch.full_like(q, float("nan")) for _ in range(3))
    sp = torch.cuda.current_stream().cuda_stream
    rc = _lib.fa_backward_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                             lse.data_ptr(), ws.data_ptr(), wsb, dq2.data_ptr(), B, H, N, d, scale,
                             1, dt, sp)
    assert rc == _lib.FA_OK
    rows = B * H * N
    loff = 4 * ((rows + 63) // 64 * 64)  # LSE * log2(e) starts on a 256-byte boundary
    d_from_dq = ws[: 4 * rows].view(torch.float32).clone()
    l_from_dq = ws[loff: loff + 4 * rows].view(torch.float32).clone()
    rc = _lib.fa_backward_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                               ws.data_ptr(), wsb, dk2.data_ptr(), dv2.data_ptr(), B, H, N, d,
                               scale, 1, dt, sp)
    assert rc == _lib.FA_OK
    for a, b in ((dq1, dq2), (dk1, dk2), (dv1, dv2)):
        assert torch.equal(a, b)
    # the standalone preprocess fills the same workspace; dK/dV from it agree
    ws.fill_(255)
    rc = _lib.fa_backward_preprocess(o.data_ptr(), do.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                                     wsb, B, H, N, d, dt, sp)
    assert rc == _lib.FA_OK
    d_pre = ws[: 4 * rows].view(torch.float32).clone()
    l_pre = ws[loff: loff + 4 * rows].view(torch.float32).clone()
    dk3, dv3 = torch.empty_like(q), torch.empty_like(q)
    rc = _lib.fa_backward_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                               ws.data_ptr(), wsb, dk3.data_ptr(), dv3.data_ptr(), B, H, N, d,
                               scale, 1, dt, sp)
    assert rc == _lib.FA_OK
    torch.cuda.synchronize()
    ref = (o.double() * do.double()).sum(-1).flatten().cpu()
    lref = (lse.double() * math.log2(math.e)).flatten().cpu()
    assert max_abs(d_pre.cpu(), -ref) < 1e-4  # the workspace holds -D
    assert max_abs(d_from_dq.cpu(), -ref) < 1e-4
    assert max_abs(l_pre.cpu(), lref) < 1e-5 and max_abs(l_from_dq.cpu(), lref) < 1e-5
    assert torch.equal(dv3, dv1)  # dV does not depend on D
    assert rel_frob(dk3.cpu(), dk1.cpu()) < 1e-3

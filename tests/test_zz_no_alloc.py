"""fa_backward_noalloc (workspace in the library's device scratch) through the C ABI.

Two calls in a row on one GPU -- the second smaller, with another head dim
and mask -- each compared with fa_backward on its own workspace: the same
kernels run, so dQ, dK and dV must agree bit for bit.  Then a problem larger
than the scratch is refused before anything is enqueued.
"""
import pytest
import torch

from exact_io_aware_09_amd import _lib
from exact_io_aware_09_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu


def _run(shape, dtype, causal, seed):
    dev = torch.device("cuda:0")
    B, H, N, d = shape
    dt = _lib.FA_BF16 if dtype == torch.bfloat16 else _lib.FA_F32
    scale = d ** -0.5
    q, k, v, do = (t.to(dev) for t in make_inputs(shape, dtype, seed))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    sp = torch.cuda.current_stream(dev).cuda_stream
    assert _lib.fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           B, H, N, d, scale, int(causal), dt, sp) == _lib.FA_OK
    ref = [torch.full_like(q, float("nan")) for _ in range(3)]
    wsb = _lib.fa_backward_workspace_bytes(B, H, N, d, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    assert _lib.fa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                            lse.data_ptr(), *(t.data_ptr() for t in ref), ws.data_ptr(), wsb,
                            B, H, N, d, scale, int(causal), dt, sp) == _lib.FA_OK
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    assert _lib.fa_backward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    do.data_ptr(), lse.data_ptr(), *(t.data_ptr() for t in got),
                                    B, H, N, d, scale, int(causal), dt, sp) == _lib.FA_OK
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(g.float()).all(), name
        assert torch.equal(g, r), f"{name} differs from fa_backward"


def test_noalloc_matches_fa_backward_on_two_calls():
    _run((2, 4, 1000, 64), torch.bfloat16, True, 31)    # 8000 rows
    _run((1, 3, 257, 128), torch.bfloat16, False, 32)   # smaller, other head dim and mask


def test_noalloc_fp32_and_largest_headline_size():
    _run((1, 1, 128, 64), torch.float32, False, 33)
    # the GPT-2-medium row count (B 64 x H 16 x N 1024) fits the scratch
    B, H, N, d = 64, 16, 1024, 64
    assert _lib.fa_backward_workspace_bytes(B, H, N, d, _lib.FA_BF16) <= 16 << 20


def test_noalloc_refuses_more_rows_than_the_scratch_holds():
    dev = torch.device("cuda:0")
    x = torch.zeros(16, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(16, dtype=torch.float32, device=dev)
    p = x.data_ptr()
    sp = torch.cuda.current_stream(dev).cuda_stream
    rc = _lib.fa_backward_noalloc(p, p, p, p, p, lse.data_ptr(), p, p, p, 64, 16, 4096, 64,
                                  0.125, 1, _lib.FA_BF16, sp)
    assert rc == _lib.FA_ERR_NO_WORKSPACE

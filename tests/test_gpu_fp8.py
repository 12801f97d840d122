"""GPU parity of the FP8 forward (fa_quantize_fp8, fa_forward_fp8).

* Quantiser: E4M3 codes and block exponent bytes bit for bit against the
  oracle's block quantisation (integer and byte results: exact), for both
  layouts, with ragged N (padded keys), all-zero blocks and blocks whose
  magnitudes differ by many binades.
* Forward: O and LSE against the oracle's attention of the dequantised
  inputs.  Two roundings separate the kernel from that definition, and the
  bounds are derived from them.  (1) The FP8 matrix instruction accumulates
  a 64-term dot product with about 13 bits: measured on the instruction
  itself, its error stays below 2^-12 of the sum of the absolute products,
  so a row's scores carry |dS_ij| <= delta_i = 2^-12 scale max_j sum_k
  |Q^_ik| |K^_jk|.  (2) The weights (times 2^8) are rounded to E4M3 before the
  product with V: 2^-4 relative for normal values, 2^-18 absolute (in units
  of the row's largest weight) for subnormal ones.  Elementwise:
    |O - O^| <= (2^-4 + 1e-3 + 3 delta_i) (P |V^|) + 2^-18 sum_j |V^_j|
                + 2^-8 |O^| + 1e-5      (2^-8: O's bfloat16 rounding)
    |LSE - LSE^| <= 2e-3 + delta_i.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_09_amd as fa
from exact_io_aware_09_amd.workloads import WORKLOADS, make_inputs, sample_rows
from oracle import fp8 as F8
from oracle.attention import scores, softmax_rows

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda:0")


def spread(x, seed):
    # per-row magnitudes over 2^-12 .. 2^4, one all-zero row
    g = torch.Generator().manual_seed(seed)
    e = torch.randint(-12, 5, x.shape[:-1] + (1,), generator=g).to(torch.float32)
    y = (x.float() * torch.exp2(e)).to(torch.bfloat16)
    rows = y.view(-1, x.shape[-1])
    rows[rows.shape[0] // 2] = 0
    return y


@pytest.mark.parametrize("shape", [(1, 2, 77, 64), (2, 1, 130, 128), (1, 1, 200, 256), (1, 1, 1, 64)])
def test_quantiser_codes_and_exponents_exact(shape):
    x = spread(make_inputs(shape, torch.bfloat16, 11)[0], 12)
    x8, xs = fa.quantize_fp8(x.to(dev()))
    v8, vs = fa.quantize_fp8(x.to(dev()), keys=True)
    torch.cuda.synchronize()
    codes, e, _ = F8.quantize_rows(x.double().numpy())
    np.testing.assert_array_equal(x8.cpu().numpy(), codes)
    N = shape[2]
    np.testing.assert_array_equal(xs.cpu().numpy()[:, :, :N].astype(np.int64), e + 127)
    assert bool((xs.cpu()[:, :, N:] == 127).all())   # padding rows: exponent 0
    vcodes, ve, _ = F8.quantize_keys(x.double().numpy())
    np.testing.assert_array_equal(v8.cpu().numpy(), vcodes)
    np.testing.assert_array_equal(vs.cpu().numpy().astype(np.int64), ve + 127)


def run_fp8(q, k, v, scale, causal):
    qd, kd, vd = (t.to(dev()) for t in (q, k, v))
    q8, qs = fa.quantize_fp8(qd)
    k8, ks = fa.quantize_fp8(kd)
    v8, vs = fa.quantize_fp8(vd, keys=True)
    o, lse = fa.forward_fp8(q8, qs, k8, ks, v8, vs, scale, causal)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check_head(o, lse, qh, kh, vh, scale, causal, rows, what):
    """o [len(rows), d], lse [len(rows)] of one head against the oracle."""
    qd = torch.from_numpy(F8.quantize_rows(qh.double().numpy())[2])
    kd = torch.from_numpy(F8.quantize_rows(kh.double().numpy())[2])
    vd = torch.from_numpy(F8.quantize_keys(vh.double().numpy())[2])
    rows = torch.as_tensor(rows, dtype=torch.long)
    s = scale * (qd[rows] @ kd.T)
    if causal:
        s = s.masked_fill(torch.arange(kd.shape[0]).unsqueeze(0) > rows.unsqueeze(1), float("-inf"))
    p, m, l = softmax_rows(s)
    ro, rl = p @ vd, m + torch.log(l)
    delta = 2.0 ** -12 * scale * (qd[rows].abs() @ kd.abs().T).max(dim=1).values
    bound = ((2.0 ** -4 + 1e-3 + 3 * delta).unsqueeze(1) * (p @ vd.abs()) + 2.0 ** -18 * vd.abs().sum(0)
             + 2.0 ** -8 * ro.abs() + 1e-5)
    err = (o.double() - ro).abs()
    worst = float((err / bound).max())
    assert worst <= 1.0, f"{what}: O error {float(err.max()):.3e}, {worst:.2f} of the bound"
    lerr = (lse.double() - rl).abs()
    assert bool((lerr <= 2e-3 + delta).all()), f"{what}: LSE error {float(lerr.max()):.3e}"


# head dim 256, N a multiple of 64, no causal mask: the kernel without mask
# code (1, 1, 256, 256); the others keep it
CASES = [((1, 2, 200, 64), 3), ((2, 1, 130, 128), 4), ((1, 1, 77, 256), 5), ((1, 2, 333, 64), 6),
         ((1, 1, 1, 64), 7), ((1, 2, 64, 128), 8), ((1, 1, 256, 256), 9)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape,seed", CASES)
def test_forward_fp8_matches_oracle(shape, seed, causal):
    B, H, N, d = shape
    q, k, v = make_inputs(shape, torch.bfloat16, seed)[:3]
    scale = d ** -0.5
    o, lse = run_fp8(q, k, v, scale, causal)
    for b in range(B):
        for h in range(H):
            check_head(o[b, h], lse[b, h], q[b, h], k[b, h], v[b, h], scale, causal, np.arange(N),
                       f"{shape} causal={causal} head ({b},{h})")


@pytest.mark.parametrize("x", [1.5, 1.625, 3.0])
def test_forward_fp8_running_maximum_lag(x):
    # One 64-key block with score 1 at key 0, the next with score x at key
    # 64, every other score 0 (scale 1): in log2 units the second block's
    # maximum exceeds the first by 1.4427 (x - 1) = 0.72, 0.90 or 2.89.  The
    # kernel raises its running maximum only past a 0.75 lag, so at 0.72 the
    # key-64 weight is 2^8.72 = 422 (E4M3 holds 448) and at 0.90 and 2.89 the
    # row rescales; a lag above 0.807 would overflow E4M3 at 0.90.  All values
    # are exact in E4M3, so quantisation is exact.
    N, d = 128, 64
    q = torch.zeros(1, 1, N, d)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, N, d)
    k[0, 0, 0, 0] = 1.0
    k[0, 0, 64, 0] = x
    v = make_inputs((1, 1, N, d), torch.bfloat16, 31)[2]
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    o, lse = run_fp8(q, k, v, 1.0, False)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    check_head(o[0, 0], lse[0, 0], q[0, 0], k[0, 0], v[0, 0], 1.0, False, np.arange(N), f"x={x}")


def test_forward_fp8_spread_magnitudes():
    # per-row magnitudes over 16 binades: every block uses its own exponent
    shape = (1, 2, 256, 64)
    q, k, v = (spread(t, 20 + i) for i, t in enumerate(make_inputs(shape, torch.bfloat16, 13)[:3]))
    o, lse = run_fp8(q, k, v, 0.125, False)
    for h in range(2):
        check_head(o[0, h], lse[0, h], q[0, h], k[0, h], v[0, h], 0.125, False, np.arange(256), f"head {h}")


@pytest.mark.parametrize("name", ["gpt2_medium", "big_d"])
def test_forward_fp8_workload_shapes(name):
    w = WORKLOADS[name]
    B, H, N, d = w.shape
    q, k, v = make_inputs(w.shape, torch.bfloat16, w.seed, w.mult)[:3]
    o, lse = run_fp8(q, k, v, w.scale, w.causal)
    for b, h in ((0, 0), (B - 1, H - 1)):
        rows = np.arange(N) if N <= 1024 else sample_rows(w.seed, b, h, H, N)[0]
        check_head(o[b, h][rows], lse[b, h][rows], q[b, h], k[b, h], v[b, h], w.scale, w.causal, rows,
                   f"{name} head ({b},{h})")


def test_forward_fp8_long_causal_sampled():
    # N = 65,536, causal: 1,024 key blocks per row; sampled rows of two heads
    w = WORKLOADS["long"]
    B, H, N, d = w.shape
    q, k, v = make_inputs(w.shape, torch.bfloat16, w.seed)[:3]
    o, lse = run_fp8(q, k, v, w.scale, True)
    for h in (0, H - 1):
        rows = np.unique(np.concatenate([sample_rows(w.seed, 0, h, H, N, count=32)[0][:32], [0, N - 1]]))
        check_head(o[0, h][rows], lse[0, h][rows], q[0, h], k[0, h], v[0, h], w.scale, True, rows,
                   f"long head {h}")


def test_forward_fp8_bitwise_deterministic():
    shape = (2, 2, 300, 128)
    q, k, v = make_inputs(shape, torch.bfloat16, 14)[:3]
    a = run_fp8(q, k, v, 0.1, True)
    b = run_fp8(q, k, v, 0.1, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("N", [31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257])
def test_forward_fp8_tile_boundaries(N):
    # sequence lengths around the 64-key blocks, the 128-row workgroups and
    # the 32-element scale blocks of V; causal, d = 128
    shape = (1, 1, N, 128)
    q, k, v = make_inputs(shape, torch.bfloat16, 200 + N)[:3]
    o, lse = run_fp8(q, k, v, 128 ** -0.5, True)
    check_head(o[0, 0], lse[0, 0], q[0, 0], k[0, 0], v[0, 0], 128 ** -0.5, True, np.arange(N), f"N={N}")

"""GPU parity of attention with dropout (fa_forward_dropout / fa_backward_dropout).

* The keep masks themselves, bit for bit: with Q = 0 every visible weight is
  1/(row length) and with V = I (d = N) the output row is the row's mask
  times 256/t / length, so O > 0 exactly where the forward kept the pair; with
  dO = I, dV > 0 exactly where the dK/dV kernel kept it.  Both are compared
  with the oracle's draws (8-bit integer decisions: exact).
* Values against the oracle's dropout attention (fp64, the oracle's mask) at
  the bfloat16 tolerances of the dense path (LSE <= 1e-3 max-abs, dQ/dK/dV
  relative Frobenius <= 5e-2), and O element by element within the bound of
  its roundings: every kept weight is rounded to bfloat16 before P V
  (relative 2^-9) and O itself is rounded to bfloat16 (relative 2^-9), so
  |O - O_ref| <= 2^-8 (A + |O_ref|) + 1e-6 with A = (256/t) sum_j Z P |V|
  (a factor 2 of slack for the fp32 sums); full tensors on small ragged
  shapes, and whole heads at the causal GPT-2-medium shape.
* p_drop = 0 reproduces fa_forward / fa_backward bit for bit.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_09_amd as fa
from exact_io_aware_09_amd.workloads import make_inputs
from oracle import attention as OA
from oracle import dropout as DR

pytestmark = pytest.mark.gpu


def dev():
    return torch.device("cuda:0")


def max_abs(a, b):
    return float((a.double() - b.double()).abs().max()) if a.numel() else 0.0


def rel_frob(a, b):
    den = float(torch.linalg.vector_norm(b.double()))
    num = float(torch.linalg.vector_norm(a.double() - b.double()))
    return num / den if den > 0 else num


def check_o(o, ro, q, k, v, scale, causal, keep, t, what):
    """Element-wise bound on O from its roundings (module docstring)."""
    pr, _, _ = OA.softmax_rows(OA.scores(q, k, scale, causal))
    a = (pr * (torch.as_tensor(keep).double() * (256.0 / t))) @ v.double().abs()
    err = (o.double() - ro.double()).abs()
    bound = 2.0 ** -8 * (a + ro.double().abs()) + 1e-6
    worst = float((err / bound).max()) if err.numel() else 0.0
    assert worst <= 1.0, f"{what}: O error reaches {worst:.3f} of its rounding bound"


def run_dropout(q, k, v, do, scale, causal, p, seed):
    qd, kd, vd, dod = (t.to(dev()) for t in (q, k, v, do))
    o, lse = fa.forward_dropout(qd, kd, vd, scale, causal, p, seed)
    dq, dk, dv = fa.backward_dropout(qd, kd, vd, o, dod, lse, scale, causal, p, seed)
    torch.cuda.synchronize()
    return tuple(t.cpu() for t in (o, lse, dq, dk, dv))


@pytest.mark.parametrize("p", [0.3, 0.998])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_masks_are_the_oracle_draws(d, causal, p):
    # N = d so that V = I and dO = I read the masks out; B*H = 6 heads.
    # p = 0.998 is the largest p with t >= 1 (one draw value in 256 kept).
    B, H, N = 2, 3, d
    seed = 0x0123456789ABCDEF
    t = DR.keep_threshold(p)
    eye = torch.eye(N, dtype=torch.bfloat16).expand(B, H, N, N).contiguous()
    zero = torch.zeros(B, H, N, d, dtype=torch.bfloat16)
    o, lse, dq, dk, dv = run_dropout(zero, zero, eye, eye, 0.125, causal, p, seed)
    z = DR.keep_masks(seed, B, H, N, t)
    vis = torch.ones(N, N, dtype=torch.bool)
    if causal:
        vis = vis.tril()
    want = z & vis
    assert torch.equal(o.float() > 0, want), "forward keep mask"
    assert torch.equal(dv.float() > 0, want.transpose(-1, -2)), "dK/dV keep mask"
    assert float(dk.float().abs().max()) == 0.0  # Q = 0


CASES = [((1, 2, 200, 64), 0.1, 3), ((2, 1, 130, 128), 0.5, 4), ((1, 1, 77, 256), 0.25, 5),
         ((1, 2, 333, 64), 0.9, 6), ((1, 1, 1, 64), 0.2, 7)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape,p,seed", CASES)
def test_dropout_matches_oracle(shape, p, seed, causal):
    B, H, N, d = shape
    q, k, v, do = make_inputs(shape, torch.bfloat16, seed)
    scale = d ** -0.5
    rng_seed = (seed << 40) | 0xBEEF
    got = run_dropout(q, k, v, do, scale, causal, p, rng_seed)
    t = DR.keep_threshold(p)
    keep = DR.keep_masks(rng_seed, B, H, N, t)
    ref = DR.attention_forward_backward_dropout(q, k, v, do, scale, causal, keep, t)
    o, lse, dq, dk, dv = got
    ro, rl, rdq, rdk, rdv = ref
    what = f"{shape} p={p} causal={causal}"
    check_o(o, ro, q, k, v, scale, causal, keep, t, what)
    assert max_abs(lse, rl) <= 1e-3, f"{what}: LSE {max_abs(lse, rl)}"
    for name, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert rel_frob(g, r) <= 5e-2, f"{what}: {name} relF {rel_frob(g, r)}"


def test_headline_shape_whole_heads():
    # causal GPT-2-medium shape with dropout 0.1; whole heads checked
    B, H, N, d = 64, 16, 1024, 64
    q, k, v, do = make_inputs((B, H, N, d), torch.bfloat16, 1)
    p, seed = 0.1, 2024
    o, lse, dq, dk, dv = run_dropout(q, k, v, do, 0.125, True, p, seed)
    t = DR.keep_threshold(p)
    idx = torch.arange(N).numpy()
    for b, h in ((0, 0), (17, 9), (63, 15)):
        keep = torch.from_numpy(DR.draws(seed, b * H + h, idx, idx) < t)
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = DR.attention_forward_backward_dropout(q[sl], k[sl], v[sl], do[sl], 0.125, True, keep, t)
        check_o(o[sl], ref[0], q[sl], k[sl], v[sl], 0.125, True, keep, t, f"({b},{h})")
        assert max_abs(lse[sl], ref[1]) <= 1e-3, f"({b},{h}) LSE {max_abs(lse[sl], ref[1])}"
        for name, g, r in (("dQ", dq, ref[2]), ("dK", dk, ref[3]), ("dV", dv, ref[4])):
            assert rel_frob(g[sl], r) <= 5e-2, f"({b},{h}) {name} relF {rel_frob(g[sl], r)}"


@pytest.mark.parametrize("causal", [False, True])
def test_p0_is_plain_attention_bitwise(causal):
    shape = (2, 2, 300, 64)
    q, k, v, do = (t.to(dev()) for t in make_inputs(shape, torch.bfloat16, 9))
    o0, l0 = fa.forward(q, k, v, 0.125, causal)
    g0 = fa.backward(q, k, v, o0, do, l0, 0.125, causal)
    o1, l1 = fa.forward_dropout(q, k, v, 0.125, causal, 0.0, 12345)
    g1 = fa.backward_dropout(q, k, v, o1, do, l1, 0.125, causal, 0.0, 12345)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


def test_same_seed_same_result_and_seed_matters():
    shape = (1, 4, 256, 64)
    q, k, v, do = (t.to(dev()) for t in make_inputs(shape, torch.bfloat16, 10))
    a = fa.forward_dropout(q, k, v, 0.125, False, 0.2, 77)[0]
    b = fa.forward_dropout(q, k, v, 0.125, False, 0.2, 77)[0]
    c = fa.forward_dropout(q, k, v, 0.125, False, 0.2, 78)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, c)


def test_long_sequence_sampled_rows():
    # N = 65,536 causal: counters reach query and key tiles up to 16,383; O, LSE
    # and dQ of sampled query rows against the oracle (full rows, the mask drawn
    # for exactly those rows)
    from oracle.attention import scores, softmax_rows
    from exact_io_aware_09_amd.workloads import WORKLOADS, sample_rows
    w = WORKLOADS["long"]
    B, H, N, d = w.shape
    q, k, v, do = make_inputs(w.shape, torch.bfloat16, w.seed)
    p, seed = 0.1, 0xFEEDFACE12345
    o, lse, dq, dk, dv = run_dropout(q, k, v, do, w.scale, True, p, seed)
    t = DR.keep_threshold(p)
    for h in (0, H - 1):
        rows = np.unique(np.concatenate([sample_rows(w.seed, 0, h, H, N, count=24)[0][:24], [N - 1]]))
        qh, kh, vh, doh = (x[0, h].double() for x in (q, k, v, do))
        s = w.scale * (qh[rows] @ kh.T)
        s = s.masked_fill(torch.arange(N).unsqueeze(0) > torch.as_tensor(rows).unsqueeze(1), float("-inf"))
        pr, m, l = softmax_rows(s)
        z = torch.from_numpy(DR.draws(seed, h, rows, np.arange(N)) < t).double() * (256.0 / t)
        ro = (pr * z) @ vh
        rl = m + torch.log(l)
        dp = (doh[rows] @ vh.T) * z
        dd = (doh[rows] * ro).sum(-1, keepdim=True)
        rdq = w.scale * ((pr * (dp - dd)) @ kh)
        a = (pr * z) @ vh.abs()
        err = (o[0, h][rows].double() - ro).abs()
        worst = float((err / (2.0 ** -8 * (a + ro.abs()) + 1e-6)).max())
        assert worst <= 1.0, f"head {h}: O error reaches {worst:.3f} of its rounding bound"
        assert max_abs(lse[0, h][rows], rl) <= 1e-3, f"head {h}: LSE"
        assert rel_frob(dq[0, h][rows], rdq) <= 5e-2, f"head {h}: dQ relF {rel_frob(dq[0, h][rows], rdq)}"


def test_dropout_bitwise_deterministic():
    shape = (2, 3, 333, 128)
    q, k, v, do = make_inputs(shape, torch.bfloat16, 12)
    a = run_dropout(q, k, v, do, 0.1, True, 0.3, 99)
    b = run_dropout(q, k, v, do, 0.1, True, 0.3, 99)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("N", [31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257])
def test_dropout_tile_boundaries(N):
    # sequence lengths around the 32-key blocks, 128-row workgroups and the
    # 4 x 4 draw tiles; causal, d = 64
    shape = (1, 2, N, 64)
    q, k, v, do = make_inputs(shape, torch.bfloat16, 100 + N)
    p, seed = 0.25, 555 + N
    o, lse, dq, dk, dv = run_dropout(q, k, v, do, 0.125, True, p, seed)
    t = DR.keep_threshold(p)
    keep = DR.keep_masks(seed, 1, 2, N, t)
    ro, rl, rdq, rdk, rdv = DR.attention_forward_backward_dropout(q, k, v, do, 0.125, True, keep, t)
    check_o(o, ro, q, k, v, 0.125, True, keep, t, f"N={N}")
    assert max_abs(lse, rl) <= 1e-3, f"N={N}"
    for name, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert rel_frob(g, r) <= 5e-2, f"N={N}: {name} relF {rel_frob(g, r)}"

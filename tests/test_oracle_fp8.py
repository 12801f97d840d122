"""Pins of the FP8 oracle: the E4M3 format, the block exponents, quantisation.

The format is checked against torch's float8_e4m3fn conversion (an
independent implementation of the same OCP format), the exponent rule against
its closed form, the quantiser against its invariants, and the attention of
quantised inputs against plain attention on inputs the format holds exactly.
"""
import numpy as np
import pytest
import torch

from oracle import fp8 as F8
from oracle.attention import attention_forward

f8 = getattr(torch, "float8_e4m3fn", None)
needs_f8 = pytest.mark.skipif(f8 is None, reason="torch without float8_e4m3fn")


def all_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


@needs_f8
def test_decode_matches_torch():
    codes = all_codes()
    want = torch.from_numpy(codes).view(f8).to(torch.float64).numpy()
    np.testing.assert_array_equal(F8.e4m3_decode(codes), want)
    assert F8.e4m3_decode(np.array([0x7E]))[0] == 448.0            # largest finite value
    assert F8.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9        # smallest subnormal
    assert np.isnan(F8.e4m3_decode(np.array([0x7F, 0xFF]))).all()  # the NaN patterns


def test_encode_inverts_decode():
    codes = all_codes()
    np.testing.assert_array_equal(F8.e4m3_encode(F8.e4m3_decode(codes)), codes)


@needs_f8
def test_round_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(3)
    vals = F8.e4m3_decode(all_codes())
    finite = np.sort(np.unique(vals[np.isfinite(vals)]))
    mids = (finite[:-1] + finite[1:]) / 2                 # exact ties (float32-representable)
    rand = rng.uniform(-448, 448, 20000) * np.exp2(rng.integers(-16, 1, 20000))
    x = np.concatenate([finite, mids, rand, [2.0 ** -10, 3 * 2.0 ** -11, 464.0, -464.0]])
    x = x[np.abs(x) <= 448.0 + 16].astype(np.float32)
    want = torch.from_numpy(x).to(f8).to(torch.float64).numpy()
    got = F8.e4m3_round(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(F8.e4m3_encode(got), torch.from_numpy(x).to(f8).view(torch.uint8).numpy())


def test_round_rejects_out_of_range():
    with pytest.raises(ValueError):
        F8.e4m3_round(np.array([465.0]))


def test_block_exponent_closed_form():
    assert F8.block_exponent(np.array([448.0, 449.0, 224.0, 224.5, 0.0, 1.0, 1.75, 1.76]))\
        .tolist() == [0, 1, -1, 0, 0, -8, -8, -7]
    rng = np.random.default_rng(4)
    a = rng.uniform(0.5, 1.0, 5000) * np.exp2(rng.integers(-100, 100, 5000))
    e = F8.block_exponent(a)
    assert np.all(a <= 448.0 * np.exp2(e)) and np.all(a > 448.0 * np.exp2(e - 1))
    assert F8.block_exponent(np.array([1e-60]))[0] == -127         # clamped
    assert F8.block_exponent(np.array([1e60]))[0] == 127


def test_quantize_blocks_invariants():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 7, 128)) * np.exp2(rng.integers(-20, 20, (3, 7, 1)))
    x[1, 2, 32:64] = 0.0                                          # an all-zero block
    codes, e, deq = F8.quantize_blocks(x)
    xb, db = x.reshape(3, 7, 4, 32), deq.reshape(3, 7, 4, 32)
    amax = np.abs(xb).max(-1)
    nz = amax > 0
    # the block maximum lands in (224, 448] before scaling back
    qmax = np.abs(db).max(-1)[nz] / np.exp2(e[nz])
    assert np.all((qmax > 224 - 16) & (qmax <= 448))
    # codes hold the dequantised values; errors within half a spacing (2^-4 relative)
    np.testing.assert_array_equal(F8.e4m3_decode(codes).reshape(3, 7, 4, 32) * np.exp2(e)[..., None], db)
    err = np.abs(db - xb)
    bound = np.maximum(np.abs(xb) * 2.0 ** -4, 2.0 ** -10 * np.exp2(e)[..., None])
    assert np.all(err <= bound)
    assert np.all(deq[1, 2, 32:64] == 0) and e[1, 2, 1] == 0


def test_quantize_keys_layout():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((2, 70, 32))
    codes, e, deq = F8.quantize_keys(v)
    assert codes.shape == (2, 32, 128) and e.shape == (2, 4, 32) and deq.shape == v.shape
    assert np.all(codes[:, :, 70:] == 0)                          # padded keys
    # block (kb, dim) covers keys 32kb .. 32kb+31 of that dim
    for kb in range(3):
        blk = v[:, 32 * kb:32 * kb + 32, :]
        amax = np.abs(blk).max(axis=1)
        np.testing.assert_array_equal(e[:, kb, :], F8.block_exponent(amax))
    np.testing.assert_array_equal(
        np.swapaxes(F8.e4m3_decode(codes), -1, -2)[:, :70, :] * np.repeat(np.exp2(e), 32, axis=1)[:, :70, :],
        deq)


@pytest.mark.parametrize("causal", [False, True])
def test_exactly_representable_inputs_give_plain_attention(causal):
    # entries k/8 with |k| <= 8 and a +-1 in every 32-block: each block has
    # exponent -8 and every entry * 256 is a multiple of 32 <= 256, which E4M3 holds
    rng = np.random.default_rng(7)
    def make(n, d):
        x = rng.integers(-8, 9, (1, 2, n, d)) / 8.0
        x[..., ::32] = 1.0
        return x
    q, k = make(40, 64), make(40, 64)
    v = np.swapaxes(make(64, 40), -1, -2)                          # +-1 in every 32-key block
    v = np.ascontiguousarray(v)
    o, lse, qd, kd, vd = F8.attention_forward_fp8(q, k, v, 0.125, causal)
    assert np.array_equal(qd.numpy(), q) and np.array_equal(kd.numpy(), k) and np.array_equal(vd.numpy(), v)
    o2, l2 = attention_forward(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), 0.125, causal)
    torch.testing.assert_close(o, o2, rtol=0, atol=1e-13)
    torch.testing.assert_close(lse, l2, rtol=0, atol=1e-13)


def test_block_quantisation_keeps_small_heads_that_one_scale_per_tensor_loses():
    # what a scale per block buys over one scale per tensor: every block uses
    # the format's full precision, so parts of the tensor far smaller than its
    # largest entry are not pushed into the subnormals (or to zero).  Here the
    # second head is 2^-16 times the first.
    rng = np.random.default_rng(8)
    shape = (1, 2, 128, 64)
    q, k, v = (rng.standard_normal(shape) for _ in range(3))
    for t in (q, k, v):
        t[:, 1] *= 2.0 ** -16
    ref_o, _ = attention_forward(*(torch.from_numpy(t) for t in (q, k, v)), 0.125, False)
    o_blk = F8.attention_forward_fp8(q, k, v, 0.125, False)[0]

    def per_tensor(t):
        s = np.abs(t).max() / 448.0
        return F8.e4m3_round(t / s) * s
    o_tns, _ = attention_forward(*(torch.from_numpy(per_tensor(t)) for t in (q, k, v)), 0.125, False)

    def worst_head_rel(o):
        return max(float(torch.linalg.vector_norm(o[:, h] - ref_o[:, h]) / torch.linalg.vector_norm(ref_o[:, h]))
                   for h in range(2))
    blk, tns = worst_head_rel(o_blk), worst_head_rel(o_tns)
    assert blk < 0.06            # about the format's 2^-4 relative rounding
    assert tns > 5 * blk

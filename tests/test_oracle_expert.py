"""Pins for the oracle's per-expert linear map (the expert between dispatch
and combine) and its double -> bf16 rounding.

Independent of the oracle's loops: exact integer arithmetic, identity and
permutation weights, torch's float -> bf16 conversion on values that fp32
holds exactly, numpy float64 matmul within one bf16 ulp, and a hand-worked
example."""
import numpy as np
import pytest
import torch

import oracle


def _bf16_bits(a32):
    return torch.from_numpy(np.asarray(a32, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _f32(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def test_f64_to_bf16_on_fp32_values_matches_torch():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    v = np.concatenate([v, np.float32([1.0, -1.0, 0.5, 3.0, 1.00390625, 1.01171875, 65280.0])])
    got = np.array([oracle.f64_to_bf16(float(a)) for a in v], np.uint16)
    np.testing.assert_array_equal(got, _bf16_bits(v))


def test_f64_to_bf16_rounds_once_from_double():
    # 1 + 2^-8 is a bf16 tie (to even: 1.0); 1 + 2^-8 + 2^-40 is above the tie
    # but rounds to the tie itself in fp32, so rounding via fp32 would give 1.0
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert oracle.f64_to_bf16(-(1.0 + 3 * 2.0 ** -8)) == 0xBF82      # tie to even upward
    assert oracle.f64_to_bf16(0.0) == 0x0000 and oracle.f64_to_bf16(-0.0) == 0x8000
    assert oracle.f64_to_bf16(255.5) == 0x4380                         # 256 after the carry


def test_worked_example():
    # two experts, H = 2, N = 2; rows 0..1 belong to expert 0, row 2 to expert 1
    x = _bf16_bits([[1.0, 2.0], [3.0, -1.0], [0.5, 0.25]])
    w = _bf16_bits([[[1.0, 0.0], [1.0, 1.0]],          # expert 0: y = (x0, x0 + x1)
                    [[2.0, 4.0], [0.0, -8.0]]])        # expert 1: y = (2 x0 + 4 x1, -8 x1)
    y = oracle.expert_linear(x, w, np.array([0, 2, 3], np.int32))
    np.testing.assert_array_equal(_f32(y), np.float32([[1.0, 3.0], [3.0, 2.0], [2.0, -2.0]]))


def test_identity_and_permutation_weights_copy_rows():
    rng = np.random.default_rng(2)
    E, H, rows = 3, 64, 40
    x = _bf16_bits(rng.standard_normal((rows, H)))
    eye = _bf16_bits(np.eye(H))
    perm = rng.permutation(H)
    pw = _bf16_bits(np.eye(H)[perm])                   # y[:, n] = x[:, perm[n]]
    w = np.stack([eye, pw, eye])
    off = np.array([0, 11, 30, rows], np.int32)
    y = oracle.expert_linear(x, w, off)
    np.testing.assert_array_equal(y[:11], x[:11])
    np.testing.assert_array_equal(y[11:30], x[11:30][:, perm])
    np.testing.assert_array_equal(y[30:], x[30:])


def test_integer_values_are_exact():
    rng = np.random.default_rng(3)
    E, H, N, rows = 2, 96, 24, 30
    xi = rng.integers(-4, 5, (rows, H))
    wi = rng.integers(-3, 4, (E, N, H))
    off = np.array([0, 13, rows], np.int32)
    y = oracle.expert_linear(_bf16_bits(xi), _bf16_bits(wi), off)
    want = np.concatenate([xi[:13] @ wi[0].T, xi[13:] @ wi[1].T])       # |sum| <= 1152
    np.testing.assert_array_equal(y, _bf16_bits(want.astype(np.float32)))


@pytest.mark.parametrize("seed", range(3))
def test_matches_numpy_matmul_within_one_bf16_ulp(seed):
    rng = np.random.default_rng(10 + seed)
    E, H, N, rows = 4, 256, 48, 70
    x = _bf16_bits(rng.standard_normal((rows, H)))
    w = _bf16_bits(rng.standard_normal((E, N, H)) * 0.05)
    cuts = np.sort(rng.integers(0, rows + 1, E - 1))
    off = np.concatenate([[0], cuts, [rows]]).astype(np.int32)          # some runs may be empty
    y = oracle.expert_linear(x, w, off)
    xf, wf = _f32(x).astype(np.float64), _f32(w).astype(np.float64)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        ref = xf[lo:hi] @ wf[e].T
        got = _f32(y[lo:hi]).astype(np.float64)
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)

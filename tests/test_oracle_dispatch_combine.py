"""Pins for the oracle's dispatch (bf16 copy, fp8 quantise) and combine.

Independent references: numpy fancy indexing, numpy's IEEE float32 division and
torch's E4M3 / bf16 conversions, exact rational evaluation of every fused
multiply-add with correct rounding, one-hot and identity-expert closed forms,
and hand-worked values.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import custom, make_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _torch_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _torch_e4m3(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


# --------------------------------------------------------------------- dispatch bf16
@pytest.mark.parametrize("name", ["tiny_T128_H1024_E8_k2_R2", "tiny_zipf_T128_H1024_E8_k2_R2"])
def test_dispatch_bf16_is_replicated_scatter(name):
    w = make_config(name)
    s = w.shape
    L = oracle.layout(w.topk_idx, s.E, s.R)
    recv = oracle.dispatch_bf16(w.x, L["pos"])
    np.testing.assert_array_equal(recv[L["pos"].ravel()], np.repeat(w.x, s.k, axis=0))
    # each token row appears exactly k times
    rows, counts = np.unique(recv.view(np.dtype((np.void, 2 * s.H))), return_counts=True)
    xs, xc = np.unique(w.x.view(np.dtype((np.void, 2 * s.H))), return_counts=True)
    assert np.array_equal(rows, xs) and np.array_equal(counts, xc * s.k)


# --------------------------------------------------------------------- dispatch fp8
def _numpy_fp8_reference(x, k):
    """Per token and 128-channel block: numpy float32 amax and IEEE division,
    torch's E4M3 conversion (x / s never exceeds 448 by more than rounding, so
    torch's missing saturation above 464 does not matter here)."""
    T, H = x.shape
    xf = _bf16_f32(x).reshape(T, H // 128, 128)
    amax = np.abs(xf).max(axis=2)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = _torch_e4m3((xf / s[:, :, None]).astype(np.float32)).reshape(T, H)
    return q, s


def test_dispatch_fp8_matches_numpy_division_and_torch_codec():
    w = custom(T=64, H=512, E=16, k=4, R=4, payload="fp8", seed=7)
    s = w.shape
    L = oracle.layout(w.topk_idx, s.E, s.R)
    q, sc = oracle.dispatch_fp8(w.x, L["pos"])
    qr, sr = _numpy_fp8_reference(w.x, s.k)
    np.testing.assert_array_equal(q[L["pos"].ravel()], np.repeat(qr, s.k, axis=0))
    np.testing.assert_array_equal(sc[L["pos"].ravel()], np.repeat(sr, s.k, axis=0))


def test_dispatch_fp8_invariants_and_error_bound():
    w = custom(T=32, H=1024, E=8, k=2, R=2, payload="fp8", seed=11)
    pos = np.arange(32 * 2, dtype=np.int32).reshape(32, 2)
    q, sc = oracle.dispatch_fp8(w.x, pos)
    xf = _bf16_f32(w.x).reshape(32, 8, 128)
    qq = q[::2].reshape(32, 8, 128)
    # the element holding the block's amax encodes to +-448
    am = np.abs(xf).argmax(axis=2)
    top = np.take_along_axis(qq, am[:, :, None], axis=2)[:, :, 0]
    assert np.all((top == 0x7E) | (top == 0xFE))
    # |decode(q) * s - x| <= 2^-4 |x| in the normal range, <= 2^-10 s below it
    deq = oracle.e4m3_to_f32(qq).astype(np.float64) * sc[::2].reshape(32, 8, 1)
    err = np.abs(deq - xf)
    normal = np.abs(xf) >= 2.0 ** -6 * sc[::2].reshape(32, 8, 1)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(xf[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * np.broadcast_to(sc[::2].reshape(32, 8, 1), xf.shape)[~normal])


def test_dispatch_fp8_worked_block():
    rows = []
    scale = None
    with open(os.path.join(GOLDEN, "fp8_block_worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            if parts[0] == "scale":
                scale = float(parts[1])
            else:
                rows.append((int(parts[0]), float(parts[1]), int(parts[2], 16)))
    x32 = np.zeros((1, 128), np.float32)
    for c, v, _ in rows:
        x32[0, c] = v
    x = _torch_bf16(x32)
    assert np.array_equal(_bf16_f32(x), x32)            # all values exact in bf16
    q, s = oracle.dispatch_fp8(x, np.zeros((1, 1), np.int32))
    assert s[0, 0] == scale
    for c, _, code in rows:
        assert q[0, c] == code, (c, hex(q[0, c]), hex(code))
    assert np.all(q[0, 8:] == 0)


def test_dispatch_fp8_zero_block_and_negative_zero():
    x32 = np.zeros((1, 256), np.float32)
    x32[0, 3] = -0.0
    x32[0, 200] = 2.0
    q, s = oracle.dispatch_fp8(_torch_bf16(x32), np.zeros((1, 1), np.int32))
    assert s[0, 0] == 1.0 and s[0, 1] == np.float32(2.0) / np.float32(448.0)
    assert q[0, 3] == 0x80 and q[0, 0] == 0x00 and q[0, 200] == 0x7E


def test_identity_fp8_matches_torch():
    rng = np.random.default_rng(5)
    q = rng.integers(0, 256, size=(16, 256), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x10                            # no NaN codes
    s = (rng.random((16, 2)) * 0.02 + 1e-4).astype(np.float32)
    y = oracle.identity_fp8(q, s)
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).float().numpy()
    ref = _torch_bf16((dec.reshape(16, 2, 128) * s[:, :, None]).reshape(16, 256))
    np.testing.assert_array_equal(y, ref)


# --------------------------------------------------------------------- combine
def _round_f32_exact(q: Fraction) -> np.float32:
    """Nearest fp32 to the rational q, ties to even mantissa."""
    f = np.float32(float(q))
    cands = [f, np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def _exact_combine(y, pos, w):
    T, k = pos.shape
    H = y.shape[1]
    yf = _bf16_f32(y)
    out = np.empty((T, H), np.float32)
    for t in range(T):
        for c in range(H):
            acc = np.float32(0.0)
            for j in range(k):
                acc = _round_f32_exact(Fraction(float(w[t, j])) * Fraction(float(yf[pos[t, j], c]))
                                       + Fraction(float(acc)))
            out[t, c] = acc
    return _torch_bf16(out)


@pytest.mark.parametrize("seed", [0, 1])
def test_combine_exact_rational_tiny(seed):
    rng = np.random.default_rng(seed)
    T, H, k = 6, 16, 4
    rows = T * k
    y = _torch_bf16(rng.standard_normal((rows, H)).astype(np.float32) * 3)
    pos = rng.permutation(rows).astype(np.int32).reshape(T, k)
    w = rng.random((T, k)).astype(np.float32)
    w[0] = [-1.5, 2.0 ** -20, 1e-3, 7.0]                   # mixed signs and scales
    np.testing.assert_array_equal(oracle.combine(y, pos, w), _exact_combine(y, pos, w))


def test_combine_slot_order_matters_and_is_followed():
    # y values chosen so that the fp32 sum depends on the order of slots
    y32 = np.array([[1.0], [2.0 ** -24], [2.0 ** -24], [-1.0]], np.float32)
    y32 = np.repeat(y32, 8, axis=1)
    y = _torch_bf16(y32)
    pos = np.array([[0, 1, 2, 3]], np.int32)
    w = np.ones((1, 4), np.float32)
    out = oracle.combine(y, pos, w)
    np.testing.assert_array_equal(out, _exact_combine(y, pos, w))
    # slot order 0..3: ((1 + 2^-24) + 2^-24) - 1 = 0 in fp32 (each add rounds back to 1)
    assert np.all(out == 0)
    out_rev = oracle.combine(y, pos[:, ::-1].copy(), w)
    assert np.all(_bf16_f32(out_rev) == np.float32(2.0 ** -23))


def test_combine_one_hot_is_identity():
    w = custom(T=64, H=256, E=8, k=4, R=2, seed=3)
    s = w.shape
    L = oracle.layout(w.topk_idx, s.E, s.R)
    recv = oracle.dispatch_bf16(w.x, L["pos"])
    onehot = np.zeros((s.T, s.k), np.float32)
    onehot[np.arange(s.T), np.arange(s.T) % s.k] = 1.0
    np.testing.assert_array_equal(oracle.combine(recv, L["pos"], onehot), w.x)


@pytest.mark.parametrize("name", ["tiny_T128_H1024_E8_k2_R2", "tiny_zipf_T128_H1024_E8_k2_R2"])
def test_combine_identity_closed_form(name):
    """Identity experts: all k rows of token t equal x[t], so the result is
    x[t] * sum_j w_j; the weights sum to 1 within k * 2^-24, so out is within
    one bf16 ulp of x and equals the float64 einsum rounded once to bf16 except
    where that value sits within a rounding error of a bf16 tie."""
    w = make_config(name)
    s = w.shape
    L = oracle.layout(w.topk_idx, s.E, s.R)
    recv = oracle.dispatch_bf16(w.x, L["pos"])
    out = oracle.combine(recv, L["pos"], w.topk_w)
    xf = _bf16_f32(w.x).astype(np.float64)
    ref = np.einsum("tk,tkh->th", w.topk_w.astype(np.float64),
                    _bf16_f32(recv[L["pos"]]).astype(np.float64))
    np.testing.assert_allclose(ref, xf * w.topk_w.astype(np.float64).sum(1, keepdims=True),
                               rtol=0, atol=0)
    ordinal = np.abs(out.astype(np.int64) - w.x.astype(np.int64))
    same_sign = (out >> 15) == (w.x >> 15)
    assert np.all(ordinal[same_sign & (xf != 0)] <= 1)
    assert np.mean(out == _torch_bf16(ref.astype(np.float32))) > 0.999


def test_pipeline_tokens_matches_full_problem():
    w = custom(T=32, H=256, E=8, k=3, R=4, payload="fp8", seed=9)
    s = w.shape
    L = oracle.layout(w.topk_idx, s.E, s.R)
    q, sc = oracle.dispatch_fp8(w.x, L["pos"])
    out_full = oracle.combine(oracle.identity_fp8(q, sc), L["pos"], w.topk_w)
    toks = np.array([0, 5, 31, 17])
    (qs, ss), out = oracle.pipeline_tokens(w.x, w.topk_idx, w.topk_w, s.E, s.R, payload="fp8",
                                           tokens=toks)
    np.testing.assert_array_equal(out, out_full[toks])
    np.testing.assert_array_equal(qs, q[L["pos"][toks]])
    np.testing.assert_array_equal(ss, sc[L["pos"][toks]])


def _find_fma_sensitive_case():
    """Search (w, y) with slot 0 = 1 * 1.0 so that the exact chain
    fma(w, y, 1) and the unfused round(1 + round(w * y)) give different bf16
    results: the unfused sum lands exactly on a bf16 tie, the fused one just
    above it.  Returned weights/values are plain fp32 / bf16."""
    P = Fraction(1, 2 ** 8) + Fraction(1, 2 ** 24)          # 1 + P is an fp32 tie
    for m in range(1, 128):
        y = np.float32(1.0 + m / 128.0)                    # exact bf16 values in [1, 2)
        w0 = np.float32(float(P / Fraction(float(y))))
        for w in (w0, np.nextafter(w0, np.float32(1)), np.nextafter(w0, np.float32(0))):
            prod = Fraction(float(w)) * Fraction(float(y))
            fused = _round_f32_exact(prod + 1)
            unfused = _round_f32_exact(Fraction(float(_round_f32_exact(prod))) + 1)
            if _torch_bf16(np.array([fused]))[0] != _torch_bf16(np.array([unfused]))[0]:
                return np.float32(w), np.float32(y)
    raise AssertionError("no case found")


def test_combine_uses_fused_multiply_add():
    w1, y1 = _find_fma_sensitive_case()
    y32 = np.zeros((2, 8), np.float32)
    y32[0] = 1.0
    y32[1] = y1
    y = _torch_bf16(y32)
    pos = np.array([[0, 1]], np.int32)
    w = np.array([[1.0, w1]], np.float32)
    np.testing.assert_array_equal(oracle.combine(y, pos, w), _exact_combine(y, pos, w))


def test_combine_chain_starts_from_positive_zero():
    # every product is -0: (+0) + (-0) = +0 under round-to-nearest, so the
    # result is +0 (a chain started from -0 would give -0)
    y = np.zeros((2, 8), np.uint16)
    pos = np.array([[0, 1]], np.int32)
    w = np.array([[-1.0, -2.0]], np.float32)
    assert np.all(oracle.combine(y, pos, w) == 0x0000)
    # -0 inputs with a positive one-hot weight also give +0
    y[:] = 0x8000
    assert np.all(oracle.combine(y, pos, np.array([[1.0, 0.0]], np.float32)) == 0x0000)

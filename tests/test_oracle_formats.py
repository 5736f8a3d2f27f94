"""Pins for the oracle's number formats: bf16 rounding and the E4M3FN codec.

Independent references: torch's own float8_e4m3fn and bfloat16 conversions,
a numpy nearest-value search written here from the OCP E4M3 value set, and
hand-worked values.
"""
import numpy as np
import pytest
import torch

import oracle


def _f32(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def _torch_e4m3(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# the non-negative finite E4M3FN values from the OCP specification's table:
# subnormals m/8 * 2^-6 (m = 0..7), normals (1 + m/8) * 2^(x-7), x = 1..15,
# except x = 15, m = 7 (NaN)
def _spec_values():
    v = [m / 8 * 2.0 ** -6 for m in range(8)]
    for x in range(1, 16):
        for m in range(8):
            if x == 15 and m == 7:
                continue
            v.append((1 + m / 8) * 2.0 ** (x - 7))
    return np.array(v, np.float64)


SPEC = _spec_values()


def _numpy_nearest_e4m3(a):
    """Independent nearest-even search over the spec's value list."""
    a = np.asarray(a, np.float32)
    mag = np.abs(a.astype(np.float64))
    hi = np.searchsorted(SPEC, mag, side="left").clip(1, 126)     # SPEC[hi-1] < mag <= SPEC[hi]
    lo = hi - 1
    dlo = mag - SPEC[lo]
    dhi = SPEC[hi] - mag
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(mag >= 448.0, 126, code)
    code = np.where(mag == 0, 0, code)
    return (code | np.where(np.signbit(a), 0x80, 0)).astype(np.uint8)


def test_decode_table_closed_form_and_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_f32(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.isnan(got[nan]).all()
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    np.testing.assert_array_equal(got[:127].astype(np.float64), SPEC)
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_encode_every_bf16_value_matches_torch():
    b = np.arange(65536, dtype=np.uint32)
    a = _f32(b << 16)
    keep = np.isfinite(a) & (np.abs(a) <= 464.0)     # torch does not saturate above 464
    a = a[keep]
    np.testing.assert_array_equal(oracle.f32_to_e4m3(a), _torch_e4m3(a))


def test_encode_ties_and_neighbours():
    mids = ((SPEC[:-1] + SPEC[1:]) / 2).astype(np.float32)    # exact in fp32
    assert np.all(mids.astype(np.float64) == (SPEC[:-1] + SPEC[1:]) / 2)
    pts = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                          SPEC.astype(np.float32)])
    pts = np.concatenate([pts, -pts])
    got = oracle.f32_to_e4m3(pts)
    np.testing.assert_array_equal(got, _numpy_nearest_e4m3(pts))
    np.testing.assert_array_equal(got, _torch_e4m3(pts))
    # ties go to the even code: 1.0625 -> 1.0, 1.1875 -> 1.25, 2^-9*1.5 -> 2*2^-9
    assert oracle.f32_to_e4m3(np.array([1.0625, 1.1875, 1.5 * 2 ** -9], np.float32)).tolist() == \
        [0x38, 0x3A, 0x02]


def test_encode_dense_sweep_matches_independent_search():
    # every 61st fp32 bit pattern from 0 up to 464.0, both signs
    bits = np.arange(0, 0x43E80000 + 1, 61, dtype=np.uint32)
    a = _f32(bits)
    np.testing.assert_array_equal(oracle.f32_to_e4m3(a), _numpy_nearest_e4m3(a))
    np.testing.assert_array_equal(oracle.f32_to_e4m3(-a), _numpy_nearest_e4m3(-a))


def test_encode_saturation_and_zero():
    a = np.array([448.0, 450.0, 464.0, 464.5, 480.0, 1e6, 3e38], np.float32)
    assert oracle.f32_to_e4m3(a).tolist() == [0x7E] * 7
    assert oracle.f32_to_e4m3(-a).tolist() == [0xFE] * 7
    assert oracle.f32_to_e4m3(np.array([0.0, -0.0, 1e-30, -1e-30], np.float32)).tolist() == \
        [0x00, 0x80, 0x00, 0x80]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        _f32(rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)),
        _f32((np.arange(4096, dtype=np.uint32) << 16) | 0x8000),       # exact ties
        _f32((np.arange(4096, dtype=np.uint32) << 16) | 0x7FFF),
        _f32((np.arange(4096, dtype=np.uint32) << 16) | 0x8001),
        np.array([3.4e38, -3.4e38, 1e-45, -0.0, 0.0], np.float32),
    ])
    a = a[np.isfinite(a)]
    np.testing.assert_array_equal(oracle.f32_to_bf16(a), _torch_bf16(a))


def test_bf16_roundtrip_exact():
    b = np.arange(65536, dtype=np.uint16)
    f = oracle.bf16_to_f32(b)
    fin = np.isfinite(f)
    np.testing.assert_array_equal(oracle.f32_to_bf16(f[fin]), b[fin])

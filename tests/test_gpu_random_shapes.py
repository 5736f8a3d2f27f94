"""GPU parity on seeded random shapes: the layout in both key orders (every
output, bit-exact against the oracle), and dispatch + combine (whole outputs)
with the separate calls, the fused layout + dispatch launch, the chunk
pipeline and the sentinel pipeline.

The shapes are drawn once from a fixed seed so that every run checks the same
cases.  They spread over what picks the layout's kernel and tiling: rows from
a few dozen to about 200 thousand, one or many tiles, tiles whose row count
is not a multiple of 64 or of 4, k from 1 to 16, up to 64 ranks and 1024
experts, up to 64 chunks, uniform and Zipf routing.  The payload is small
(H <= 40 channels) so that the oracle's dispatch and combine take
milliseconds.
"""
import numpy as np
import pytest
import torch

import combine_top_route_amd as ubep
import oracle
from combine_top_route_amd.buffers import run_path
from workloads import custom
from gpu_helpers import LAYOUT_KEYS, assert_layout_equal, device_status, say, to_np, upload

pytestmark = pytest.mark.gpu

GROUPED_KEYS = LAYOUT_KEYS + ("expert_offset",)


def _divisors(n, cap):
    return [d for d in range(1, min(n, cap) + 1) if n % d == 0]


def _draw_shapes(n, seed=20261203):
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < n:
        R = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 32, 64]))
        tps = int(rng.integers(1, 769))
        T = R * tps
        epr = int(rng.integers(1, 17))
        E = R * epr
        if E > 1024:
            continue
        k = int(rng.integers(1, min(16, E) + 1))
        if T * k > 200_000:
            continue
        C = int(rng.choice(_divisors(T, 64)))
        H = int(rng.choice([8, 16, 24, 40]))
        routing = "zipf" if rng.random() < 0.4 else "topk"
        shapes.append(dict(T=T, H=H, E=E, k=k, R=R, C=C, routing=routing,
                           seed=int(rng.integers(1, 1 << 30))))
    return shapes


SHAPES = _draw_shapes(32)
IDS = [f"T{s['T']}E{s['E']}k{s['k']}R{s['R']}C{s['C']}H{s['H']}{s['routing'][0]}" for s in SHAPES]


def _grouped_equal(got, ref, C):
    for key in GROUPED_KEYS:
        if key == "chunk_offset" and C == 1:
            continue
        a, r = np.asarray(got[key]).ravel(), np.asarray(ref[key]).ravel()
        assert np.array_equal(a, r), f"{key}: {np.count_nonzero(a != r)} mismatches"


@pytest.mark.parametrize("spec", SHAPES, ids=IDS)
def test_random_shape_layouts_and_path(spec):
    w = custom(weights="softmax", **spec)
    s = w.shape
    C = s.C
    say(f"random shape {spec}")
    b = upload(w)
    # rank order, separate calls
    ubep.ubep_layout(b.shape, b.topk_idx, b.pos, b.expert_count, b.rank_count, b.recv_offset,
                     b.send_offset, b.chunk_offset if C > 1 else None, b.recv_src, b.ws)
    ubep.ubep_dispatch(b.shape, ubep.BF16, b.x, b.pos, b.recv, None, b.ws)
    ubep.ubep_combine(b.shape, b.recv, b.pos, b.topk_w, b.out, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    ref = oracle.layout(w.topk_idx, s.E, s.R, C)
    assert_layout_equal({k: to_np(getattr(b, k)) for k in LAYOUT_KEYS}, ref, C)
    recv = oracle.dispatch_bf16(w.x, ref["pos"])
    out = oracle.combine(recv, ref["pos"], w.topk_w)
    np.testing.assert_array_equal(to_np(b.recv), recv)
    np.testing.assert_array_equal(to_np(b.out), out)

    # rank order, fused layout + dispatch launch (its own tiling)
    b.pos.fill_(-1)
    b.recv.zero_()
    b.out.zero_()
    ubep.ubep_layout_dispatch(b.shape, b.topk_idx, b.x, b.pos, b.expert_count, b.rank_count,
                              b.recv_offset, b.send_offset, b.chunk_offset if C > 1 else None,
                              b.recv_src, b.recv, b.ws)
    ubep.ubep_combine(b.shape, b.recv, b.pos, b.topk_w, b.out, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    assert_layout_equal({k: to_np(getattr(b, k)) for k in LAYOUT_KEYS}, ref, C)
    np.testing.assert_array_equal(to_np(b.recv), recv)
    np.testing.assert_array_equal(to_np(b.out), out)

    # expert order on the same workspace
    eoff = torch.empty(s.E + 1, dtype=torch.int32, device="cuda")
    ubep.ubep_layout_grouped(b.shape, b.topk_idx, b.pos, b.expert_count, eoff, b.rank_count,
                             b.recv_offset, b.send_offset, b.chunk_offset if C > 1 else None,
                             b.recv_src, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    got = {k: to_np(getattr(b, k)) for k in LAYOUT_KEYS}
    got["expert_offset"] = to_np(eoff)
    _grouped_equal(got, oracle.layout_grouped(w.topk_idx, s.E, s.R, C), C)


@pytest.mark.parametrize("spec", SHAPES[::2], ids=IDS[::2])
def test_random_shape_pipelines(spec):
    """The chunk pipeline (index order and the device's LPT order) and the
    sentinel pipeline against the oracle's dispatch + combine, whole outputs."""
    w = custom(weights="softmax", **spec)
    s = w.shape
    say(f"random shape pipelines {spec}")
    b = upload(w)
    ref = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    recv = oracle.dispatch_bf16(w.x, ref["pos"])
    out = oracle.combine(recv, ref["pos"], w.topk_w)
    for order in (None, "lpt"):
        b.out.zero_()
        b.recv.zero_()
        run_path(b, chunked=True, chunk_order=order)
        torch.cuda.synchronize()
        assert device_status(b) == ubep.OK, order
        np.testing.assert_array_equal(to_np(b.recv), recv, err_msg=str(order))
        np.testing.assert_array_equal(to_np(b.out), out, err_msg=str(order))
    # sentinel pipeline: every receive row's first 16 bytes start as the
    # sentinel and hold it again after the call
    ubep.ubep_recv_sentinel_init(b.recv, s.T * s.k, s.H)
    b.out.zero_()
    ubep.ubep_dispatch_combine_sentinel(b.shape, b.x, b.pos, b.topk_w, b.recv, b.out, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    np.testing.assert_array_equal(to_np(b.out), out)
    got = to_np(b.recv)
    assert np.all(got[:, :8] == 0xFFFF)
    np.testing.assert_array_equal(got[:, 8:], recv[:, 8:])


FP8_SHAPES = [dict(s, H=128 * (1 + i % 3), payload="fp8") for i, s in enumerate(SHAPES[1::4])]


@pytest.mark.parametrize("spec", FP8_SHAPES,
                         ids=[f"T{s['T']}E{s['E']}k{s['k']}R{s['R']}H{s['H']}" for s in FP8_SHAPES])
def test_random_shape_fp8_path(spec):
    """fp8 payload: codes, scales, the identity expert's bf16 rows and the
    combined output, whole, against the oracle."""
    w = custom(weights="softmax", **spec)
    s = w.shape
    say(f"random shape fp8 {spec}")
    b = upload(w)
    run_path(b)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    ref = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    q, sc = oracle.dispatch_fp8(w.x, ref["pos"])
    np.testing.assert_array_equal(to_np(b.recv), q)
    np.testing.assert_array_equal(to_np(b.recv_scale), sc)
    y = oracle.identity_fp8(q, sc)
    np.testing.assert_array_equal(to_np(b.y), y)
    np.testing.assert_array_equal(to_np(b.out), oracle.combine(y, ref["pos"], w.topk_w))

"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: layout, offsets and dispatched bytes (bf16 rows, fp8 codes and scales)
bit-exact; combine bit-exact (the kernel runs the same slot-ordered fp32 FMA
chain and rounding as the oracle, so no tolerance is needed; the identity
property test separately allows one bf16 ulp against x).
"""
import numpy as np
import pytest
import torch

import combine_top_route_amd as ubep
import oracle
from combine_top_route_amd.buffers import alloc_buffers, run_path
from workloads import CONFIGS, custom, generate
from gpu_helpers import (LAYOUT_KEYS, assert_layout_equal, assert_path_whole, device_status,
                         dtype_of, gpu_layout, oracle_layout, say, shape_of, to_np, upload,
                         workload)

pytestmark = pytest.mark.gpu

SMALL = ["tiny_T128_H1024_E8_k2_R2", "tiny_zipf_T128_H1024_E8_k2_R2"]
FULL = ["dsv3_decode_T4096_H7168_E256_k8_R32", "dsv3_decode_zipf_T4096_H7168_E256_k8_R32",
        "qwen3_prefill_fp8_T16384_H4096_E128_k8_R16",
        "prefill_grouped_zipf_T65536_H7168_E256_k8_R64_C16"]

# shapes small enough for a whole-output oracle comparison; they span several
# layout tiles, ragged wave tails, odd k, tiles of one token, and all
# ids on one rank
MEDIUM = [
    dict(T=512, H=256, E=16, k=3, R=4, C=4, routing="topk", seed=1),
    dict(T=960, H=520, E=24, k=5, R=6, C=5, routing="zipf", seed=2),        # H % 16 != 0
    dict(T=2048, H=1024, E=64, k=8, R=8, C=8, routing="zipf", seed=3),
    dict(T=96, H=128, E=12, k=1, R=12, C=96, routing="topk", seed=4),       # k = 1, chunk = token
    dict(T=4096, H=64, E=256, k=8, R=32, C=2, routing="topk", seed=5),      # several tiles
    dict(T=1000, H=64, E=10, k=10, R=5, C=1, routing="topk", seed=6),       # k = E
    dict(T=64, H=8, E=2, k=2, R=1, C=1, routing="topk", seed=7),            # one rank, tiny H
    # the row kernels' instantiations that the full-size workloads run:
    # H = 7168 (groups of 128 threads, 7 vectors each; decode and large
    # prefill) with a ragged last block of one token, and H = 4096 (combine
    # groups of 128 threads, 4 vectors each; the combine of the fp8 prefill)
    dict(T=255, H=7168, E=40, k=8, R=5, C=3, routing="zipf", seed=10),
    dict(T=512, H=7168, E=256, k=8, R=32, C=2, routing="topk", seed=11),
    dict(T=384, H=4096, E=128, k=8, R=16, C=1, routing="topk", seed=12),
    # 42000 rows, odd k: 240 tiles of 175 rows (not a multiple of 64)
    dict(T=6000, H=32, E=56, k=7, R=8, C=3, routing="zipf", seed=13),
]


def _small_workload(spec, payload="bf16"):
    spec = dict(spec)
    return custom(weights="softmax", payload=payload, **spec)


def _full_compare(w, fused=False):
    s = w.shape
    say(f"full compare {w.recipe.note or s} fused={fused}")
    b = upload(w)
    run_path(b, fused=fused)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    L = oracle_layout(w)
    assert_layout_equal({k: to_np(getattr(b, k)) for k in ("pos", "expert_count", "rank_count",
                                                            "recv_offset", "send_offset",
                                                            "chunk_offset", "recv_src")}, L, s.C)
    if w.recipe.payload == "fp8":
        q, sc = oracle.dispatch_fp8(w.x, L["pos"])
        np.testing.assert_array_equal(to_np(b.recv), q)
        np.testing.assert_array_equal(to_np(b.recv_scale), sc)
        y = oracle.identity_fp8(q, sc)
        np.testing.assert_array_equal(to_np(b.y), y)
    else:
        y = oracle.dispatch_bf16(w.x, L["pos"])
        np.testing.assert_array_equal(to_np(b.recv), y)
    out = oracle.combine(y, L["pos"], w.topk_w)
    np.testing.assert_array_equal(to_np(b.out), out)
    return b


@pytest.mark.parametrize("name", SMALL)
def test_small_configs_bit_exact(name):
    _full_compare(workload(name))


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("spec", MEDIUM, ids=lambda s: f"T{s['T']}H{s['H']}E{s['E']}k{s['k']}R{s['R']}C{s['C']}")
def test_medium_shapes_bit_exact(spec, fused):
    """fused: ubep_layout_dispatch (layout workers and data workers in one launch)."""
    _full_compare(_small_workload(spec), fused=fused)


# worker caps that make layout workgroups take several tiles each: gather mode
# (few tiles; 32 tiles on 4 workers is exactly the per-worker claim limit,
# which the cap of 1 is raised to) and look-back mode (256 tiles x 256 ranks)
CAPPED = [
    (dict(T=1024, H=64, E=64, k=8, R=16, C=4, routing="zipf", seed=21), 1),
    (dict(T=1024, H=64, E=64, k=8, R=16, C=4, routing="zipf", seed=21), 5),
    (dict(T=16384, H=16, E=256, k=2, R=256, C=4, routing="topk", seed=22), 5),
]


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("spec,cap", CAPPED, ids=["gather-cap1", "gather-cap5", "lookback-cap5"])
def test_layout_workers_taking_several_tiles(spec, cap, fused):
    ubep.ubep_set_layout_workers(cap)
    try:
        _full_compare(_small_workload(spec), fused=fused)
    finally:
        ubep.ubep_set_layout_workers(0)


@pytest.mark.parametrize("spec", [dict(T=256, H=512, E=16, k=4, R=4, C=2, routing="zipf", seed=8),
                                  dict(T=128, H=1024, E=8, k=2, R=2, C=1, routing="topk", seed=9),
                                  # H = 4096: the 256-thread groups of the fp8 prefill
                                  dict(T=384, H=4096, E=128, k=8, R=16, C=1, routing="topk", seed=13),
                                  dict(T=129, H=4096, E=24, k=6, R=3, C=1, routing="zipf", seed=14),
                                  # H = 7168 (56 blocks of 128 channels; 448 threads a row)
                                  dict(T=64, H=7168, E=8, k=2, R=2, C=1, routing="topk", seed=15)],
                         ids=lambda s: f"T{s['T']}H{s['H']}E{s['E']}k{s['k']}")
def test_fp8_shapes_bit_exact(spec):
    _full_compare(_small_workload(spec, payload="fp8"))


@pytest.mark.parametrize("name", FULL)
def test_full_size_layout_bit_exact(name):
    w = workload(name)
    say(f"layout {name}")
    b = upload(w)
    got = gpu_layout(b)
    assert device_status(b) == ubep.OK
    assert_layout_equal(got, oracle_layout(w), w.shape.C)


def _check_full_path(name, chunked=False, order=None, fused=False):
    """The whole path at a full-size workload: layout bit-exact, then every
    dispatched row (bf16 rows, or fp8 codes and scales and the identity
    expert's output) and every combined token against the oracle."""
    w = workload(name)
    s = w.shape
    say(f"full path {name} chunked={chunked} order={order} fused={fused}")
    b = upload(w)
    run_path(b, chunked=chunked, chunk_order=order, fused=fused)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    assert_layout_equal({k: to_np(getattr(b, k)) for k in LAYOUT_KEYS}, oracle_layout(w), s.C)
    assert_path_whole(b, w, y=b.y if w.recipe.payload == "fp8" else None)
    return b


@pytest.mark.parametrize("name", FULL)
def test_full_size_path_whole_output(name):
    _check_full_path(name)


@pytest.mark.parametrize("name", FULL[:2])
def test_full_size_fused_layout_dispatch_whole_output(name):
    _check_full_path(name, fused=True)


@pytest.mark.parametrize("order", [None, "lpt"], ids=["index-order", "lpt-order"])
def test_large_prefill_chunked_whole_output(order):
    _check_full_path("prefill_grouped_zipf_T65536_H7168_E256_k8_R64_C16", chunked=True, order=order)


def test_fp8_codec_on_every_bf16_value():
    """Blocks whose amax is 448 have scale exactly 1, so the kernel's E4M3
    encoder sees every finite bf16 value in [-448, 448] unchanged."""
    b16 = np.arange(65536, dtype=np.uint32)
    f = ((b16 << 16).view(np.float32))
    vals = b16[np.isfinite(f) & (np.abs(f) <= 448.0)].astype(np.uint16)
    per = 127
    nblk = (len(vals) + per - 1) // per
    H = 128 * 8
    T = 2 * ((nblk + 15) // 16)                         # even, so that R = 2 divides it
    x = np.zeros((T * 8, 128), np.uint16)
    x[:, 0] = 0x43E0                                   # 448.0
    flat = x[:nblk, 1:].reshape(-1)
    flat[:len(vals)] = vals
    x[:nblk, 1:] = flat.reshape(nblk, per)
    x = x.reshape(T, H)
    # other blocks: random scales to exercise the division
    rng = np.random.default_rng(3)
    idx = np.stack([rng.permutation(8)[:2] for _ in range(T)]).astype(np.int32)
    wts = np.full((T, 2), 0.5, np.float32)
    shape = dict(T=T, H=H, E=8, k=2, R=2, C=1)
    say(f"fp8 codec sweep T={T}")
    bb = alloc_buffers(shape, ubep.FP8_E4M3, x_bits=x, topk_idx=idx, topk_w=wts)
    run_path(bb)
    torch.cuda.synchronize()
    L = oracle.layout(idx, 8, 2)
    q, sc = oracle.dispatch_fp8(x, L["pos"])
    np.testing.assert_array_equal(to_np(bb.recv_scale), sc)
    np.testing.assert_array_equal(to_np(bb.recv), q)
    np.testing.assert_array_equal(to_np(bb.y), oracle.identity_fp8(q, sc))


def test_fp8_random_scales_bit_exact():
    rng = np.random.default_rng(11)
    T, H = 512, 1024
    x32 = rng.standard_normal((T, H)).astype(np.float32) * np.exp(rng.uniform(-8, 8, (T, H // 128, 1))
                                                                  ).repeat(128, 2).reshape(T, H)
    x = torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    idx = np.stack([rng.permutation(16)[:4] for _ in range(T)]).astype(np.int32)
    wts = rng.random((T, 4)).astype(np.float32)
    shape = dict(T=T, H=H, E=16, k=4, R=4, C=1)
    say("fp8 random scales")
    bb = alloc_buffers(shape, ubep.FP8_E4M3, x_bits=x, topk_idx=idx, topk_w=wts)
    run_path(bb)
    torch.cuda.synchronize()
    L = oracle.layout(idx, 16, 4)
    q, sc = oracle.dispatch_fp8(x, L["pos"])
    np.testing.assert_array_equal(to_np(bb.recv_scale), sc)
    np.testing.assert_array_equal(to_np(bb.recv), q)
    y = oracle.identity_fp8(q, sc)
    np.testing.assert_array_equal(to_np(bb.out), oracle.combine(y, L["pos"], wts))


def test_combine_arbitrary_y_and_weights():
    """Combine on y that is not a copy of x (independent rows, signed weights)."""
    rng = np.random.default_rng(21)
    T, H, E, k, R = 304, 2048, 32, 6, 8
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = (rng.standard_normal((T, k)) * 2).astype(np.float32)
    y32 = rng.standard_normal((T * k, H)).astype(np.float32) * 4
    y = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    shape = dict(T=T, H=H, E=E, k=k, R=R, C=1)
    say("combine arbitrary y")
    b = alloc_buffers(shape, ubep.BF16, topk_idx=idx, topk_w=w)
    got = gpu_layout(b)
    yd = torch.from_numpy(y.view(np.int16)).cuda().view(torch.bfloat16)
    ubep.ubep_combine(shape, yd, b.pos, b.topk_w, b.out, b.ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(b.out), oracle.combine(y, got["pos"], w))


def test_identity_property_full_size():
    """Any size: with identity experts every output is within one bf16 ulp of x."""
    w = workload("dsv3_decode_zipf_T4096_H7168_E256_k8_R32")
    say("identity property dsv3 zipf")
    b = upload(w)
    run_path(b)
    torch.cuda.synchronize()
    xo = b.x.view(torch.int16).to(torch.int32)
    oo = b.out.view(torch.int16).to(torch.int32)
    same_sign = (xo < 0) == (oo < 0)
    d = (xo - oo).abs()
    assert int(d[same_sign & (xo != 0)].max()) <= 1

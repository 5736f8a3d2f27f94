"""GPU parity of the expert-grouped layout (ubep_layout_grouped) against the
oracle, bit-exact, and of dispatch + combine driven by its positions."""
import numpy as np
import pytest
import torch

import combine_top_route_amd as ubep
import oracle
from workloads import custom
from gpu_helpers import device_status, say, to_np, upload, workload

pytestmark = pytest.mark.gpu

KEYS = ("pos", "expert_count", "expert_offset", "rank_count", "recv_offset", "send_offset",
        "chunk_offset", "recv_src")

# single-workgroup layout (<= 4096 rows, few keys), gather mode, look-back
# mode (65536 rows x 256 experts, or capped workers), ragged tails, k = 1, k = E
SPECS = [
    dict(T=128, H=64, E=8, k=2, R=2, C=1, routing="topk", seed=31),
    dict(T=512, H=256, E=16, k=3, R=4, C=4, routing="topk", seed=32),
    dict(T=960, H=520, E=24, k=5, R=6, C=5, routing="zipf", seed=33),
    dict(T=2048, H=1024, E=64, k=8, R=8, C=8, routing="zipf", seed=34),
    dict(T=96, H=128, E=12, k=1, R=12, C=96, routing="topk", seed=35),
    dict(T=4096, H=64, E=256, k=8, R=32, C=2, routing="topk", seed=36),
    dict(T=1000, H=64, E=10, k=10, R=5, C=1, routing="topk", seed=37),
    dict(T=8192, H=16, E=256, k=8, R=16, C=4, routing="zipf", seed=38),
    dict(T=16384, H=16, E=512, k=4, R=64, C=16, routing="topk", seed=39),
]
SPEC_IDS = [f"T{s['T']}E{s['E']}k{s['k']}R{s['R']}C{s['C']}" for s in SPECS]


def _grouped(b):
    s = b.shape
    eoff = torch.empty(s["E"] + 1, dtype=torch.int32, device="cuda")
    ubep.ubep_layout_grouped(s, b.topk_idx, b.pos, b.expert_count, eoff, b.rank_count,
                             b.recv_offset, b.send_offset, b.chunk_offset if s["C"] > 1 else None,
                             b.recv_src, b.ws)
    torch.cuda.synchronize()
    got = {k: to_np(getattr(b, k)) for k in KEYS if k != "expert_offset"}
    got["expert_offset"] = to_np(eoff)
    return got


def _assert_equal(got, ref, C):
    for key in KEYS:
        if key == "chunk_offset" and C == 1:
            continue
        a, r = np.asarray(got[key]).ravel(), np.asarray(ref[key]).ravel()
        if not np.array_equal(a, r):
            bad = np.flatnonzero(a != r)
            raise AssertionError(f"{key}: {bad.size} mismatches, first at {bad[:5]}: "
                                 f"gpu {a[bad[:5]]} oracle {r[bad[:5]]}")


@pytest.mark.parametrize("cap", [0, 3], ids=["default", "cap3"])
@pytest.mark.parametrize("spec", SPECS, ids=SPEC_IDS)
def test_grouped_layout_and_path_bit_exact(spec, cap):
    w = custom(weights="softmax", **spec)
    s = w.shape
    say(f"grouped layout {spec} cap={cap}")
    b = upload(w)
    ubep.ubep_set_layout_workers(cap)
    try:
        got = _grouped(b)
    finally:
        ubep.ubep_set_layout_workers(0)
    assert device_status(b) == ubep.OK
    ref = oracle.layout_grouped(w.topk_idx, s.E, s.R, s.C)
    _assert_equal(got, ref, s.C)
    # dispatch and combine take the grouped positions unchanged
    ubep.ubep_dispatch(b.shape, ubep.BF16, b.x, b.pos, b.recv, None, b.ws)
    ubep.ubep_combine(b.shape, b.recv, b.pos, b.topk_w, b.out, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    recv = oracle.dispatch_bf16(w.x, ref["pos"])
    np.testing.assert_array_equal(to_np(b.recv), recv)
    np.testing.assert_array_equal(to_np(b.out), oracle.combine(recv, ref["pos"], w.topk_w))


@pytest.mark.parametrize("name", ["dsv3_decode_T4096_H7168_E256_k8_R32",
                                  "dsv3_decode_zipf_T4096_H7168_E256_k8_R32",
                                  "qwen3_prefill_fp8_T16384_H4096_E128_k8_R16",
                                  "prefill_grouped_zipf_T65536_H7168_E256_k8_R64_C16"])
def test_grouped_layout_full_size(name):
    w = workload(name)
    s = w.shape
    say(f"grouped layout full size {name}")
    b = upload(w)
    got = _grouped(b)
    assert device_status(b) == ubep.OK
    _assert_equal(got, oracle.layout_grouped(w.topk_idx, s.E, s.R, s.C), s.C)


def test_orders_alternate_on_one_workspace():
    """Rank-order and expert-order calls share the workspace's epoch state."""
    w = custom(T=4096, H=16, E=256, k=8, R=32, C=4, routing="zipf", weights="softmax", seed=40)
    s = w.shape
    say("alternating layout orders")
    b = upload(w)
    ref_g = oracle.layout_grouped(w.topk_idx, s.E, s.R, s.C)
    ref_r = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    for i in range(3):
        _assert_equal(_grouped(b), ref_g, s.C)
        ubep.ubep_layout(s.as_dict(), b.topk_idx, b.pos, b.expert_count, b.rank_count,
                         b.recv_offset, b.send_offset, b.chunk_offset, b.recv_src, b.ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(b.pos), ref_r["pos"])
        np.testing.assert_array_equal(to_np(b.recv_src), ref_r["recv_src"])
    assert device_status(b) == ubep.OK


@pytest.mark.parametrize("T", [128, 8192])
def test_grouped_bad_expert_id_reported(T):
    w = custom(T=T, H=16, E=64, k=4, R=8, C=1, routing="topk", weights="softmax", seed=41)
    idx = w.topk_idx.copy()
    idx[T // 3, 2] = 64
    say(f"grouped bad id T={T}")
    b = upload(w)
    b.topk_idx.copy_(torch.from_numpy(idx).cuda())
    got = _grouped(b)
    assert device_status(b) == ubep.ERR_BAD_EXPERT_ID
    assert np.all((got["pos"] >= 0) & (got["pos"] < T * 4))


@pytest.mark.parametrize("pipeline", ["chunked", "sentinel"])
def test_pipelines_take_grouped_positions(pipeline):
    """The one-launch pipelines move rows by pos, whatever its order: with the
    expert-grouped layout they give the oracle's combine bit for bit."""
    w = custom(T=2048, H=512, E=64, k=6, R=8, C=4, routing="zipf", weights="softmax", seed=42)
    s = w.shape
    say(f"grouped positions through the {pipeline} pipeline")
    b = upload(w)
    _grouped(b)
    if pipeline == "chunked":
        ubep.ubep_dispatch_combine_chunked(b.shape, b.x, b.pos, b.topk_w, b.recv, b.out,
                                           [3, 1, 0, 2], b.ws)
    else:
        ubep.ubep_recv_sentinel_init(b.recv, s.T * s.k, s.H)
        ubep.ubep_dispatch_combine_sentinel(b.shape, b.x, b.pos, b.topk_w, b.recv, b.out, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    L = oracle.layout_grouped(w.topk_idx, s.E, s.R, s.C)
    recv = oracle.dispatch_bf16(w.x, L["pos"])
    np.testing.assert_array_equal(to_np(b.out), oracle.combine(recv, L["pos"], w.topk_w))

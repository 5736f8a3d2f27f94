"""GPU parity of ubep_gate (top-k router) against the oracle gate, through the
C ABI.  Bar: expert ids bit-exact (both sides decide every selection with the
same fp32 comparisons); weights within 32 fp32 ulps of the oracle's
(double-evaluated, rounded once): the kernel's expf is within 1-2 ulps per
term, the fp32 sum of k <= 32 terms adds at most k/2 ulps, the division half
an ulp, so (k/2 + 4) <= 20 ulps, rounded up."""
import numpy as np
import pytest
import torch

import combine_top_route_amd as ubep
import oracle
from combine_top_route_amd.buffers import alloc_buffers, run_path
from workloads import CONFIGS, router_logits
from gpu_helpers import device_status, say, to_np

pytestmark = pytest.mark.gpu

WEIGHT_ULPS = 32
NORM = {"softmax": (ubep.GATE_SOFTMAX, oracle.SOFTMAX), "sigmoid": (ubep.GATE_SIGMOID, oracle.SIGMOID)}


def _ulps(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def _gpu_gate(z, k, groups=1, keep=1, norm="softmax"):
    T, E = z.shape
    zt = torch.from_numpy(np.ascontiguousarray(z, np.float32)).cuda()
    idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), -1.0, dtype=torch.float32, device="cuda")
    ubep.ubep_gate(T, E, k, zt, idx, w, groups, keep, NORM[norm][0])
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy()


def _compare(z, k, groups=1, keep=1, norm="softmax"):
    gi, gw = _gpu_gate(z, k, groups, keep, norm)
    oi, ow = oracle.gate(z, k, groups, keep, NORM[norm][1])
    np.testing.assert_array_equal(gi, oi)
    assert _ulps(gw, ow).max() <= WEIGHT_ULPS, _ulps(gw, ow).max()
    return gi, gw


@pytest.mark.parametrize("name", ["tiny_T128_H1024_E8_k2_R2", "dsv3_decode_T4096_H7168_E256_k8_R32",
                                  "dsv3_decode_zipf_T4096_H7168_E256_k8_R32",
                                  "qwen3_prefill_fp8_T16384_H4096_E128_k8_R16",
                                  "prefill_grouped_zipf_T65536_H7168_E256_k8_R64_C16"])
def test_gate_on_workload_logits(name):
    r = CONFIGS[name]
    z = router_logits(r)
    grouped = r.routing == "group_zipf"
    say(f"gate {name}")
    _compare(z, r.shape.k, r.n_groups if grouped else 1, r.topk_groups if grouped else 1, r.weights)


@pytest.mark.parametrize("T,E,k,G,keep", [(1, 1, 1, 1, 1), (37, 8, 2, 1, 1), (300, 64, 6, 8, 3),
                                          (257, 96, 32, 3, 2), (100, 1000, 8, 50, 7),
                                          (64, 1024, 32, 64, 64), (513, 256, 8, 8, 4),
                                          (200, 130, 5, 13, 1), (70, 33, 33, 1, 1),
                                          # the 16-lanes-per-token kernel: E in {64, 128, 256},
                                          # k <= 16, groups spanning 1, 2, 4, 8 or 16 lanes
                                          (1000, 128, 8, 1, 1), (777, 256, 16, 16, 5),
                                          (129, 256, 4, 2, 1), (65, 128, 8, 4, 2),
                                          (100, 256, 12, 4, 3), (333, 64, 16, 4, 4),
                                          (50, 256, 17, 1, 1)])
@pytest.mark.parametrize("norm", ["softmax", "sigmoid"])
def test_gate_random_shapes(T, E, k, G, keep, norm):
    if k > 32:
        pytest.skip("k > 32 is beyond the library's limit")
    z = (2.0 * np.random.default_rng(T * 7 + E).standard_normal((T, E))).astype(np.float32)
    say(f"gate T={T} E={E} k={k} G={G} keep={keep} {norm}")
    _compare(z, k, G, keep, norm)


def test_gate_unaligned_logits_take_the_general_kernel():
    """Logits that are not 16-byte aligned (a view one float in) are served
    by the general kernel with the same results."""
    T, E, k = 300, 256, 8
    z = (2.0 * np.random.default_rng(9).standard_normal((T * E + 1,))).astype(np.float32)
    zt = torch.from_numpy(z).cuda()[1:].view(T, E)
    idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), -1.0, dtype=torch.float32, device="cuda")
    say("gate on unaligned logits")
    ubep.ubep_gate(T, E, k, zt, idx, w, 8, 4, ubep.GATE_SIGMOID)
    torch.cuda.synchronize()
    oi, ow = oracle.gate(z[1:].reshape(T, E), k, 8, 4, oracle.SIGMOID)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    assert _ulps(w.cpu().numpy(), ow).max() <= WEIGHT_ULPS


def test_gate_heavy_ties():
    rng = np.random.default_rng(3)
    z = rng.integers(-2, 3, size=(500, 256)).astype(np.float32)
    z[:3] = 0.0
    z[3, ::2] = -0.0
    z[4] = -0.0
    z[5, 1::2] = -0.0
    say("gate ties")
    gi, gw = _compare(z, 8, 8, 4, "softmax")
    assert gi[0].tolist() == list(range(8))
    _compare(z, 8, 1, 1, "sigmoid")


def test_gate_feeds_the_path():
    """gate -> layout -> dispatch -> combine on the gate's own outputs, every
    stage equal to the oracle on the same inputs."""
    r = CONFIGS["dsv3_decode_T4096_H7168_E256_k8_R32"]
    s = r.shape
    z = router_logits(r)
    say("gate feeds the path")
    gi, gw = _compare(z, s.k, norm=r.weights)
    x = np.random.default_rng(4).standard_normal((s.T, s.H)).astype(np.float32)
    x_bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    b = alloc_buffers(s.as_dict(), ubep.BF16, "cuda", x_bits=x_bits, topk_idx=gi, topk_w=gw)
    run_path(b)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    L = oracle.layout(gi, s.E, s.R, s.C)
    np.testing.assert_array_equal(to_np(b.pos), L["pos"])
    rows = np.random.default_rng(5).choice(s.T, 64, replace=False)
    y = oracle.dispatch_bf16(x_bits, L["pos"])
    out = oracle.combine(y, L["pos"], gw)
    np.testing.assert_array_equal(to_np(b.out)[rows], out[rows])


def test_gate_rejects_invalid_shapes_before_launch():
    z = torch.zeros((4, 16), dtype=torch.float32, device="cuda")
    i = torch.zeros((4, 4), dtype=torch.int32, device="cuda")
    w = torch.zeros((4, 4), dtype=torch.float32, device="cuda")
    for kw, code in ((dict(groups=3), ubep.ERR_INVALID_ARG), (dict(groups=4, keep_groups=5), ubep.ERR_INVALID_ARG),
                     (dict(groups=8, keep_groups=1), ubep.ERR_INVALID_ARG), (dict(norm=5), ubep.ERR_INVALID_ARG)):
        with pytest.raises(ubep.UbepError) as e:
            ubep.ubep_gate(4, 16, 4, z, i, w, **kw)
        assert e.value.code == code


GATE_LAYOUT_CASES = [
    # (workload, groups, keep): the counting kernels
    ("dsv3_decode_T4096_H7168_E256_k8_R32", 1, 1),
    ("dsv3_decode_zipf_T4096_H7168_E256_k8_R32", 1, 1),
    ("qwen3_prefill_fp8_T16384_H4096_E128_k8_R16", 1, 1),
    ("prefill_grouped_zipf_T65536_H7168_E256_k8_R64_C16", 8, 4),
]


def _gate_layout_check(z, s, groups, keep, norm, calls=2, interleave=False):
    """ubep_gate_layout against ubep_gate + ubep_layout and the oracle, on
    consecutive calls (the counts are cleared for the next call).
    interleave: a plain ubep_layout on the same workspace after each call
    (it takes other tiles: about 128 where ubep_gate_layout keeps the
    largest), checked against the oracle too."""
    from gpu_helpers import LAYOUT_KEYS, assert_layout_equal
    sd = s.as_dict() if hasattr(s, "as_dict") else dict(s)
    T, E, k = sd["T"], sd["E"], sd["k"]
    oi, ow = oracle.gate(z, k, groups, keep, NORM[norm][1])
    L = oracle.layout(oi, E, sd["R"], sd["C"])
    zt = torch.from_numpy(np.ascontiguousarray(z, np.float32)).cuda()
    b = alloc_buffers(dict(sd, H=8), ubep.BF16)
    for call in range(calls):
        for key in LAYOUT_KEYS:
            getattr(b, key).fill_(-7)
        b.topk_idx.fill_(-1)
        ubep.ubep_gate_layout(dict(sd, H=8), zt, b.topk_idx, b.topk_w, b.pos, b.expert_count,
                              b.rank_count, b.recv_offset, b.send_offset,
                              b.chunk_offset if sd["C"] > 1 else None, b.recv_src, b.ws,
                              groups=groups, keep_groups=keep, norm=NORM[norm][0])
        torch.cuda.synchronize()
        assert device_status(b) == ubep.OK, call
        np.testing.assert_array_equal(to_np(b.topk_idx), oi)
        assert _ulps(to_np(b.topk_w), ow).max() <= WEIGHT_ULPS
        assert_layout_equal({key: to_np(getattr(b, key)) for key in LAYOUT_KEYS}, L, sd["C"])
        if interleave:
            for key in LAYOUT_KEYS:
                getattr(b, key).fill_(-7)
            ubep.ubep_layout(dict(sd, H=8), b.topk_idx, b.pos, b.expert_count, b.rank_count,
                             b.recv_offset, b.send_offset, b.chunk_offset if sd["C"] > 1 else None,
                             b.recv_src, b.ws)
            torch.cuda.synchronize()
            assert device_status(b) == ubep.OK, call
            assert_layout_equal({key: to_np(getattr(b, key)) for key in LAYOUT_KEYS}, L, sd["C"])


def test_gate_layout_and_layout_share_a_workspace():
    """The decode shape: ubep_gate_layout (32 tiles of 1024 rows) and
    ubep_layout (128 tiles of 256 rows) alternating on one workspace."""
    r = CONFIGS["dsv3_decode_T4096_H7168_E256_k8_R32"]
    say("gate_layout and layout alternating")
    _gate_layout_check(router_logits(r), r.shape, 1, 1, r.weights, calls=3, interleave=True)


@pytest.mark.parametrize("name,groups,keep", GATE_LAYOUT_CASES, ids=[c[0] for c in GATE_LAYOUT_CASES])
def test_gate_layout_matches_gate_then_layout(name, groups, keep):
    r = CONFIGS[name]
    say(f"gate_layout {name}")
    _gate_layout_check(router_logits(r), r.shape, groups, keep, r.weights)


@pytest.mark.parametrize("T,E,k,R,C,groups,keep", [
    (4096, 64, 6, 8, 2, 8, 3),        # E = 64, two chunks
    (2048, 128, 16, 16, 4, 4, 2),     # k = 16
    (512, 96, 4, 4, 1, 1, 1),         # E = 96: the two separate calls
    (96, 256, 8, 32, 1, 1, 1),        # tiles of 3 tokens: the two separate calls
])
def test_gate_layout_shapes(T, E, k, R, C, groups, keep):
    z = (2.0 * np.random.default_rng(T + E).standard_normal((T, E))).astype(np.float32)
    say(f"gate_layout T={T} E={E} k={k} R={R} C={C} G={groups}/{keep}")
    _gate_layout_check(z, dict(T=T, E=E, k=k, R=R, C=C), groups, keep, "sigmoid")

"""The allocation-free layout (ubep_layout_noalloc) through the C ABI: its
outputs must equal ubep_layout's (with a caller workspace) bit for bit, on
consecutive calls that share the library's per-device scratch array, the
second with a smaller input; shapes whose workspace exceeds the array are
rejected before anything runs."""
import numpy as np
import pytest
import torch

import combine_top_route_amd as ubep
import oracle
from combine_top_route_amd.buffers import alloc_buffers
from workloads import custom, make_config
from gpu_helpers import LAYOUT_KEYS, assert_layout_equal, device_status, say, to_np, upload

pytestmark = pytest.mark.gpu


def _outputs(b):
    return {k: to_np(getattr(b, k)).copy() for k in LAYOUT_KEYS}


def _noalloc(b, status, reset=0):
    s = b.shape
    for k in LAYOUT_KEYS:
        getattr(b, k).fill_(-7)
    ubep.ubep_layout_noalloc(s, b.topk_idx, b.pos, b.expert_count, b.rank_count, b.recv_offset,
                             b.send_offset, b.chunk_offset if s["C"] > 1 else None, b.recv_src,
                             status, reset)
    torch.cuda.synchronize()
    return _outputs(b)


def _with_workspace(b):
    s = b.shape
    for k in LAYOUT_KEYS:
        getattr(b, k).fill_(-7)
    ubep.ubep_layout(s, b.topk_idx, b.pos, b.expert_count, b.rank_count, b.recv_offset,
                     b.send_offset, b.chunk_offset if s["C"] > 1 else None, b.recv_src, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    return _outputs(b)


def _same(a, b, C):
    for k in LAYOUT_KEYS:
        if k == "chunk_offset" and C == 1:
            continue
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_noalloc_layout_matches_workspace_layout_on_consecutive_calls():
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cases = [make_config("dsv3_decode_zipf_T4096_H7168_E256_k8_R32"),          # 128 tiles
             custom(T=1024, H=8, E=64, k=8, R=16, C=4, routing="zipf", seed=71),  # smaller
             custom(T=96, H=8, E=12, k=3, R=6, C=2, routing="topk", seed=72),     # one workgroup
             make_config("prefill_grouped_zipf_T65536_H7168_E256_k8_R64_C16")]    # 128 tiles
    for w in cases:
        s = w.shape
        say(f"noalloc layout {s}")
        b = alloc_buffers(dict(s.as_dict(), H=8), ubep.BF16, topk_idx=w.topk_idx)
        got = _noalloc(b, status)
        assert int(status.item()) == ubep.OK
        ref = _with_workspace(b)
        _same(got, ref, s.C)
        assert_layout_equal(got, oracle.layout(w.topk_idx, s.E, s.R, s.C), s.C)
        again = _noalloc(b, status)                                # the array as the call left it
        assert int(status.item()) == ubep.OK
        _same(again, ref, s.C)


def test_noalloc_layout_reports_errors_and_resets():
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    idx = np.tile(np.arange(8, dtype=np.int32)[None, :2], (1024, 1))
    idx[5, 1] = 99                                                   # E = 8: out of range
    b = alloc_buffers(dict(T=1024, H=8, E=8, k=2, R=2, C=1), ubep.BF16, topk_idx=idx)
    say("noalloc layout bad id")
    _noalloc(b, status)
    assert int(status.item()) == ubep.ERR_BAD_EXPERT_ID
    status.zero_()
    idx[5, 1] = 3
    b.topk_idx.copy_(torch.from_numpy(idx).cuda())
    got = _noalloc(b, status, reset=1)
    assert int(status.item()) == ubep.OK
    assert_layout_equal(got, oracle.layout(idx, 8, 2, 1), 1)


def test_noalloc_layout_falls_back_to_larger_tiles():
    """A shape whose workspace (laid out for about 128 tiles) exceeds the
    array, while its largest tiles need less: the call takes those tiles."""
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    w = custom(T=16384, H=8, E=2048, k=8, R=64, C=1, routing="topk", seed=73)
    s = w.shape
    assert ubep.ubep_workspace_bytes(s.as_dict()) > 8 << 20
    say(f"noalloc layout larger tiles {s}")
    b = alloc_buffers(s.as_dict(), ubep.BF16, topk_idx=w.topk_idx)
    got = _noalloc(b, status)
    assert int(status.item()) == ubep.OK
    assert_layout_equal(got, oracle.layout(w.topk_idx, s.E, s.R, s.C), s.C)


def test_noalloc_layout_rejects_shapes_beyond_the_array():
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    shape = dict(T=1 << 20, H=8, E=256, k=8, R=64, C=16)            # about 24 MiB of workspace
    assert ubep.ubep_workspace_bytes(shape) > 8 << 20
    t = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(ubep.UbepError) as e:
        ubep.ubep_layout_noalloc(shape, t, t, t, t, t, t, t, None, status)
    assert e.value.code == ubep.ERR_UNSUPPORTED
    with pytest.raises(ubep.UbepError) as e:                        # no status word
        ubep.ubep_layout_noalloc(dict(T=8, H=8, E=4, k=2, R=2, C=1), t, t, t, t, t, t, None, None,
                                 None)
    assert e.value.code == ubep.ERR_INVALID_ARG

"""The path captured in a HIP graph (torch.cuda.CUDAGraph on ROCm) and
replayed: every replay, with eager library work between replays, must give
the eager result bit for bit.  The kernels use no memset nodes; the layout's
and the chunk pipeline's counters live in the workspace and reset themselves
at the end of every call, so a replayed call finds them as an eager one does."""
import numpy as np
import pytest
import torch

import combine_top_route_amd as ubep
import oracle
from combine_top_route_amd.buffers import alloc_buffers, run_path
from workloads import custom, make_config
from gpu_helpers import device_status, say, to_np, upload

pytestmark = pytest.mark.gpu


def _replay_and_check(b, eager_out, eager_pos, chunked, other):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):            # one eager call on the capture stream first
        run_path(b, stream=s, chunked=chunked)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run_path(b, stream=torch.cuda.current_stream(), chunked=chunked)
    for r in range(4):
        b.out.zero_()
        b.pos.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert device_status(b) == ubep.OK, r
        np.testing.assert_array_equal(to_np(b.pos), eager_pos)
        np.testing.assert_array_equal(to_np(b.out), eager_out)
        run_path(other)                   # eager work on other buffers between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("chunked", [False, True], ids=["unfused", "chunked"])
def test_graph_replays_match_eager(chunked):
    w = custom(T=1024, H=512, E=64, k=8, R=16, C=4, routing="zipf", seed=41)
    L = oracle.layout(w.topk_idx, 64, 16, 4)
    ref = oracle.combine(oracle.dispatch_bf16(w.x, L["pos"]), L["pos"], w.topk_w)
    b = upload(w)
    other = upload(custom(T=256, H=128, E=16, k=4, R=4, C=2, seed=42))
    say(f"graph replay chunked={chunked}")
    _replay_and_check(b, ref, L["pos"], chunked, other)


def test_graph_replays_decode_shape():
    w = make_config("dsv3_decode_T4096_H7168_E256_k8_R32")
    s = w.shape
    b = upload(w)
    run_path(b)
    torch.cuda.synchronize()
    # the eager result the replays must reproduce is itself the oracle's
    L = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    eager_out, eager_pos = to_np(b.out).copy(), to_np(b.pos).copy()
    np.testing.assert_array_equal(eager_pos, L["pos"])
    np.testing.assert_array_equal(eager_out,
                                  oracle.combine(oracle.dispatch_bf16(w.x, L["pos"]), L["pos"],
                                                 w.topk_w))
    other = upload(custom(T=128, H=1024, E=8, k=2, R=2, seed=43))
    say("graph replay decode shape")
    _replay_and_check(b, eager_out, eager_pos, False, other)

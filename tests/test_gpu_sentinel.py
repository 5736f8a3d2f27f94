"""GPU parity of the sentinel-polling pipeline (ubep_dispatch_combine_sentinel):
token-granular readiness carried by the first 16 bytes of each receive row.
Bar: out bit-exact to the oracle's dispatch + combine; recv equal to the
oracle's dispatch except channels 0..7 of every row, which hold the sentinel
again after the call; errors and time-outs reported, never hung."""
import numpy as np
import pytest
import torch

import combine_top_route_amd as ubep
import oracle
from combine_top_route_amd.buffers import run_path
from workloads import custom
from gpu_helpers import device_status, say, to_np, upload, workload

pytestmark = pytest.mark.gpu

SENT = 0xFFFF

SPECS = [
    dict(T=128, H=1024, E=8, k=2, R=2, C=1, routing="topk", seed=51),
    dict(T=512, H=256, E=16, k=3, R=4, C=1, routing="topk", seed=52),
    dict(T=960, H=520, E=24, k=5, R=6, C=1, routing="zipf", seed=53),     # ragged row tail
    dict(T=2048, H=1024, E=64, k=8, R=8, C=1, routing="zipf", seed=54),
    dict(T=97 * 2, H=64, E=10, k=10, R=2, C=1, routing="topk", seed=55),   # k = E, tiny rows
    dict(T=3, H=8, E=3, k=1, R=3, C=1, routing="topk", seed=56),           # one unit per row
]


def _layout(b):
    s = b.shape
    ubep.ubep_layout(s, b.topk_idx, b.pos, b.expert_count, b.rank_count, b.recv_offset,
                     b.send_offset, None, b.recv_src, b.ws)


def _run(b, **kw):
    ubep.ubep_dispatch_combine_sentinel(b.shape, b.x, b.pos, b.topk_w, b.recv, b.out, b.ws, **kw)
    torch.cuda.synchronize()


def _check_recv(recv, ref):
    """recv == the oracle's dispatch, except channels 0..7 (the sentinel)."""
    got = to_np(recv)
    assert np.all(got[:, :8] == SENT)
    np.testing.assert_array_equal(got[:, 8:], ref[:, 8:])


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: f"T{s['T']}H{s['H']}E{s['E']}k{s['k']}")
def test_sentinel_pipeline_bit_exact(spec):
    w = custom(weights="softmax", **spec)
    s = w.shape
    say(f"sentinel pipeline {spec}")
    b = upload(w)
    ubep.ubep_recv_sentinel_init(b.recv, s.T * s.k, s.H)
    _layout(b)
    L = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    recv = oracle.dispatch_bf16(w.x, L["pos"])
    out = oracle.combine(recv, L["pos"], w.topk_w)
    for call in range(2):          # the second call relies on the restored sentinels
        b.out.zero_()
        _run(b)
        assert device_status(b) == ubep.OK, call
        np.testing.assert_array_equal(to_np(b.out), out)
        _check_recv(b.recv, recv)


@pytest.mark.parametrize("name", ["dsv3_decode_T4096_H7168_E256_k8_R32",
                                  "dsv3_decode_zipf_T4096_H7168_E256_k8_R32"])
def test_sentinel_pipeline_full_size(name):
    w = workload(name)
    s = w.shape
    say(f"sentinel pipeline full size {name}")
    b = upload(w)
    run_path(b)                                    # unfused reference on the device
    torch.cuda.synchronize()
    ref_out = b.out.clone()
    ubep.ubep_recv_sentinel_init(b.recv, s.T * s.k, s.H)
    b.out.zero_()
    _run(b)
    assert device_status(b) == ubep.OK
    assert torch.equal(b.out.view(torch.int16), ref_out.view(torch.int16))
    head = b.recv[:, :8].contiguous().view(torch.int16)
    assert bool((head == -1).all())
    # every dispatched row past channel 7: recv[pos[t][j], 8:] == x[t, 8:]
    got = b.recv.index_select(0, b.pos.reshape(-1).long()).view(s.T, s.k, s.H)[:, :, 8:]
    want = b.x[:, 8:].unsqueeze(1).expand(-1, s.k, -1)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    rng = np.random.default_rng(5)
    toks = np.unique(np.concatenate([[0, s.T - 1], rng.integers(0, s.T, 48)]))
    _, out_ref = oracle.pipeline_tokens(w.x, w.topk_idx, w.topk_w, s.E, s.R, tokens=toks)
    np.testing.assert_array_equal(to_np(b.out[torch.from_numpy(toks).cuda()]), out_ref)


def test_sentinel_timeout_is_reported_not_hung():
    w = custom(T=256, H=256, E=16, k=4, R=4, C=1, seed=57)
    s = w.shape
    b = upload(w)
    ubep.ubep_recv_sentinel_init(b.recv, s.T * s.k, s.H)
    _layout(b)
    say("sentinel time-out (row heads withheld, 20 us limit)")
    _run(b, spin_limit_ns=20000, debug_flags=1)
    assert device_status(b) == ubep.ERR_TIMEOUT
    assert np.all(to_np(b.recv)[:, :8] == SENT)      # sentinels are still in place
    _run(b)                                          # and a normal call afterwards is exact
    assert device_status(b) == ubep.OK
    L = oracle.layout(w.topk_idx, s.E, s.R)
    out = oracle.combine(oracle.dispatch_bf16(w.x, L["pos"]), L["pos"], w.topk_w)
    np.testing.assert_array_equal(to_np(b.out), out)


def test_sentinel_word_in_input_is_reported():
    w = custom(T=64, H=128, E=8, k=2, R=2, C=1, seed=58)
    s = w.shape
    x = w.x.copy()
    x[9, 2:4] = SENT                                  # an aligned channel pair 0xFFFF 0xFFFF
    b = upload(w)
    b.x.copy_(torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16))
    ubep.ubep_recv_sentinel_init(b.recv, s.T * s.k, s.H)
    _layout(b)
    say("sentinel word in x")
    _run(b, spin_limit_ns=20000)
    assert device_status(b) == ubep.ERR_SENTINEL_DATA
    assert np.all(to_np(b.recv)[:, :8] == SENT)
    # every other token is still combined exactly
    L = oracle.layout(w.topk_idx, s.E, s.R)
    out = oracle.combine(oracle.dispatch_bf16(w.x, L["pos"]), L["pos"], w.topk_w)
    keep = np.arange(s.T) != 9
    np.testing.assert_array_equal(to_np(b.out)[keep], out[keep])


def test_sentinel_bad_position_skipped():
    w = custom(T=64, H=256, E=8, k=2, R=2, C=1, seed=59)
    s = w.shape
    b = upload(w)
    ubep.ubep_recv_sentinel_init(b.recv, s.T * s.k, s.H)
    _layout(b)
    torch.cuda.synchronize()
    pos0 = to_np(b.pos).copy()
    pos = pos0.copy()
    pos[20, 1] = s.T * s.k + 5                        # outside [0, T*k)
    b.pos.copy_(torch.from_numpy(pos).cuda())
    say("sentinel bad position")
    _run(b, spin_limit_ns=20000)
    assert device_status(b) == ubep.ERR_BAD_POSITION
    # the skipped slot adds nothing: fma(0, y, acc) == acc for finite y
    y = oracle.dispatch_bf16(w.x, pos0)
    wts = w.topk_w.copy()
    wts[20, 1] = 0.0
    np.testing.assert_array_equal(to_np(b.out), oracle.combine(y, pos0, wts))

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
from gpu_helpers import assert_path_whole, device_status, say, to_np, upload, workload

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
    """Full-size decode workloads: every combined token and every dispatched
    row (past the sentinel channels) against the oracle, on two calls in a row."""
    w = workload(name)
    s = w.shape
    say(f"sentinel pipeline full size {name}")
    b = upload(w)
    ubep.ubep_recv_sentinel_init(b.recv, s.T * s.k, s.H)
    _layout(b)
    torch.cuda.synchronize()
    L = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    np.testing.assert_array_equal(to_np(b.pos), L["pos"])
    for call in range(2):          # the second call relies on the restored sentinels
        b.out.zero_()
        _run(b)
        assert device_status(b) == ubep.OK, call
        head = b.recv[:, :8].contiguous().view(torch.int16)
        assert bool((head == -1).all())
        assert_path_whole(b, w, skip_channels=8)


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


def test_sentinel_late_producers_bit_exact():
    """Debug bit 1 holds every third producer back (about 25 us) before it
    writes the rows' first channels: consumers meet rows that arrive late,
    and the results stay exact on two calls in a row."""
    w = custom(T=2048, H=1024, E=64, k=8, R=8, C=1, routing="zipf", weights="softmax", seed=61)
    s = w.shape
    b = upload(w)
    ubep.ubep_recv_sentinel_init(b.recv, s.T * s.k, s.H)
    _layout(b)
    L = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    recv = oracle.dispatch_bf16(w.x, L["pos"])
    out = oracle.combine(recv, L["pos"], w.topk_w)
    for call in range(2):
        say(f"sentinel late producers, call {call}")
        b.out.zero_()
        _run(b, debug_flags=2)
        assert device_status(b) == ubep.OK, call
        np.testing.assert_array_equal(to_np(b.out), out)
        _check_recv(b.recv, recv)


def test_sentinel_gives_up_after_one_limit_whatever_the_status():
    """A bad position is recorded first, then every row head is withheld: the
    first expired wait must end all later ones although the status word
    keeps the earlier error (about one 50 ms limit in all, not one per task:
    16384 tasks on a few thousand workgroups)."""
    import time
    w = custom(T=65536, H=8, E=2, k=1, R=2, C=1, routing="topk", weights="softmax", seed=62)
    s = w.shape
    b = upload(w)
    ubep.ubep_recv_sentinel_init(b.recv, s.T * s.k, s.H)
    _layout(b)
    torch.cuda.synchronize()
    pos0 = to_np(b.pos).copy()
    pos = pos0.copy()
    pos[0, 0] = s.T * s.k + 3
    b.pos.copy_(torch.from_numpy(pos).cuda())
    say("sentinel give-up after a bad position (50 ms limit, heads withheld)")
    t0 = time.perf_counter()
    _run(b, spin_limit_ns=50_000_000, debug_flags=1)
    dt = time.perf_counter() - t0
    assert device_status(b) == ubep.ERR_BAD_POSITION
    assert dt < 0.3, f"{dt:.3f} s"
    assert np.all(to_np(b.recv)[:, :8] == SENT)
    b.pos.copy_(torch.from_numpy(pos0).cuda())      # the give-up word was reset
    _run(b)
    assert device_status(b) == ubep.OK
    out = oracle.combine(oracle.dispatch_bf16(w.x, pos0), pos0, w.topk_w)
    np.testing.assert_array_equal(to_np(b.out), out)

"""GPU edge cases and error paths, through the C ABI.

Every kernel still exits normally: bad ids and positions are detected and
recorded by the kernels' own checks; the time-out path is forced from the host
with a tiny spin limit and the debug flag that withholds the ready flags.
"""
import numpy as np
import pytest
import torch

import combine_top_route_amd as ubep
import oracle
from combine_top_route_amd.buffers import alloc_buffers, run_path
from workloads import custom
from gpu_helpers import assert_layout_equal, device_status, gpu_layout, say, to_np, upload
from gpu_helpers import workload as workload_full

pytestmark = pytest.mark.gpu


def _layout_case(T, E, k, R, C, idx, H=8):
    shape = dict(T=T, H=H, E=E, k=k, R=R, C=C)
    b = alloc_buffers(shape, ubep.BF16, topk_idx=idx)
    got = gpu_layout(b)
    assert device_status(b) == ubep.OK
    assert_layout_equal(got, oracle.layout(idx, E, R, C), C)


def test_all_rows_to_one_rank():
    T, k, E, R = 4096, 8, 256, 32
    idx = np.tile(np.arange(248, 256, dtype=np.int32), (T, 1))        # all on the last rank
    say("all rows to one rank")
    _layout_case(T, E, k, R, 4, idx)


def test_single_token_and_single_expert_per_rank():
    say("single token")
    _layout_case(1, 4, 3, 1, 1, np.array([[3, 0, 2]], np.int32))
    rng = np.random.default_rng(0)
    idx = np.stack([rng.permutation(64)[:8] for _ in range(640)]).astype(np.int32)
    say("E == R")
    _layout_case(640, 64, 8, 64, 10, idx)


@pytest.mark.parametrize("R,E,k,T,C", [(1024, 8192, 32, 2048, 256), (1024, 1024, 1, 1024, 1)])
def test_limit_shapes(R, E, k, T, C):
    rng = np.random.default_rng(R + E)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    say(f"limits R={R} E={E} k={k}")
    _layout_case(T, E, k, R, C, idx)


def test_many_rows_layout():
    """8M rows (T = 2^20, k = 8): tiles at the 4096-row maximum."""
    rng = np.random.default_rng(5)
    T, k, E, R = 1 << 20, 8, 256, 64
    idx = (np.argsort(rng.random((T, 16)), axis=1)[:, :k] * 16 + rng.integers(0, 16, (T, 1))).astype(np.int32)
    say("8M-row layout")
    _layout_case(T, E, k, R, 16, idx)


def test_workspace_reuse_across_shapes():
    """The look-back state and tickets are cleared by each call."""
    rng = np.random.default_rng(9)
    shapes = [dict(T=1024, E=32, k=4, R=8, C=4), dict(T=96, E=12, k=3, R=6, C=2),
              dict(T=1024, E=32, k=4, R=8, C=4)]
    nws = max(ubep.ubep_workspace_bytes(dict(H=8, **s)) for s in shapes)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    for s in shapes:
        idx = np.stack([rng.permutation(s["E"])[:s["k"]] for _ in range(s["T"])]).astype(np.int32)
        shape = dict(H=8, **s)
        b = alloc_buffers(shape, ubep.BF16, topk_idx=idx)
        b.ws = ws
        say(f"reuse {s}")
        got = gpu_layout(b)
        assert device_status(b) == ubep.OK
        assert_layout_equal(got, oracle.layout(idx, s["E"], s["R"], s["C"]), s["C"])


def test_bad_expert_id_reported():
    idx = np.tile(np.array([[0, 1]], np.int32), (64, 1))
    idx[17, 1] = 8                                   # E = 8: out of range
    idx[40, 0] = -3
    b = alloc_buffers(dict(T=64, H=64, E=8, k=2, R=2, C=1), ubep.BF16, topk_idx=idx)
    say("bad expert id")
    got = gpu_layout(b)
    assert device_status(b) == ubep.ERR_BAD_EXPERT_ID
    assert device_status(b) == ubep.OK               # reading clears it
    p = got["pos"].ravel()                            # positions stay a bijection in range
    assert np.array_equal(np.sort(p), np.arange(128))


def test_bad_position_reported_and_skipped():
    shape = dict(T=8, H=64, E=4, k=2, R=2, C=1)
    b = alloc_buffers(shape, ubep.BF16, topk_idx=np.zeros((8, 2), np.int32),
                      x_bits=np.full((8, 64), 0x3F80, np.uint16))
    pos = torch.arange(16, dtype=torch.int32, device="cuda").reshape(8, 2)
    pos[3, 1] = 16
    pos[5, 0] = -1
    b.recv.zero_()
    say("bad position")
    ubep.ubep_dispatch(shape, ubep.BF16, b.x, pos, b.recv, None, b.ws)
    assert device_status(b) == ubep.ERR_BAD_POSITION
    r = to_np(b.recv)
    assert np.all(r[np.setdiff1d(np.arange(16), [7, 10])] == 0x3F80)
    assert np.all(r[[7, 10]] == 0)
    ubep.ubep_combine(shape, b.recv, pos, b.topk_w, b.out, b.ws)
    assert device_status(b) == ubep.ERR_BAD_POSITION


def test_chunked_timeout_is_reported_not_hung():
    w = custom(T=256, H=256, E=16, k=4, R=4, C=4, seed=1)
    b = upload(w)
    s = w.shape.as_dict()
    ubep.ubep_layout(s, b.topk_idx, b.pos, b.expert_count, b.rank_count, b.recv_offset,
                     b.send_offset, b.chunk_offset, b.recv_src, b.ws)
    say("chunked time-out (flags withheld, 20 us limit)")
    ubep.ubep_dispatch_combine_chunked(s, b.x, b.pos, b.topk_w, b.recv, b.out, None, b.ws,
                                       spin_limit_ns=20000, debug_flags=1)
    assert device_status(b) == ubep.ERR_TIMEOUT
    # the pipeline reset its counters: a normal call afterwards is exact
    run_path(b, chunked=True)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    L = oracle.layout(w.topk_idx, 16, 4, 4)
    out = oracle.combine(oracle.dispatch_bf16(w.x, L["pos"]), L["pos"], w.topk_w)
    np.testing.assert_array_equal(to_np(b.out), out)


def test_chunked_late_producers_bit_exact():
    """Debug bit 1 holds every third D task back (about 25 us) before it
    raises its chunk's flag: C tasks wait on late chunks, results stay exact."""
    w = custom(T=2048, H=1024, E=64, k=8, R=16, C=8, routing="zipf", seed=5)
    s = w.shape
    L = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    y = oracle.dispatch_bf16(w.x, L["pos"])
    out = oracle.combine(y, L["pos"], w.topk_w)
    b = upload(w)
    sd = s.as_dict()
    ubep.ubep_layout(sd, b.topk_idx, b.pos, b.expert_count, b.rank_count, b.recv_offset,
                     b.send_offset, b.chunk_offset, b.recv_src, b.ws)
    for call in range(2):
        say(f"chunked late producers, call {call}")
        b.out.zero_()
        ubep.ubep_dispatch_combine_chunked(sd, b.x, b.pos, b.topk_w, b.recv, b.out, None, b.ws,
                                           debug_flags=2)
        torch.cuda.synchronize()
        assert device_status(b) == ubep.OK
        np.testing.assert_array_equal(to_np(b.recv), y)
        np.testing.assert_array_equal(to_np(b.out), out)


def test_chunked_gives_up_after_one_limit_whatever_the_status():
    """A bad position is recorded first, then every flag is withheld: the
    first expired wait must end all later ones (about one 50 ms limit, not
    one per C task: 16384 of them on a few thousand workgroups)."""
    import time
    w = custom(T=65536, H=8, E=2, k=1, R=2, C=256, routing="topk", seed=6)
    s = w.shape
    sd = s.as_dict()
    b = upload(w)
    ubep.ubep_layout(sd, b.topk_idx, b.pos, b.expert_count, b.rank_count, b.recv_offset,
                     b.send_offset, b.chunk_offset, b.recv_src, b.ws)
    torch.cuda.synchronize()
    pos0 = to_np(b.pos).copy()
    pos = pos0.copy()
    pos[0, 0] = s.T * s.k + 3
    b.pos.copy_(torch.from_numpy(pos).cuda())
    say("chunked give-up after a bad position (50 ms limit, flags withheld)")
    t0 = time.perf_counter()
    ubep.ubep_dispatch_combine_chunked(sd, b.x, b.pos, b.topk_w, b.recv, b.out, None, b.ws,
                                       spin_limit_ns=50_000_000, debug_flags=1)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert device_status(b) == ubep.ERR_BAD_POSITION
    assert dt < 0.3, f"{dt:.3f} s"
    b.pos.copy_(torch.from_numpy(pos0).cuda())      # the give-up word was reset
    run_path(b, chunked=True)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    out = oracle.combine(oracle.dispatch_bf16(w.x, pos0), pos0, w.topk_w)
    np.testing.assert_array_equal(to_np(b.out), out)


def _lpt_by_definition(L):
    """Chunks by descending largest per-rank row count, ties to the lower id."""
    cd = np.diff(np.vstack([L["chunk_offset"], L["rank_count"][None]]), axis=0)   # [C, R]
    return sorted(range(cd.shape[0]), key=lambda c: (-int(cd[c].max()), c))


LPT_SPECS = [dict(T=2048, H=8, E=64, k=8, R=16, C=16, routing="zipf", seed=4),
             dict(T=4096, H=8, E=256, k=8, R=32, C=256, routing="zipf", seed=7),   # many ties
             dict(T=960, H=8, E=24, k=5, R=6, C=5, routing="topk", seed=8),
             dict(T=512, H=8, E=16, k=3, R=4, C=1, routing="topk", seed=9)]


@pytest.mark.parametrize("spec", LPT_SPECS, ids=lambda s: f"T{s['T']}R{s['R']}C{s['C']}")
def test_chunk_order_lpt_matches_definition(spec):
    w = custom(**spec)
    s = w.shape
    b = upload(w)
    say(f"LPT order {spec}")
    got = gpu_layout(b)
    order = torch.full((s.C,), -1, dtype=torch.int32, device="cuda")
    ubep.ubep_chunk_order_lpt(s.as_dict(), b.chunk_offset if s.C > 1 else None, b.rank_count, order)
    torch.cuda.synchronize()
    L = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    assert_layout_equal(got, L, s.C)
    assert to_np(order).tolist() == _lpt_by_definition(L)


def test_chunk_order_lpt_large_prefill():
    w = workload_full("prefill_grouped_zipf_T65536_H7168_E256_k8_R64_C16")
    s = w.shape
    b = alloc_buffers(dict(s.as_dict(), H=8), ubep.BF16, topk_idx=w.topk_idx)
    say("LPT order, 65536-token prefill")
    gpu_layout(b)
    order = torch.full((s.C,), -1, dtype=torch.int32, device="cuda")
    ubep.ubep_chunk_order_lpt(s.as_dict(), b.chunk_offset, b.rank_count, order)
    torch.cuda.synchronize()
    L = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    want = _lpt_by_definition(L)
    assert to_np(order).tolist() == want
    assert want != list(range(s.C))                  # skew makes the order differ from identity


@pytest.mark.parametrize("order", ["identity", "reversed", "lpt", "random", "lpt-device"])
def test_chunked_order_invariance(order):
    w = custom(T=2048, H=1024, E=64, k=8, R=16, C=16, routing="zipf", seed=4)
    s = w.shape
    L = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    if order == "identity":
        o = list(range(16))
    elif order == "reversed":
        o = list(range(15, -1, -1))
    elif order == "lpt":
        o = _lpt_by_definition(L)
    elif order == "lpt-device":
        o = "lpt"
    else:
        o = list(np.random.default_rng(2).permutation(16))
    b = upload(w)
    say(f"chunk order {order}")
    run_path(b, chunked=True, chunk_order=o)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    y = oracle.dispatch_bf16(w.x, L["pos"])
    np.testing.assert_array_equal(to_np(b.recv), y)
    np.testing.assert_array_equal(to_np(b.out), oracle.combine(y, L["pos"], w.topk_w))


def test_invalid_arguments_rejected_before_launch():
    b = alloc_buffers(dict(T=8, H=64, E=4, k=2, R=2, C=1), ubep.BF16)
    with pytest.raises(ubep.UbepError) as e:
        ubep.ubep_layout(dict(T=0, H=64, E=4, k=2, R=2, C=1), b.topk_idx, b.pos, b.expert_count,
                         b.rank_count, b.recv_offset, b.send_offset, None, None, b.ws)
    assert e.value.code == ubep.ERR_INVALID_ARG
    with pytest.raises(ubep.UbepError) as e:   # workspace too small
        ubep.ubep_layout(dict(T=8, H=64, E=4, k=2, R=2, C=1), b.topk_idx, b.pos, b.expert_count,
                         b.rank_count, b.recv_offset, b.send_offset, None, None, b.ws[:16])
    assert e.value.code == ubep.ERR_INVALID_ARG
    with pytest.raises(ubep.UbepError) as e:   # bf16 dispatch with a scale buffer
        ubep.ubep_dispatch(dict(T=8, H=64, E=4, k=2, R=2, C=1), ubep.BF16, b.x, b.pos, b.recv,
                           b.topk_w, b.ws)
    assert e.value.code == ubep.ERR_INVALID_ARG
    with pytest.raises(ubep.UbepError) as e:   # chunk order not a permutation
        ubep.ubep_dispatch_combine_chunked(dict(T=8, H=64, E=4, k=2, R=2, C=2), b.x, b.pos,
                                           b.topk_w, b.recv, b.out, [0, 0], b.ws)
    assert e.value.code == ubep.ERR_INVALID_ARG


def test_fused_and_separate_calls_share_a_workspace():
    """Layout epochs and tickets hand over between the fused launch, the
    separate layout, and the chunk pipeline on one workspace."""
    w = custom(T=1024, H=512, E=64, k=8, R=16, C=4, routing="zipf", seed=12)
    s = w.shape
    L = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    y = oracle.dispatch_bf16(w.x, L["pos"])
    out = oracle.combine(y, L["pos"], w.topk_w)
    b = upload(w)
    for mode in ("fused", "separate", "fused", "chunked", "fused", "fused"):
        say(f"shared workspace: {mode}")
        b.out.zero_()
        run_path(b, fused=mode == "fused", chunked=mode == "chunked")
        torch.cuda.synchronize()
        assert device_status(b) == ubep.OK, mode
        np.testing.assert_array_equal(to_np(b.pos), L["pos"])
        np.testing.assert_array_equal(to_np(b.recv), y)
        np.testing.assert_array_equal(to_np(b.out), out)


def test_launch_timing_events_time_the_kernel_and_change_nothing():
    w = custom(T=512, H=1024, E=32, k=4, R=8, seed=31)
    s = w.shape
    b = upload(w)
    say("launch-recorded timing events")
    run_path(b)
    torch.cuda.synchronize()
    ref = to_np(b.out).copy()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    b.out.zero_()
    ubep.ubep_time_next_launch(e0, e1)
    ubep.ubep_combine(s.as_dict(), b.y, b.pos, b.topk_w, b.out, b.ws)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3
    assert 0.0 < us < 10000.0, us
    np.testing.assert_array_equal(to_np(b.out), ref)
    assert device_status(b) == ubep.OK


def _exact_path(w, b):
    s = w.shape
    L = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    y = oracle.dispatch_bf16(w.x, L["pos"])
    out = oracle.combine(y, L["pos"], w.topk_w)
    b.out.zero_()
    run_path(b)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    np.testing.assert_array_equal(to_np(b.recv), y)
    np.testing.assert_array_equal(to_np(b.out), out)


def test_block_tickets_reset_across_grids():
    """Dispatch and combine hand their later workgroups token blocks from
    ticket counters in the workspace; grids of at least eight times the
    workgroups the chip holds at once use them (65536 tokens of 4 per
    workgroup), and alternating grid sizes on one workspace must stay exact."""
    shapes = [dict(T=65536, H=64, E=64, k=4, R=16), dict(T=98304, H=128, E=32, k=4, R=8),
              dict(T=65536, H=64, E=64, k=4, R=16)]
    nws = max(ubep.ubep_workspace_bytes(dict(C=1, **s)) for s in shapes)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    for i, sh in enumerate(shapes):
        w = custom(seed=50 + i, **sh)
        b = upload(w)
        b.ws = ws
        say(f"block tickets {sh}")
        _exact_path(w, b)


def test_stale_block_ticket_is_reported_and_init_recovers():
    w = custom(T=65536, H=64, E=64, k=4, R=16, seed=60)
    b = upload(w)
    s = w.shape.as_dict()
    ubep.ubep_layout(s, b.topk_idx, b.pos, b.expert_count, b.rank_count, b.recv_offset,
                     b.send_offset, None, None, b.ws)
    ubep.ubep_dispatch(s, ubep.BF16, b.x, b.pos, b.recv, None, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    b.ws.view(torch.int32)[256] = 1 << 30          # the combine's ticket word, left behind
    say("stale combine ticket")
    ubep.ubep_combine(s, b.y, b.pos, b.topk_w, b.out, b.ws)
    assert device_status(b) == ubep.ERR_WORKSPACE
    ubep.ubep_workspace_init(b.ws)
    _exact_path(w, b)

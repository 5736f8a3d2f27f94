"""GPU parity of the per-expert linear map (ubep_expert_linear, MFMA) against
the oracle, and of the whole MoE layer it completes: expert-grouped layout ->
dispatch -> expert -> combine.

Tolerance (the GPU accumulates bf16 products in fp32 in the hardware's
order, the oracle in double; both round once to bf16).  With v32 the GPU's
fp32 sum, v the exact sum and S = sum |x_c w_c|:
  |bf16(v32) - v32| <= 2^-8 |v32|,  |v32 - v| <= H 2^-24 S  (any order),
  |bf16(v) - v| <= 2^-8 |v|
(bf16 keeps 8 significant bits, so its unit roundoff is 2^-8), hence
|gpu - oracle| <= 2^-7 max(|gpu|, |oracle|) + 2 H 2^-24 S, checked per
element: one bf16 ulp where the exact sum sits next to a rounding midpoint.  Identity weights make every sum a single product, which is exact:
there the bar is bit-exact."""
import numpy as np
import pytest
import torch

import combine_top_route_amd as ubep
import oracle
from workloads import custom
from gpu_helpers import device_status, say, to_np, upload, workload

pytestmark = pytest.mark.gpu


def _f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _grouped_layout(b):
    s = b.shape
    eoff = torch.empty(s["E"] + 1, dtype=torch.int32, device="cuda")
    ubep.ubep_layout_grouped(s, b.topk_idx, b.pos, b.expert_count, eoff, b.rank_count,
                             b.recv_offset, b.send_offset, b.chunk_offset if s["C"] > 1 else None,
                             None, b.ws)
    return eoff


def _weights(E, N, H, seed, scale):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn((E, N, H), generator=g, device="cuda") * scale).to(torch.bfloat16)


def _packed(W):
    E, N, H = W.shape
    P = torch.empty_like(W)
    ubep.ubep_expert_pack_weights(E, N, H, W, P)
    return P


def test_pack_weights_is_the_block_permutation():
    E, N, H = 3, 256, 192
    W = _weights(E, N, H, 60, 1.0)
    got = _bits(_packed(W))
    want = _bits(W).reshape(E, N // 128, 128, H // 64, 64).transpose(0, 1, 3, 2, 4).ravel()
    np.testing.assert_array_equal(got.ravel(), want)


def _check_rows(x_bits, w_bits, e_of_row, y_gpu, y_ref):
    """Per-element bound above on the rows given (x_bits [n, H], w_bits the
    weights of each row's expert via e_of_row)."""
    H = x_bits.shape[1]
    xa = np.abs(_f64(x_bits))
    S = np.stack([np.abs(_f64(w_bits[e])) @ xa[i] for i, e in enumerate(e_of_row)])
    g, r = _f64(y_gpu), _f64(y_ref)
    tol = 2.0 ** -7 * np.maximum(np.abs(g), np.abs(r)) + 2 * H * 2.0 ** -24 * S
    bad = np.abs(g - r) > tol
    if bad.any():
        for i, n in np.argwhere(bad)[:4]:
            exact = float(_f64(w_bits[e_of_row[i]])[n] @ _f64(x_bits)[i])
            say(f"row {i} col {n}: gpu {g[i, n]!r} oracle {r[i, n]!r} exact {exact!r} "
                f"S {S[i, n]!r} tol {tol[i, n]!r}")
    assert not bad.any(), f"{bad.sum()} elements outside the bound; first {np.argwhere(bad)[:3]}"


SPECS = [
    dict(T=512, H=256, E=8, k=2, R=2, C=1, N=256, routing="zipf", seed=61),
    dict(T=1000, H=1024, E=16, k=4, R=4, C=1, N=384, routing="topk", seed=62),
    dict(T=96, H=64, E=32, k=3, R=8, C=1, N=128, routing="zipf", seed=63),   # many empty experts
    dict(T=2048, H=512, E=64, k=8, R=8, C=1, N=128, routing="topk", seed=64),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: f"T{s['T']}H{s['H']}E{s['E']}k{s['k']}N{s['N']}")
def test_expert_linear_matches_oracle(spec):
    spec = dict(spec)
    N = spec.pop("N")
    w = custom(weights="softmax", **spec)
    s = w.shape
    say(f"expert linear {spec} N={N}")
    b = upload(w)
    eoff = _grouped_layout(b)
    ubep.ubep_dispatch(b.shape, ubep.BF16, b.x, b.pos, b.recv, None, b.ws)
    W = _weights(s.E, N, s.H, spec["seed"], 0.05)
    y = torch.empty((s.T * s.k, N), dtype=torch.bfloat16, device="cuda")
    ubep.ubep_expert_linear(b.shape, N, eoff, b.recv, _packed(W), y, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    off = to_np(eoff)
    xr, wb = _bits(b.recv), _bits(W)
    ref = oracle.expert_linear(xr, wb, off)
    e_of_row = np.repeat(np.arange(s.E), np.diff(off))
    _check_rows(xr, wb, e_of_row, _bits(y), ref)


def test_identity_weights_are_bit_exact():
    """w[e] = I: every output is one exact product, so y == x bit for bit."""
    w = custom(T=640, H=256, E=8, k=3, R=4, C=1, routing="zipf", weights="softmax", seed=65)
    s = w.shape
    say("expert linear identity weights")
    b = upload(w)
    eoff = _grouped_layout(b)
    ubep.ubep_dispatch(b.shape, ubep.BF16, b.x, b.pos, b.recv, None, b.ws)
    W = torch.eye(s.H, device="cuda", dtype=torch.bfloat16).expand(s.E, -1, -1).contiguous()
    y = torch.full((s.T * s.k, s.H), 7.0, dtype=torch.bfloat16, device="cuda")
    ubep.ubep_expert_linear(b.shape, s.H, eoff, b.recv, _packed(W), y, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    assert torch.equal(y.view(torch.int16), b.recv.view(torch.int16))


def test_moe_layer_end_to_end():
    """layout (expert order) -> dispatch -> expert -> combine; combine is
    bit-exact on the GPU's expert outputs, the expert within the bound."""
    w = custom(T=768, H=512, E=16, k=4, R=4, C=1, routing="zipf", weights="softmax", seed=66)
    s = w.shape
    say("moe layer end to end")
    b = upload(w)
    eoff = _grouped_layout(b)
    ubep.ubep_dispatch(b.shape, ubep.BF16, b.x, b.pos, b.recv, None, b.ws)
    W = _weights(s.E, s.H, s.H, 66, 0.04)
    y = torch.empty((s.T * s.k, s.H), dtype=torch.bfloat16, device="cuda")
    ubep.ubep_expert_linear(b.shape, s.H, eoff, b.recv, _packed(W), y, b.ws)
    ubep.ubep_combine(b.shape, y, b.pos, b.topk_w, b.out, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    L = oracle.layout_grouped(w.topk_idx, s.E, s.R)
    np.testing.assert_array_equal(to_np(b.pos), L["pos"])
    np.testing.assert_array_equal(to_np(eoff), L["expert_offset"])
    recv = oracle.dispatch_bf16(w.x, L["pos"])
    wb = _bits(W)
    ref = oracle.expert_linear(recv, wb, L["expert_offset"])
    e_of_row = np.repeat(np.arange(s.E), np.diff(L["expert_offset"]))
    yg = _bits(y)
    _check_rows(recv, wb, e_of_row, yg, ref)
    np.testing.assert_array_equal(to_np(b.out), oracle.combine(yg, L["pos"], w.topk_w))


def test_expert_linear_full_depth_sampled():
    """The DeepSeek-V3 decode shape (H = 7168, 256 experts, Zipf routing) with
    N = 512 output channels; sampled rows of hot, cold and boundary experts."""
    wl = workload("dsv3_decode_zipf_T4096_H7168_E256_k8_R32")
    s = wl.shape
    N = 512
    say("expert linear full depth sampled")
    b = upload(wl)
    eoff = _grouped_layout(b)
    ubep.ubep_dispatch(b.shape, ubep.BF16, b.x, b.pos, b.recv, None, b.ws)
    W = _weights(s.E, N, s.H, 67, 0.02)
    y = torch.empty((s.T * s.k, N), dtype=torch.bfloat16, device="cuda")
    ubep.ubep_expert_linear(b.shape, N, eoff, b.recv, _packed(W), y, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.OK
    off = to_np(eoff)
    cnt = np.diff(off)
    hot = int(np.argmax(cnt))
    picks = [hot, int(np.argmin(np.where(cnt > 0, cnt, 1 << 30))), 0, s.E - 1, s.E // 2]
    rng = np.random.default_rng(7)
    for e in dict.fromkeys(picks):
        if cnt[e] == 0:
            continue
        rows = np.unique(np.concatenate([[off[e], off[e + 1] - 1],
                                         rng.integers(off[e], off[e + 1], 6)]))
        xr = _bits(b.recv[torch.from_numpy(rows).cuda()])
        we = _bits(W[e])[None]
        sub_off = np.array([0, len(rows)], np.int32)
        ref = oracle.expert_linear(xr, we, sub_off)
        _check_rows(xr, we, np.zeros(len(rows), int), _bits(y[torch.from_numpy(rows).cuda()]), ref)


def test_bad_expert_offsets_reported_and_skipped():
    """An offset past T*k is reported; that expert's rows are skipped and the
    others are computed as usual."""
    w = custom(T=256, H=128, E=8, k=2, R=2, C=1, routing="topk", weights="softmax", seed=68)
    s = w.shape
    say("expert linear bad offsets")
    b = upload(w)
    eoff = _grouped_layout(b)
    ubep.ubep_dispatch(b.shape, ubep.BF16, b.x, b.pos, b.recv, None, b.ws)
    torch.cuda.synchronize()
    good = to_np(eoff).copy()
    bad = good.copy()
    bad[8] = s.T * s.k + 1000                       # expert 7 ends past the receive rows
    eb = torch.from_numpy(bad).cuda()
    W = _weights(s.E, 128, s.H, 68, 0.05)
    y = torch.zeros((s.T * s.k, 128), dtype=torch.bfloat16, device="cuda")
    ubep.ubep_expert_linear(b.shape, 128, eb, b.recv, _packed(W), y, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.ERR_BAD_POSITION
    xr, wb = _bits(b.recv), _bits(W)
    lo = good[7]
    ref = oracle.expert_linear(xr[:lo], wb[:7], good[:8])
    e_of_row = np.repeat(np.arange(7), np.diff(good[:8]))
    _check_rows(xr[:lo], wb, e_of_row, _bits(y[:lo]), ref)
    assert not bool(y[lo:].view(torch.int16).any())  # expert 7's rows untouched


@pytest.mark.parametrize("case", ["reversed", "nonzero_start"])
def test_inconsistent_expert_offsets_reported(case):
    """Offsets inside [0, T*k] that are not non-decreasing from 0 are reported.
    reversed: expert 3's run ends before it starts, so it is skipped while the
    runs that stay intact are computed as usual; nonzero_start: the offsets
    start at 1, reported, and every run is still computed over its rows."""
    w = custom(T=256, H=128, E=8, k=2, R=2, C=1, routing="topk", weights="softmax", seed=69)
    s = w.shape
    say(f"expert linear inconsistent offsets: {case}")
    b = upload(w)
    eoff = _grouped_layout(b)
    ubep.ubep_dispatch(b.shape, ubep.BF16, b.x, b.pos, b.recv, None, b.ws)
    torch.cuda.synchronize()
    good = to_np(eoff).copy()
    assert good[3] >= 2 and good[5] > good[4] > good[3]
    bad = good.copy()
    if case == "reversed":
        bad[4] = good[3] - 1                        # run 3 = [good[3], good[3] - 1)
    else:
        bad[0] = 1
    W = _weights(s.E, 128, s.H, 69, 0.05)
    y = torch.zeros((s.T * s.k, 128), dtype=torch.bfloat16, device="cuda")
    ubep.ubep_expert_linear(b.shape, 128, torch.from_numpy(bad).cuda(), b.recv, _packed(W), y, b.ws)
    torch.cuda.synchronize()
    assert device_status(b) == ubep.ERR_BAD_POSITION
    xr, wb, yb = _bits(b.recv), _bits(W), _bits(y)
    if case == "reversed":
        keep = list(range(3)) + list(range(5, 8))   # experts whose runs are untouched
    else:
        keep = list(range(1, 8))
    for e in keep:
        lo, hi = int(good[e]), int(good[e + 1])
        if e == 2 and case == "reversed":
            hi -= 1                                  # its last row is also in expert 4's run
        if hi <= lo:
            continue
        off = np.array([0, hi - lo], np.int32)
        ref = oracle.expert_linear(xr[lo:hi], wb[e:e + 1], off)
        _check_rows(xr[lo:hi], wb, np.full(hi - lo, e), yb[lo:hi], ref)
    if case == "nonzero_start":                     # expert 0 over its rows from 1
        lo, hi = 1, int(good[1])
        ref = oracle.expert_linear(xr[lo:hi], wb[0:1], np.array([0, hi - lo], np.int32))
        _check_rows(xr[lo:hi], wb, np.zeros(hi - lo, int), yb[lo:hi], ref)

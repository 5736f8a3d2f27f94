"""Pins for the oracle's dispatch layout (counts, offsets, stable positions).

Each pin is independent of the oracle's own loops: numpy's bincount / cumsum /
stable argsort, Python's tuple sort on tiny inputs, a hand-worked example, and
invariants that any correct layout satisfies.
"""
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from workloads import CONFIGS, custom, generate, make_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _numpy_layout(idx, E, R, C):
    T, k = idx.shape
    epr = E // R
    d = (idx // epr).ravel()
    t = np.repeat(np.arange(T), k)
    expert_count = np.bincount(idx.ravel(), minlength=E)
    rank_count = np.bincount(d, minlength=R)
    recv_offset = np.concatenate([[0], np.cumsum(rank_count)])
    # a stable sort of the flattened (t, j) sequence by destination rank is the
    # (rank, token, slot) order; regions are packed in rank order, so the
    # inverse permutation is the absolute receive row
    order = np.argsort(d, kind="stable")
    pos = np.empty(T * k, np.int64)
    pos[order] = np.arange(T * k)
    src = t // (T // R)
    sd = np.zeros((R, R), np.int64)
    np.add.at(sd, (src, d), 1)
    send_offset = np.cumsum(sd, axis=0) - sd
    ch = t // (T // C)
    cd = np.zeros((C, R), np.int64)
    np.add.at(cd, (ch, d), 1)
    chunk_offset = np.cumsum(cd, axis=0) - cd
    return dict(pos=pos.reshape(T, k), expert_count=expert_count, rank_count=rank_count,
                recv_offset=recv_offset, send_offset=send_offset, chunk_offset=chunk_offset,
                recv_src=order)


def _assert_layout_equal(a, b):
    for key in ("pos", "expert_count", "rank_count", "recv_offset", "send_offset",
                "chunk_offset", "recv_src"):
        np.testing.assert_array_equal(np.asarray(a[key]), np.asarray(b[key]), err_msg=key)


def _brute_force(idx, E, R):
    """Enumerate all rows, sort by the key tuple (rank, token, slot), number them."""
    T, k = idx.shape
    epr = E // R
    rows = [(int(idx[t, j]) // epr, t, j) for t in range(T) for j in range(k)]
    pos = np.empty((T, k), np.int64)
    for p, (_, t, j) in enumerate(sorted(rows)):
        pos[t, j] = p
    return pos


def test_worked_example():
    vals = {}
    with open(os.path.join(GOLDEN, "layout_worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, *rest = line.split()
            vals[name] = [int(v) for v in rest]
    T, k, E, R, C = (vals[n][0] for n in ("T", "k", "E", "R", "C"))
    idx = np.array(vals["topk_idx"], np.int32).reshape(T, k)
    got = oracle.layout(idx, E, R, C)
    np.testing.assert_array_equal(got["pos"].ravel(), vals["pos"])
    np.testing.assert_array_equal(got["expert_count"], vals["expert_count"])
    np.testing.assert_array_equal(got["rank_count"], vals["rank_count"])
    np.testing.assert_array_equal(got["recv_offset"], vals["recv_offset"])
    np.testing.assert_array_equal(got["send_offset"].ravel(), vals["send_offset"])
    np.testing.assert_array_equal(got["chunk_offset"].ravel(), vals["chunk_offset"])
    np.testing.assert_array_equal(got["recv_src"], vals["recv_src"])


@pytest.mark.parametrize("name", [n for n in CONFIGS if "T65536" not in n])
def test_layout_matches_numpy_on_configs(name):
    w = make_config(name)
    s = w.shape
    got = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    _assert_layout_equal(got, _numpy_layout(w.topk_idx, s.E, s.R, s.C))


def test_layout_large_prefill_routing_matches_numpy():
    r = CONFIGS["prefill_grouped_zipf_T65536_H7168_E256_k8_R64_C16"]
    w = generate(r, tokens=1)          # routing for all tokens, x for one
    s = w.shape
    got = oracle.layout(w.topk_idx, s.E, s.R, s.C)
    _assert_layout_equal(got, _numpy_layout(w.topk_idx, s.E, s.R, s.C))


@pytest.mark.parametrize("seed", range(6))
def test_layout_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    T, E, R, k = 9, 6, 3, 3
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    got = oracle.layout(idx, E, R, 3)
    np.testing.assert_array_equal(got["pos"], _brute_force(idx, E, R))


@settings(max_examples=60, deadline=None)
@given(data=st.data())
def test_layout_property(data):
    R = data.draw(st.sampled_from([1, 2, 3, 4, 8]))
    epr = data.draw(st.integers(1, 4))
    E = R * epr
    k = data.draw(st.integers(1, min(E, 8)))
    T = R * data.draw(st.integers(1, 16))
    C = data.draw(st.sampled_from([c for c in (1, 2, 4, T) if T % c == 0]))
    skew = data.draw(st.booleans())
    rng = np.random.default_rng(data.draw(st.integers(0, 2**31)))
    if skew:                         # most tokens pick the same low experts
        p = 1.0 / np.arange(1, E + 1) ** 2.0
        p /= p.sum()
        idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    else:
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    idx = idx.astype(np.int32)
    got = oracle.layout(idx, E, R, C)
    _assert_layout_equal(got, _numpy_layout(idx, E, R, C))
    # invariants of any correct layout
    assert got["rank_count"].sum() == T * k == got["recv_offset"][-1]
    assert got["expert_count"].sum() == T * k
    assert np.array_equal(np.sort(got["pos"].ravel()), np.arange(T * k))        # bijection
    np.testing.assert_array_equal(got["send_offset"][-1] + np.bincount(
        (idx[-(T // R):] // epr).ravel(), minlength=R), got["rank_count"])
    for d in range(R):               # rows of each region ascend in (t, j)
        lo, hi = got["recv_offset"][d], got["recv_offset"][d + 1]
        src = got["recv_src"][lo:hi]
        assert np.all(np.diff(src) > 0)
        assert np.all(idx.ravel()[src] // epr == d)


def test_bad_expert_id_and_shape():
    idx = np.array([[0, 1], [2, 7]], np.int32)
    with pytest.raises(oracle.OracleError) as ei:
        oracle.layout(idx, 4, 2)
    assert ei.value.code == oracle.BAD_EXPERT_ID
    idx[1, 1] = -1
    with pytest.raises(oracle.OracleError) as ei:
        oracle.layout(idx, 4, 2)
    assert ei.value.code == oracle.BAD_EXPERT_ID
    assert oracle.check_shape(4, 8, 6, 2, 4) == oracle.INVALID_ARG      # E % R != 0
    assert oracle.check_shape(6, 8, 8, 2, 4) == oracle.INVALID_ARG      # T % R != 0
    assert oracle.check_shape(8, 8, 8, 2, 4, 3) == oracle.INVALID_ARG   # T % C != 0
    assert oracle.check_shape(8, 64, 8, 2, 4, 1, fp8=True) == oracle.INVALID_ARG
    assert oracle.check_shape(8, 128, 8, 2, 4, 1, fp8=True) == oracle.OK


def test_degenerate_layouts():
    # every row to one rank (maximum skew), one rank, one expert per rank
    T, k, E, R = 16, 2, 8, 4
    idx = np.tile(np.array([[0, 1]], np.int32), (T, 1))
    got = oracle.layout(idx, E, R)
    assert got["rank_count"].tolist() == [T * k, 0, 0, 0]
    np.testing.assert_array_equal(got["pos"].ravel(), np.arange(T * k))
    got = oracle.layout(idx, E, 1)
    np.testing.assert_array_equal(got["pos"].ravel(), np.arange(T * k))
    idx = np.stack([np.random.default_rng(3).permutation(8)[:k] for _ in range(T)]).astype(np.int32)
    _assert_layout_equal(oracle.layout(idx, 8, 8, 4), _numpy_layout(idx, 8, 8, 4))
    # one token
    idx = np.array([[5, 2, 7]], np.int32)
    got = oracle.layout(idx, 8, 1)
    assert got["pos"].ravel().tolist() == [0, 1, 2]

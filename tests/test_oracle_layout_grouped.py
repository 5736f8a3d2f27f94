"""Pins for the oracle's expert-grouped layout (rows of each region ordered by
(expert, token, slot)).

Independent of the oracle's loops: numpy's bincount / cumsum / stable argsort
by expert id, Python's tuple sort on tiny inputs, a hand-worked example, the
rank-order layout in the special case of one expert per rank, and invariants.
"""
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from workloads import CONFIGS, generate, make_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
KEYS = ("pos", "expert_count", "expert_offset", "rank_count", "recv_offset", "send_offset",
        "chunk_offset", "recv_src")


def _numpy_grouped(idx, E, R, C):
    T, k = idx.shape
    epr = E // R
    e = idx.ravel()
    d = e // epr
    t = np.repeat(np.arange(T), k)
    expert_count = np.bincount(e, minlength=E)
    expert_offset = np.concatenate([[0], np.cumsum(expert_count)])
    rank_count = np.bincount(d, minlength=R)
    # a stable sort of the flattened (t, j) sequence by expert id is the
    # (expert, token, slot) order; runs are packed in expert order, so the
    # inverse permutation is the absolute receive row
    order = np.argsort(e, kind="stable")
    pos = np.empty(T * k, np.int64)
    pos[order] = np.arange(T * k)
    sd = np.zeros((R, R), np.int64)
    np.add.at(sd, (t // (T // R), d), 1)
    cd = np.zeros((C, R), np.int64)
    np.add.at(cd, (t // (T // C), d), 1)
    return dict(pos=pos.reshape(T, k), expert_count=expert_count, expert_offset=expert_offset,
                rank_count=rank_count, recv_offset=np.concatenate([[0], np.cumsum(rank_count)]),
                send_offset=np.cumsum(sd, axis=0) - sd, chunk_offset=np.cumsum(cd, axis=0) - cd,
                recv_src=order)


def _assert_equal(a, b):
    for key in KEYS:
        np.testing.assert_array_equal(np.asarray(a[key]), np.asarray(b[key]), err_msg=key)


def test_worked_example():
    vals = {}
    with open(os.path.join(GOLDEN, "layout_grouped_worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, *rest = line.split()
            vals[name] = [int(v) for v in rest]
    T, k, E, R, C = (vals[n][0] for n in ("T", "k", "E", "R", "C"))
    idx = np.array(vals["topk_idx"], np.int32).reshape(T, k)
    got = oracle.layout_grouped(idx, E, R, C)
    for key in KEYS:
        np.testing.assert_array_equal(np.asarray(got[key]).ravel(), vals[key], err_msg=key)


@pytest.mark.parametrize("name", [n for n in CONFIGS if "T65536" not in n])
def test_matches_numpy_on_configs(name):
    w = make_config(name)
    s = w.shape
    _assert_equal(oracle.layout_grouped(w.topk_idx, s.E, s.R, s.C),
                  _numpy_grouped(w.topk_idx, s.E, s.R, s.C))


def test_large_prefill_routing_matches_numpy():
    w = generate(CONFIGS["prefill_grouped_zipf_T65536_H7168_E256_k8_R64_C16"], tokens=1)
    s = w.shape
    _assert_equal(oracle.layout_grouped(w.topk_idx, s.E, s.R, s.C),
                  _numpy_grouped(w.topk_idx, s.E, s.R, s.C))


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    T, E, R, k = 9, 6, 3, 3
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    rows = sorted((int(idx[t, j]) // (E // R), int(idx[t, j]), t, j)
                  for t in range(T) for j in range(k))
    want = np.empty((T, k), np.int64)
    for p, (_, _, t, j) in enumerate(rows):
        want[t, j] = p
    np.testing.assert_array_equal(oracle.layout_grouped(idx, E, R, 3)["pos"], want)


def test_one_expert_per_rank_is_rank_order():
    rng = np.random.default_rng(11)
    T, E, k = 64, 16, 4
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    g = oracle.layout_grouped(idx, E, E, 4)
    r = oracle.layout(idx, E, E, 4)
    for key in ("pos", "expert_count", "rank_count", "recv_offset", "send_offset",
                "chunk_offset", "recv_src"):
        np.testing.assert_array_equal(g[key], r[key], err_msg=key)
    np.testing.assert_array_equal(g["expert_offset"], r["recv_offset"])


@settings(max_examples=60, deadline=None)
@given(data=st.data())
def test_property(data):
    R = data.draw(st.sampled_from([1, 2, 3, 4, 8]))
    epr = data.draw(st.integers(1, 6))
    E = R * epr
    k = data.draw(st.integers(1, min(E, 8)))
    T = R * data.draw(st.integers(1, 16))
    C = data.draw(st.sampled_from([c for c in (1, 2, 4, T) if T % c == 0]))
    rng = np.random.default_rng(data.draw(st.integers(0, 2**31)))
    if data.draw(st.booleans()):     # skewed: most tokens pick the same low experts
        p = 1.0 / np.arange(1, E + 1) ** 2.0
        idx = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)])
    else:
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    idx = idx.astype(np.int32)
    got = oracle.layout_grouped(idx, E, R, C)
    _assert_equal(got, _numpy_grouped(idx, E, R, C))
    rank = oracle.layout(idx, E, R, C)
    assert np.array_equal(np.sort(got["pos"].ravel()), np.arange(T * k))       # bijection
    for key in ("expert_count", "rank_count", "recv_offset", "send_offset", "chunk_offset"):
        np.testing.assert_array_equal(got[key], rank[key], err_msg=key)
    for e in range(E):               # each expert's run holds its rows in (t, j) order
        lo, hi = got["expert_offset"][e], got["expert_offset"][e + 1]
        src = got["recv_src"][lo:hi]
        assert np.all(np.diff(src) > 0) and np.all(idx.ravel()[src] == e)
    for d in range(R):               # a region holds the same rows in either order
        lo, hi = rank["recv_offset"][d], rank["recv_offset"][d + 1]
        np.testing.assert_array_equal(np.sort(got["recv_src"][lo:hi]), rank["recv_src"][lo:hi])


def test_degenerate_and_errors():
    T, k, E, R = 16, 2, 8, 4
    idx = np.tile(np.array([[1, 0]], np.int32), (T, 1))    # every token to experts 1 and 0
    got = oracle.layout_grouped(idx, E, R)
    assert got["expert_count"].tolist() == [T, T, 0, 0, 0, 0, 0, 0]
    np.testing.assert_array_equal(got["pos"][:, 1], np.arange(T))        # expert 0 first
    np.testing.assert_array_equal(got["pos"][:, 0], T + np.arange(T))
    got = oracle.layout_grouped(np.array([[5, 2, 7]], np.int32), 8, 1)   # one token, one rank
    assert got["pos"].ravel().tolist() == [1, 0, 2]
    with pytest.raises(oracle.OracleError) as ei:
        oracle.layout_grouped(np.array([[0, 8], [1, 2]], np.int32), 8, 2)
    assert ei.value.code == oracle.BAD_EXPERT_ID

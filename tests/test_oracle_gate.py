"""CPU pins of the oracle's gate (top-k router on fp32 logits).

The oracle's selection is compared with numpy's stable sorts (an independent
library route to the same order: larger logit first, ties to the lower id),
its group filter with numpy sorts of each group, its weights with the float64
closed forms, and everything with a hand-worked example
(tests/golden/gate_worked_example.txt).
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    out = {}
    with open(os.path.join(GOLDEN, "gate_worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = [float(v) for v in vals]
    return out


def _ulps(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def _numpy_select(z, k, groups=1, keep=1):
    """Selection through numpy sorts: group scores from np.sort, kept groups by
    lexsort (score desc, group id asc), experts by a stable argsort of -z."""
    T, E = z.shape
    gs = E // groups
    zg = z.reshape(T, groups, gs)
    srt = np.sort(zg, axis=2)
    score = srt[:, :, -1] if gs == 1 else (srt[:, :, -1] + srt[:, :, -2]).astype(np.float32)
    idx = np.empty((T, k), np.int64)
    for t in range(T):
        order = np.lexsort((np.arange(groups), -score[t]))
        allowed = np.zeros(E, bool)
        for g in order[:keep]:
            allowed[g * gs:(g + 1) * gs] = True
        cand = np.where(allowed, -z[t], np.inf)
        idx[t] = np.argsort(cand, kind="stable")[:k]
    return idx


def _numpy_weights(z, idx, norm):
    zs = np.take_along_axis(z.astype(np.float64), idx, axis=1)
    if norm == oracle.SOFTMAX:
        v = np.exp(zs - zs[:, :1])
    else:
        v = 1.0 / (1.0 + np.exp(-zs))
    return (v / v.sum(axis=1, keepdims=True)).astype(np.float32)


def test_gate_hand_worked_example():
    g = _golden()
    z = np.array([g["logits"]], np.float32)
    k, G, keep = int(g["k"][0]), int(g["groups"][0]), int(g["keep_groups"][0])
    for norm, key in ((oracle.SOFTMAX, "softmax_w"), (oracle.SIGMOID, "sigmoid_w")):
        idx, w = oracle.gate(z, k, G, keep, norm)
        assert idx[0].tolist() == [int(v) for v in g["topk_idx"]]
        np.testing.assert_allclose(w[0], g[key], rtol=0, atol=2e-7)


@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (64, 6), (256, 8), (128, 8), (96, 32)])
def test_gate_selection_matches_stable_sort(E, k):
    z = np.random.default_rng(E * 31 + k).standard_normal((300, E)).astype(np.float32)
    idx, _ = oracle.gate(z, k)
    np.testing.assert_array_equal(idx, _numpy_select(z, k))


def test_gate_ties_go_to_the_lower_id():
    rng = np.random.default_rng(7)
    z = rng.integers(-2, 3, size=(400, 32)).astype(np.float32)     # many equal logits
    z[:5] = 0.0
    z[5] = -0.0                                                      # -0 equals +0
    for k in (1, 3, 8):
        idx, w = oracle.gate(z, k)
        np.testing.assert_array_equal(idx, _numpy_select(z, k))
        assert idx[0].tolist() == list(range(k))
    idx, w = oracle.gate(z[:1], 4)                                   # equal logits: equal weights
    assert np.all(w == np.float32(0.25))


@pytest.mark.parametrize("E,G,keep,k", [(256, 8, 4, 8), (64, 8, 3, 6), (8, 4, 2, 3), (32, 32, 5, 5),
                                        (48, 3, 1, 16), (16, 2, 2, 16)])
def test_gate_groups_match_numpy(E, G, keep, k):
    z = np.random.default_rng(E + G + keep).standard_normal((300, E)).astype(np.float32)
    for norm in (oracle.SOFTMAX, oracle.SIGMOID):
        idx, _ = oracle.gate(z, k, G, keep, norm)
        np.testing.assert_array_equal(idx, _numpy_select(z, k, G, keep))


def test_gate_group_filter_can_drop_the_best_expert():
    """A plain top-k would take expert 2 here; the group rule must not."""
    z = np.array([[0.5, 0.4, 2.0, -3.0, 0.1, 0.2, 1.0, 0.6]], np.float32)
    plain, _ = oracle.gate(z, 3)
    grouped, _ = oracle.gate(z, 3, 4, 2)
    assert 2 in plain[0] and 2 not in grouped[0]


@pytest.mark.parametrize("norm", [oracle.SOFTMAX, oracle.SIGMOID])
def test_gate_weights_match_closed_form(norm):
    z = (3.0 * np.random.default_rng(11).standard_normal((500, 64))).astype(np.float32)
    idx, w = oracle.gate(z, 8, 8, 4, norm)
    assert _ulps(w, _numpy_weights(z, idx.astype(np.int64), norm)).max() <= 1
    assert np.all(w > 0)
    np.testing.assert_allclose(w.astype(np.float64).sum(axis=1), 1.0, atol=8 * 2.0 ** -24)
    assert np.all(np.diff(w, axis=1) <= 0)          # larger logit, larger weight


def test_gate_single_slot_weight_is_one():
    z = np.random.default_rng(3).standard_normal((50, 16)).astype(np.float32)
    for norm in (oracle.SOFTMAX, oracle.SIGMOID):
        idx, w = oracle.gate(z, 1, norm=norm)
        assert np.all(w == 1.0)
        np.testing.assert_array_equal(idx[:, 0], np.argmax(z, axis=1))


def test_gate_ids_distinct_and_in_kept_groups():
    E, G, keep, k = 256, 8, 4, 8
    z = np.random.default_rng(5).standard_normal((400, E)).astype(np.float32)
    idx, _ = oracle.gate(z, k, G, keep)
    assert all(len(set(r)) == k for r in idx.tolist())
    assert all(len(set(e // (E // G) for e in r)) <= keep for r in idx.tolist())


def test_gate_rejects_what_the_definition_excludes():
    z = np.zeros((2, 12), np.float32)
    for kw in (dict(k=3, groups=5), dict(k=3, groups=4, keep_groups=5), dict(k=7, groups=4, keep_groups=2),
               dict(k=0), dict(k=2, norm=2)):
        with pytest.raises(ValueError):
            oracle.gate(z, **kw)


def test_gate_softmax_large_logits_stay_finite():
    """exp of a logit near 1000 overflows even in double; the definition is
    shift-invariant, so the weights must equal those of the shifted logits."""
    z = np.random.default_rng(9).standard_normal((40, 32)).astype(np.float32)
    _, w_ref = oracle.gate(z, 4)
    idx, w = oracle.gate(z + np.float32(1000.0), 4)
    assert np.all(np.isfinite(w))
    np.testing.assert_allclose(w, _numpy_weights(z + np.float32(1000.0), idx.astype(np.int64),
                                                 oracle.SOFTMAX), rtol=0, atol=2e-7)
    np.testing.assert_allclose(w, w_ref, rtol=0, atol=2e-5)   # shift by 1000 rounds the logits


@pytest.mark.parametrize("name", ["tiny_T128_H1024_E8_k2_R2", "dsv3_decode_T4096_H7168_E256_k8_R32",
                                  "prefill_grouped_zipf_T65536_H7168_E256_k8_R64_C16"])
def test_gate_reproduces_the_generators_routing(name):
    """The workload generator selects with numpy sorts on float64 keys; the
    oracle gate on the same keys rounded to fp32 must pick the same experts
    (no two keys of a token are within fp32 rounding of each other here)."""
    from workloads import CONFIGS, generate, router_logits
    r = CONFIGS[name]
    grouped = r.routing == "group_zipf"
    idx, w = oracle.gate(router_logits(r), r.shape.k, r.n_groups if grouped else 1,
                         r.topk_groups if grouped else 1,
                         oracle.SIGMOID if r.weights == "sigmoid" else oracle.SOFTMAX)
    ref = generate(r, tokens=1)
    np.testing.assert_array_equal(idx, ref.topk_idx)
    if r.routing == "topk":                     # same logits up to fp32 rounding: same weights
        np.testing.assert_allclose(w, ref.topk_w, rtol=0, atol=1e-6)

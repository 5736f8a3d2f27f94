"""The seeded input generator: determinism and the structure each recipe promises."""
import numpy as np
import pytest

from workloads import CONFIGS, custom, generate, make_config


def test_same_seed_same_bytes():
    a = make_config("tiny_T128_H1024_E8_k2_R2")
    b = make_config("tiny_T128_H1024_E8_k2_R2")
    assert a.x.tobytes() == b.x.tobytes()
    assert a.topk_idx.tobytes() == b.topk_idx.tobytes()
    assert a.topk_w.tobytes() == b.topk_w.tobytes()
    c = make_config("tiny_T128_H1024_E8_k2_R2", seed=77)
    assert c.x.tobytes() != a.x.tobytes()


@pytest.mark.parametrize("name", [n for n in CONFIGS if "T65536" not in n])
def test_recipe_structure(name):
    w = make_config(name)
    s = w.shape
    assert w.x.shape == (s.T, s.H) and w.x.dtype == np.uint16
    assert w.topk_idx.shape == (s.T, s.k) and w.topk_idx.dtype == np.int32
    assert w.topk_w.shape == (s.T, s.k) and w.topk_w.dtype == np.float32
    # k distinct ids in range
    srt = np.sort(w.topk_idx, axis=1)
    assert np.all(np.diff(srt, axis=1) > 0)
    assert w.topk_idx.min() >= 0 and w.topk_idx.max() < s.E
    # weights normalised
    assert np.all(w.topk_w > 0)
    assert np.max(np.abs(w.topk_w.astype(np.float64).sum(1) - 1)) <= s.k * 2.0 ** -24
    # activations are standard normal
    xf = (w.x.astype(np.uint32) << 16).view(np.float32)
    assert abs(xf.mean()) < 0.01 and abs(xf.std() - 1) < 0.01


def test_group_limited_routing_uses_at_most_four_groups():
    w = generate(CONFIGS["prefill_grouped_zipf_T65536_H7168_E256_k8_R64_C16"], tokens=1)
    groups = w.topk_idx // 32
    n = np.array([len(set(r)) for r in groups])
    assert n.max() <= 4 and n.min() >= 1
    # Zipf popularity makes the hottest expert far above the mean
    cnt = np.bincount(w.topk_idx.ravel(), minlength=256)
    assert cnt.max() > 5 * cnt.mean()


def test_uniform_routing_is_balanced_and_zipf_is_not():
    u = make_config("dsv3_decode_T4096_H7168_E256_k8_R32")
    z = make_config("dsv3_decode_zipf_T4096_H7168_E256_k8_R32")
    cu = np.bincount(u.topk_idx.ravel() // 8, minlength=32)
    cz = np.bincount(z.topk_idx.ravel() // 8, minlength=32)
    assert cu.max() / cu.mean() < 1.2
    assert cz.max() / cz.mean() > 3


def test_selection_is_descending_score():
    # with the topk recipe, slot 0 holds the largest logit: check that weights
    # (monotone in the logit for both softmax and sigmoid rules) are descending
    w = custom(T=256, H=8, E=16, k=4, R=4, seed=2, weights="sigmoid")
    assert np.all(np.diff(w.topk_w, axis=1) <= 0)

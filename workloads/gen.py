"""Seeded synthetic inputs for MoE token dispatch / combine.

This module only draws inputs: token activations ``x`` (bf16 bit patterns),
per-token selected experts ``topk_idx`` and gate weights ``topk_w``.  It holds
none of the dispatch/combine arithmetic (no counting, scanning, placement,
quantisation or reduction); both the CPU oracle and the HIP path consume the
arrays it returns.

The pages ("NJU x Huawei UBEP: Reengineering MoE Expert Parallelism", opening
section) say each token is sent to the device that hosts its *selected* expert;
they do not describe the gate.  The routing recipes below are therefore input
conventions, stated once here:

* ``topk``      - top-k of i.i.d. N(0,1) logits z[t, e]; larger score first,
                  equal scores -> lower expert id.
* ``zipf``      - Gumbel-top-k over expert popularity p(pi(i)) ~ (i+1)^-s for a
                  seeded permutation pi: keys log p_e + Gumbel_e.  The top-k of
                  those keys is k successive draws without replacement with
                  probabilities proportional to p (Kool et al., ICML 2019).
* ``group_zipf``- the same keys, restricted to the best ``topk_groups`` of
                  ``n_groups`` contiguous expert groups, a group scored by the
                  sum of its two best keys (DeepSeek-V3's group-limited rule).

Weights are computed from z at the selected experts in float64 and rounded
once to float32:

* ``softmax``   - w_j = exp(z_j) / sum_i exp(z_i) over the k selected
* ``sigmoid``   - w_j = sigma(z_j) / sum_i sigma(z_i) over the k selected

Activations are standard normal float32 rounded to bf16 by torch's own
conversion (round to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Shape:
    T: int          # tokens
    H: int          # hidden size (channels per token row)
    E: int          # experts
    k: int          # experts selected per token
    R: int          # virtual expert-parallel ranks
    C: int = 1      # pipeline chunks

    def as_dict(self):
        return dict(T=self.T, H=self.H, E=self.E, k=self.k, R=self.R, C=self.C)


@dataclass(frozen=True)
class Recipe:
    shape: Shape
    routing: str = "topk"        # topk | zipf | group_zipf
    weights: str = "softmax"     # softmax | sigmoid
    payload: str = "bf16"        # bf16 | fp8 (dispatch payload type)
    zipf_s: float = 1.2
    n_groups: int = 8
    topk_groups: int = 4
    seed: int = 0
    note: str = ""


@dataclass
class Workload:
    recipe: Recipe
    x: np.ndarray          # uint16 [T, H]  bf16 bit patterns
    topk_idx: np.ndarray   # int32  [T, k]
    topk_w: np.ndarray     # float32 [T, k]
    extra: dict = field(default_factory=dict)

    @property
    def shape(self) -> Shape:
        return self.recipe.shape


# Named workloads.  Each name states the shape it stands for.
CONFIGS: dict[str, Recipe] = {
    # small case, 2 virtual ranks of 4 experts, top-2 of 8
    "tiny_T128_H1024_E8_k2_R2": Recipe(
        Shape(T=128, H=1024, E=8, k=2, R=2), routing="topk", weights="softmax", seed=1001,
        note="T=128, H=1024 bf16, E=8 top-2 softmax, R=2"),
    # DeepSeek-V3-shaped decode step
    "dsv3_decode_T4096_H7168_E256_k8_R32": Recipe(
        Shape(T=4096, H=7168, E=256, k=8, R=32), routing="topk", weights="sigmoid", seed=1002,
        note="DeepSeek-V3-shaped decode: T=4096, H=7168 bf16, E=256 top-8 sigmoid, R=32"),
    # the small case with Zipf(1.2) expert popularity
    "tiny_zipf_T128_H1024_E8_k2_R2": Recipe(
        Shape(T=128, H=1024, E=8, k=2, R=2), routing="zipf", weights="softmax", seed=1003,
        note="T=128 with Zipf(1.2) routing; skew bounded at 2x by the shape"),
    # the DeepSeek-V3 decode shape with Zipf(1.2) expert popularity
    "dsv3_decode_zipf_T4096_H7168_E256_k8_R32": Recipe(
        Shape(T=4096, H=7168, E=256, k=8, R=32), routing="zipf", weights="sigmoid", seed=1013,
        note="DeepSeek-V3 decode shape with Zipf(1.2) routing"),
    # Qwen3-MoE-shaped prefill chunk, fp8 e4m3 dispatch payload
    "qwen3_prefill_fp8_T16384_H4096_E128_k8_R16": Recipe(
        Shape(T=16384, H=4096, E=128, k=8, R=16), routing="topk", weights="softmax",
        payload="fp8", seed=1004,
        note="Qwen3-MoE prefill: T=16384, H=4096, E=128 top-8 softmax, R=16, fp8 e4m3 dispatch"),
    # large prefill, group-limited Zipf routing, 16 pipeline chunks
    "prefill_grouped_zipf_T65536_H7168_E256_k8_R64_C16": Recipe(
        Shape(T=65536, H=7168, E=256, k=8, R=64, C=16), routing="group_zipf", weights="sigmoid",
        seed=1005,
        note="T=65536, H=7168 bf16, E=256 group-limited (8x32, top-4 groups) top-8, "
             "Zipf(1.2), R=64, C=16"),
}

DEFAULT_BENCH = "dsv3_decode_T4096_H7168_E256_k8_R32"
SMALL = "tiny_T128_H1024_E8_k2_R2"


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(4)
    return [np.random.Generator(np.random.PCG64(s)) for s in kids]


def _to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _topk_desc(keys: np.ndarray, k: int) -> np.ndarray:
    # larger key first; equal keys -> lower column index (stable sort of -key)
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k]


def _select(recipe: Recipe, z: np.ndarray, g_perm, g_gum) -> np.ndarray:
    s = recipe.shape
    if recipe.routing == "topk":
        return _topk_desc(z, s.k)
    logp = np.empty(s.E, dtype=np.float64)
    perm = g_perm.permutation(s.E)
    ranks = np.arange(1, s.E + 1, dtype=np.float64)
    p = ranks ** (-recipe.zipf_s)
    p /= p.sum()
    logp[perm] = np.log(p)
    gumbel = g_gum.gumbel(size=(s.T, s.E))
    keys = logp[None, :] + gumbel
    if recipe.routing == "zipf":
        return _topk_desc(keys, s.k)
    if recipe.routing == "group_zipf":
        G = recipe.n_groups
        assert s.E % G == 0
        gsz = s.E // G
        kg = keys.reshape(s.T, G, gsz)
        top2 = -np.sort(-kg, axis=2)[:, :, :2].sum(axis=2)          # [T, G]
        keep = _topk_desc(top2, recipe.topk_groups)                  # [T, topk_groups]
        mask = np.zeros((s.T, G), dtype=bool)
        np.put_along_axis(mask, keep, True, axis=1)
        masked = np.where(np.repeat(mask, gsz, axis=1), keys, -np.inf)
        return _topk_desc(masked, s.k)
    raise ValueError(f"unknown routing {recipe.routing!r}")


def _weights(kind: str, zsel: np.ndarray) -> np.ndarray:
    if kind == "softmax":
        m = zsel.max(axis=1, keepdims=True)
        e = np.exp(zsel - m)
        w = e / e.sum(axis=1, keepdims=True)
    elif kind == "sigmoid":
        sg = 1.0 / (1.0 + np.exp(-zsel))
        w = sg / sg.sum(axis=1, keepdims=True)
    else:
        raise ValueError(f"unknown weights {kind!r}")
    return w.astype(np.float32)


def generate(recipe: Recipe, tokens: int | None = None) -> Workload:
    """Draw one workload.  ``tokens`` (optional) draws only the first rows of x
    for a quick sample; routing always covers all T tokens."""
    s = recipe.shape
    g_x, g_z, g_perm, g_gum = _streams(recipe.seed)
    z = g_z.standard_normal(size=(s.T, s.E))
    idx = _select(recipe, z, g_perm, g_gum).astype(np.int32)
    zsel = np.take_along_axis(z, idx.astype(np.int64), axis=1)
    w = _weights(recipe.weights, zsel)
    nx = s.T if tokens is None else min(tokens, s.T)
    x32 = g_x.standard_normal(size=(nx, s.H), dtype=np.float32)
    x = _to_bf16_bits(x32)
    return Workload(recipe=recipe, x=x, topk_idx=np.ascontiguousarray(idx),
                    topk_w=np.ascontiguousarray(w))


def router_logits(recipe: Recipe) -> np.ndarray:
    """fp32 router logits [T, E] for a gate to select from: the N(0,1) logits
    of `topk` routing, or the Zipf selection keys (log popularity + Gumbel
    noise) of the skewed routings.  Drawn from the same streams as generate()."""
    s = recipe.shape
    _, g_z, g_perm, g_gum = _streams(recipe.seed)
    z = g_z.standard_normal(size=(s.T, s.E))
    if recipe.routing == "topk":
        return z.astype(np.float32)
    logp = np.empty(s.E, dtype=np.float64)
    perm = g_perm.permutation(s.E)
    p = np.arange(1, s.E + 1, dtype=np.float64) ** (-recipe.zipf_s)
    p /= p.sum()
    logp[perm] = np.log(p)
    return (logp[None, :] + g_gum.gumbel(size=(s.T, s.E))).astype(np.float32)


def make_config(name: str, seed: int | None = None) -> Workload:
    r = CONFIGS[name]
    if seed is not None:
        r = Recipe(**{**r.__dict__, "seed": seed})
    return generate(r)


def custom(T, H, E, k, R, C=1, routing="topk", weights="softmax", payload="bf16", seed=0,
           **kw) -> Workload:
    return generate(Recipe(Shape(T=T, H=H, E=E, k=k, R=R, C=C), routing=routing,
                           weights=weights, payload=payload, seed=seed, **kw))

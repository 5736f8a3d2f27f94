"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
pull results back to the host; compute oracle references on the CPU."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import combine_top_route_amd as ubep
import oracle
from combine_top_route_amd.buffers import alloc_buffers, run_path
from workloads import CONFIGS, generate, make_config

LAYOUT_KEYS = ("pos", "expert_count", "rank_count", "recv_offset", "send_offset", "chunk_offset",
               "recv_src")


def say(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=3)
def workload(name: str):
    return make_config(name)


def shape_of(w) -> dict:
    return w.shape.as_dict()


def dtype_of(w) -> int:
    return ubep.FP8_E4M3 if w.recipe.payload == "fp8" else ubep.BF16


def upload(w, device="cuda"):
    return alloc_buffers(shape_of(w), dtype_of(w), device, x_bits=w.x, topk_idx=w.topk_idx,
                         topk_w=w.topk_w)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def gpu_layout(b) -> dict:
    s = b.shape
    ubep.ubep_layout(s, b.topk_idx, b.pos, b.expert_count, b.rank_count, b.recv_offset,
                     b.send_offset, b.chunk_offset if s["C"] > 1 else None, b.recv_src, b.ws)
    torch.cuda.synchronize()
    return {k: to_np(getattr(b, k)) for k in LAYOUT_KEYS}


def oracle_layout(w) -> dict:
    s = w.shape
    return oracle.layout(w.topk_idx, s.E, s.R, s.C)


def assert_layout_equal(got: dict, ref: dict, C: int):
    for key in LAYOUT_KEYS:
        if key == "chunk_offset" and C == 1:
            continue
        a, r = np.asarray(got[key]).ravel(), np.asarray(ref[key]).ravel()
        if not np.array_equal(a, r):
            bad = np.flatnonzero(a != r)
            raise AssertionError(f"{key}: {bad.size} mismatches, first at {bad[:5]}: "
                                 f"gpu {a[bad[:5]]} oracle {r[bad[:5]]}")


def device_status(b) -> int:
    return ubep.ubep_get_device_status(b.ws)


def bf16_ordinal_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|ordinal(a) - ordinal(b)| over bf16 bit patterns (monotone integer map)."""
    def ordv(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + u)
    return np.abs(ordv(a) - ordv(b))

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


def token_slices(s, budget_bytes: int = 1 << 29):
    """Contiguous token ranges whose k receive rows hold at most about
    budget_bytes of bf16 (one range at least one token long)."""
    step = max(1, budget_bytes // (s.k * s.H * 2))
    return [(t0, min(s.T, t0 + step)) for t0 in range(0, s.T, step)]


def assert_path_whole(b, w, skip_channels: int = 0, y=None):
    """Every dispatched row and every combined token of the device buffers `b`
    against the oracle, slice by slice: the oracle dispatches, applies the
    identity expert to and combines each token range on its own (dispatch and
    combine of a token touch only that token's k rows, so a range's results
    equal the whole problem's there).  b.pos must already equal the oracle's
    layout.  skip_channels: leading channels of every receive row not compared
    (the sentinel pipeline leaves its readiness word there).  y: the device
    combine input to compare as well (the fp8 identity expert's output)."""
    s = w.shape
    fp8 = w.recipe.payload == "fp8"
    n_checked = 0
    for t0, t1 in token_slices(s):
        toks = np.arange(t0, t1)
        rows_ref, out_ref = oracle.pipeline_tokens(w.x, w.topk_idx, w.topk_w, s.E, s.R, s.C,
                                                   payload=w.recipe.payload, tokens=toks)
        rows = b.pos[t0:t1].reshape(-1).long()
        if fp8:
            q_ref, sc_ref = rows_ref
            q_ref = q_ref.reshape(-1, s.H)
            sc_ref = sc_ref.reshape(-1, s.H // 128)
            np.testing.assert_array_equal(to_np(b.recv.index_select(0, rows)), q_ref,
                                          err_msg=f"fp8 codes, tokens {t0}..{t1}")
            np.testing.assert_array_equal(to_np(b.recv_scale.index_select(0, rows)), sc_ref,
                                          err_msg=f"fp8 scales, tokens {t0}..{t1}")
            if y is not None:
                np.testing.assert_array_equal(to_np(y.index_select(0, rows)),
                                              oracle.identity_fp8(q_ref, sc_ref),
                                              err_msg=f"identity expert, tokens {t0}..{t1}")
        else:
            got = to_np(b.recv.index_select(0, rows))
            want = rows_ref.reshape(-1, s.H)
            np.testing.assert_array_equal(got[:, skip_channels:], want[:, skip_channels:],
                                          err_msg=f"dispatched rows, tokens {t0}..{t1}")
        np.testing.assert_array_equal(to_np(b.out[t0:t1]), out_ref,
                                      err_msg=f"combined tokens {t0}..{t1}")
        n_checked += t1 - t0
    assert n_checked == s.T

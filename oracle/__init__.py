"""CPU oracle for MoE token dispatch / combine -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does.

Thin numpy wrappers over ``oracle.c`` (plain single-threaded C).  Each wrapper
allocates its own outputs and returns numpy arrays.  The definitions and the
readings of the pages they follow are stated in ``oracle.c``.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB: another build of oracle.c (the sanitizer run of the tests)
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

OK, INVALID_ARG, UNSUPPORTED, BAD_EXPERT_ID = 0, 1, 2, 3

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        i64, i32, p = C.c_int64, C.c_int32, C.c_void_p
        L.oracle_check_shape.argtypes = [i64, i64, i32, i32, i32, i32, C.c_int]
        L.oracle_check_shape.restype = C.c_int
        L.oracle_layout.argtypes = [i64, i32, i32, i32, i32, p, p, p, p, p, p, p, p]
        L.oracle_layout.restype = C.c_int
        L.oracle_layout_grouped.argtypes = [i64, i32, i32, i32, i32, p, p, p, p, p, p, p, p, p]
        L.oracle_layout_grouped.restype = C.c_int
        L.oracle_dispatch_bf16.argtypes = [i64, i64, i32, p, p, p]
        L.oracle_dispatch_bf16.restype = None
        L.oracle_dispatch_fp8.argtypes = [i64, i64, i32, p, p, p, p]
        L.oracle_dispatch_fp8.restype = None
        L.oracle_identity_fp8.argtypes = [i64, i64, p, p, p]
        L.oracle_identity_fp8.restype = None
        L.oracle_combine.argtypes = [i64, i64, i32, p, p, p, p]
        L.oracle_combine.restype = None
        L.oracle_expert_linear.argtypes = [i32, i64, i64, p, p, p, p]
        L.oracle_expert_linear.restype = None
        L.oracle_f64_to_bf16.argtypes = [C.c_double]
        L.oracle_f64_to_bf16.restype = C.c_uint16
        L.oracle_gate.argtypes = [i64, i32, i32, i32, i32, C.c_int, p, p, p]
        L.oracle_gate.restype = C.c_int
        for n in ("oracle_f32_to_e4m3_array", "oracle_f32_to_bf16_array",
                  "oracle_e4m3_to_f32_array"):
            getattr(L, n).argtypes = [i64, p, p]
            getattr(L, n).restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


def check_shape(T, H, E, k, R, C_=1, fp8=False) -> int:
    return lib().oracle_check_shape(T, H, E, k, R, C_, int(bool(fp8)))


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle status {code}")
        self.code = code


def layout(topk_idx: np.ndarray, E: int, R: int, C: int = 1, want_src: bool = True) -> dict:
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    out = dict(
        pos=np.empty((T, k), np.int32),
        expert_count=np.empty(E, np.int32),
        rank_count=np.empty(R, np.int32),
        recv_offset=np.empty(R + 1, np.int32),
        send_offset=np.empty((R, R), np.int32),
        chunk_offset=np.empty((C, R), np.int32),
        recv_src=np.empty(T * k, np.int32) if want_src else None,
    )
    st = lib().oracle_layout(T, E, k, R, C, _p(idx), _p(out["pos"]), _p(out["expert_count"]),
                             _p(out["rank_count"]), _p(out["recv_offset"]),
                             _p(out["send_offset"]), _p(out["chunk_offset"]),
                             _p(out["recv_src"]))
    if st != OK:
        raise OracleError(st)
    return out


def layout_grouped(topk_idx: np.ndarray, E: int, R: int, C: int = 1, want_src: bool = True) -> dict:
    """Expert-grouped layout: rows of each region in (expert, token, slot)
    order, plus expert_offset [E+1]."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    out = dict(
        pos=np.empty((T, k), np.int32),
        expert_count=np.empty(E, np.int32),
        expert_offset=np.empty(E + 1, np.int32),
        rank_count=np.empty(R, np.int32),
        recv_offset=np.empty(R + 1, np.int32),
        send_offset=np.empty((R, R), np.int32),
        chunk_offset=np.empty((C, R), np.int32),
        recv_src=np.empty(T * k, np.int32) if want_src else None,
    )
    st = lib().oracle_layout_grouped(T, E, k, R, C, _p(idx), _p(out["pos"]),
                                     _p(out["expert_count"]), _p(out["expert_offset"]),
                                     _p(out["rank_count"]), _p(out["recv_offset"]),
                                     _p(out["send_offset"]), _p(out["chunk_offset"]),
                                     _p(out["recv_src"]))
    if st != OK:
        raise OracleError(st)
    return out


def dispatch_bf16(x: np.ndarray, pos: np.ndarray, n_rows: int | None = None,
                  recv: np.ndarray | None = None) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    T, H = x.shape
    k = pos.shape[1]
    n_rows = T * k if n_rows is None else n_rows
    if recv is None:
        recv = np.zeros((n_rows, H), np.uint16)
    assert recv.shape == (n_rows, H) and recv.dtype == np.uint16 and recv.flags["C_CONTIGUOUS"]
    lib().oracle_dispatch_bf16(T, H, k, _p(x), _p(pos), _p(recv))
    return recv


def dispatch_fp8(x: np.ndarray, pos: np.ndarray, n_rows: int | None = None):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    T, H = x.shape
    k = pos.shape[1]
    assert H % 128 == 0
    n_rows = T * k if n_rows is None else n_rows
    q = np.zeros((n_rows, H), np.uint8)
    s = np.zeros((n_rows, H // 128), np.float32)
    lib().oracle_dispatch_fp8(T, H, k, _p(x), _p(pos), _p(q), _p(s))
    return q, s


def identity_fp8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    rows, H = q.shape
    y = np.empty((rows, H), np.uint16)
    lib().oracle_identity_fp8(rows, H, _p(q), _p(s), _p(y))
    return y


def combine(y: np.ndarray, pos: np.ndarray, topk_w: np.ndarray,
            out: np.ndarray | None = None) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.uint16)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, k = pos.shape
    H = y.shape[1]
    if out is None:
        out = np.empty((T, H), np.uint16)
    assert out.shape == (T, H) and out.dtype == np.uint16 and out.flags["C_CONTIGUOUS"]
    lib().oracle_combine(T, H, k, _p(y), _p(pos), _p(w), _p(out))
    return out


def f32_to_e4m3(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().oracle_f32_to_e4m3_array(a.size, _p(a), _p(out))
    return out


def e4m3_to_f32(c) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float32)
    lib().oracle_e4m3_to_f32_array(c.size, _p(c), _p(out))
    return out


def f32_to_bf16(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_f32_to_bf16_array(a.size, _p(a), _p(out))
    return out


def bf16_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


SOFTMAX, SIGMOID = 0, 1


def gate(logits: np.ndarray, k: int, groups: int = 1, keep_groups: int = 1,
         norm: int = SOFTMAX):
    """Top-k router on fp32 logits [T, E] -> (topk_idx int32 [T, k], topk_w fp32 [T, k]).
    Raises ValueError on arguments the definition excludes."""
    z = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = z.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    st = lib().oracle_gate(T, E, k, groups, keep_groups, norm, _p(z), _p(idx), _p(w))
    if st != OK:
        raise ValueError(f"oracle_gate: status {st}")
    return idx, w


def pipeline_tokens(x, topk_idx, topk_w, E, R, C=1, payload="bf16", tokens=None):
    """Oracle dispatch -> identity expert -> combine on a subset of tokens.

    Dispatch and combine of token t touch only token t's own k rows, so the
    outputs for a subset equal the outputs of the full problem at those tokens.
    The subset is laid out compactly (row t*k + j for sampled token t, slot j).
    Returns (rows, out): rows[n, k, ...] the dispatched rows in slot order and
    out[n, H] the combined tokens."""
    x = np.asarray(x)
    if tokens is None:
        tokens = np.arange(x.shape[0])
    tokens = np.asarray(tokens, dtype=np.int64)
    xs = np.ascontiguousarray(x[tokens])
    ws = np.ascontiguousarray(np.asarray(topk_w)[tokens])
    n, k = ws.shape
    H = xs.shape[1]
    pos_local = np.arange(n * k, dtype=np.int32).reshape(n, k)
    if payload == "bf16":
        recv = dispatch_bf16(xs, pos_local)
        y = recv
        rows = recv.reshape(n, k, H)
    else:
        q, s = dispatch_fp8(xs, pos_local)
        y = identity_fp8(q, s)
        rows = (q.reshape(n, k, H), s.reshape(n, k, H // 128))
    out = combine(y, pos_local, ws)
    return rows, out


def f64_to_bf16(v: float) -> int:
    return int(lib().oracle_f64_to_bf16(float(v)))


def expert_linear(x: np.ndarray, w: np.ndarray, expert_offset: np.ndarray) -> np.ndarray:
    """y[r] = bf16(x[r] @ w[e].T) in double for the rows r of expert e's run.
    x bf16 bits [rows, H]; w bf16 bits [E, N, H]; expert_offset int32 [E+1]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    off = np.ascontiguousarray(expert_offset, dtype=np.int32)
    E, N, H = w.shape
    assert x.shape[1] == H and off.shape == (E + 1,) and off[-1] <= x.shape[0]
    y = np.zeros((x.shape[0], N), np.uint16)
    lib().oracle_expert_linear(E, H, N, _p(off), _p(x), _p(w), _p(y))
    return y

"""ctypes binding of libubep.so (include/ubep.h, include/ubep_testing.h).

Argument marshalling only: tensors become raw pointers, the current torch
stream becomes the HIP stream, and a non-zero ubep_status raises UbepError.
Every computation runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libubep.so")

OK = 0
ERR_INVALID_ARG = 1
ERR_UNSUPPORTED = 2
ERR_BAD_EXPERT_ID = 3
ERR_TIMEOUT = 4
ERR_HIP = 5
ERR_BAD_POSITION = 6
ERR_WORKSPACE = 7
ERR_SENTINEL_DATA = 8
STATUS_NAMES = {OK: "UBEP_OK", ERR_INVALID_ARG: "UBEP_ERR_INVALID_ARG",
                ERR_UNSUPPORTED: "UBEP_ERR_UNSUPPORTED", ERR_BAD_EXPERT_ID: "UBEP_ERR_BAD_EXPERT_ID",
                ERR_TIMEOUT: "UBEP_ERR_TIMEOUT", ERR_HIP: "UBEP_ERR_HIP",
                ERR_BAD_POSITION: "UBEP_ERR_BAD_POSITION", ERR_WORKSPACE: "UBEP_ERR_WORKSPACE",
                ERR_SENTINEL_DATA: "UBEP_ERR_SENTINEL_DATA"}

BF16 = 0
FP8_E4M3 = 1


class ubep_shape(C.Structure):
    _fields_ = [("T", C.c_int64), ("H", C.c_int64), ("E", C.c_int32), ("k", C.c_int32),
                ("R", C.c_int32), ("C", C.c_int32)]


GATE_SOFTMAX = 0
GATE_SIGMOID = 1


class ubep_gate_shape(C.Structure):
    _fields_ = [("T", C.c_int64), ("E", C.c_int32), ("k", C.c_int32), ("groups", C.c_int32),
                ("keep_groups", C.c_int32), ("norm", C.c_int32)]


class UbepError(RuntimeError):
    def __init__(self, code: int, where: str = ""):
        self.code = code
        super().__init__(f"{where}: {STATUS_NAMES.get(code, code)} ({status_str(code)})")


_lib = None


def lib() -> C.CDLL:
    """Load libubep.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m combine_top_route_amd.build` (or __graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        P, S, I32, I64, U32, U64, SZ = (C.c_void_p, C.POINTER(ubep_shape), C.c_int32, C.c_int64,
                                        C.c_uint32, C.c_uint64, C.c_size_t)
        sig = {
            "ubep_abi_version": ([], C.c_int),
            "ubep_status_str": ([C.c_int], C.c_char_p),
            "ubep_check_shape": ([S, C.c_int], C.c_int),
            "ubep_workspace_bytes": ([S], SZ),
            "ubep_workspace_init": ([P, SZ, P], C.c_int),
            "ubep_layout": ([S, P, P, P, P, P, P, P, P, P, SZ, P], C.c_int),
            "ubep_layout_noalloc": ([S, P, P, P, P, P, P, P, P, P, C.c_int, P], C.c_int),
            "ubep_layout_grouped": ([S, P, P, P, P, P, P, P, P, P, P, SZ, P], C.c_int),
            "ubep_gate": ([C.POINTER(ubep_gate_shape), P, P, P, P], C.c_int),
            "ubep_gate_layout": ([C.POINTER(ubep_gate_shape), S, P, P, P, P, P, P, P, P, P, P, P, SZ,
                                  P], C.c_int),
            "ubep_layout_dispatch": ([S, P, P, P, P, P, P, P, P, P, P, P, SZ, P], C.c_int),
            "ubep_dispatch": ([S, C.c_int, P, P, P, P, P, SZ, P], C.c_int),
            "ubep_combine": ([S, P, P, P, P, P, SZ, P], C.c_int),
            "ubep_dispatch_combine_chunked": ([S, P, P, P, P, P, P, P, P, U64, U32, P, SZ, P], C.c_int),
            "ubep_chunk_order_lpt": ([S, P, P, P, P], C.c_int),
            "ubep_dispatch_combine_sentinel": ([S, P, P, P, P, P, U64, U32, P, SZ, P], C.c_int),
            "ubep_recv_sentinel_init": ([P, I64, I64, P], C.c_int),
            "ubep_expert_linear": ([S, I64, P, P, P, P, P, SZ, P], C.c_int),
            "ubep_expert_pack_weights": ([I32, I64, I64, P, P, P], C.c_int),
            "ubep_get_device_status": ([P, SZ, P, C.POINTER(C.c_int)], C.c_int),
            "ubep_identity_expert_fp8": ([I64, I64, P, P, P, P], C.c_int),
            "ubep_copy": ([P, P, SZ, P], C.c_int),
            "ubep_stream_probe": ([P, P, I64, C.c_int, C.c_int, P], C.c_int),
            "ubep_set_layout_workers": ([I32], C.c_int),
            "ubep_time_next_launch": ([P, P], C.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def status_str(code: int) -> str:
    return lib().ubep_status_str(code).decode()


def _shape(s) -> ubep_shape:
    if isinstance(s, ubep_shape):
        return s
    if isinstance(s, dict):
        return ubep_shape(s["T"], s["H"], s["E"], s["k"], s["R"], s.get("C", 1))
    return ubep_shape(s.T, s.H, s.E, s.k, s.R, getattr(s, "C", 1))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check(code: int, where: str):
    if code != OK:
        raise UbepError(code, where)


def ubep_abi_version() -> int:
    return lib().ubep_abi_version()


def ubep_check_shape(shape, dtype: int = BF16) -> int:
    s = _shape(shape)
    return lib().ubep_check_shape(C.byref(s), dtype)


def ubep_workspace_bytes(shape) -> int:
    s = _shape(shape)
    return lib().ubep_workspace_bytes(C.byref(s))


def ubep_workspace_init(ws, stream=None):
    _check(lib().ubep_workspace_init(_ptr(ws), _nbytes(ws), _stream(stream)), "ubep_workspace_init")


def ubep_gate(T, E, k, logits, topk_idx, topk_w, groups=1, keep_groups=1, norm=GATE_SOFTMAX,
              stream=None):
    g = ubep_gate_shape(T, E, k, groups, keep_groups, norm)
    _check(lib().ubep_gate(C.byref(g), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _stream(stream)),
           "ubep_gate")


def ubep_gate_layout(shape, logits, topk_idx, topk_w, pos, expert_count, rank_count, recv_offset,
                     send_offset, chunk_offset, recv_src, ws, groups=1, keep_groups=1,
                     norm=GATE_SOFTMAX, stream=None):
    s = _shape(shape)
    g = ubep_gate_shape(s.T, s.E, s.k, groups, keep_groups, norm)
    _check(lib().ubep_gate_layout(C.byref(g), C.byref(s), _ptr(logits), _ptr(topk_idx),
                                  _ptr(topk_w), _ptr(pos), _ptr(expert_count), _ptr(rank_count),
                                  _ptr(recv_offset), _ptr(send_offset), _ptr(chunk_offset),
                                  _ptr(recv_src), _ptr(ws), _nbytes(ws), _stream(stream)),
           "ubep_gate_layout")


def ubep_layout(shape, topk_idx, pos, expert_count, rank_count, recv_offset, send_offset,
                chunk_offset, recv_src, ws, stream=None):
    s = _shape(shape)
    _check(lib().ubep_layout(C.byref(s), _ptr(topk_idx), _ptr(pos), _ptr(expert_count),
                             _ptr(rank_count), _ptr(recv_offset), _ptr(send_offset),
                             _ptr(chunk_offset), _ptr(recv_src), _ptr(ws), _nbytes(ws),
                             _stream(stream)), "ubep_layout")


def ubep_layout_noalloc(shape, topk_idx, pos, expert_count, rank_count, recv_offset, send_offset,
                        chunk_offset, recv_src, status, reset=0, stream=None):
    s = _shape(shape)
    _check(lib().ubep_layout_noalloc(C.byref(s), _ptr(topk_idx), _ptr(pos), _ptr(expert_count),
                                     _ptr(rank_count), _ptr(recv_offset), _ptr(send_offset),
                                     _ptr(chunk_offset), _ptr(recv_src), _ptr(status), int(reset),
                                     _stream(stream)), "ubep_layout_noalloc")


def ubep_layout_grouped(shape, topk_idx, pos, expert_count, expert_offset, rank_count, recv_offset,
                        send_offset, chunk_offset, recv_src, ws, stream=None):
    s = _shape(shape)
    _check(lib().ubep_layout_grouped(C.byref(s), _ptr(topk_idx), _ptr(pos), _ptr(expert_count),
                                     _ptr(expert_offset), _ptr(rank_count), _ptr(recv_offset),
                                     _ptr(send_offset), _ptr(chunk_offset), _ptr(recv_src),
                                     _ptr(ws), _nbytes(ws), _stream(stream)), "ubep_layout_grouped")


def ubep_layout_dispatch(shape, topk_idx, x, pos, expert_count, rank_count, recv_offset,
                         send_offset, chunk_offset, recv_src, recv, ws, stream=None):
    s = _shape(shape)
    _check(lib().ubep_layout_dispatch(C.byref(s), _ptr(topk_idx), _ptr(x), _ptr(pos),
                                      _ptr(expert_count), _ptr(rank_count), _ptr(recv_offset),
                                      _ptr(send_offset), _ptr(chunk_offset), _ptr(recv_src),
                                      _ptr(recv), _ptr(ws), _nbytes(ws), _stream(stream)),
           "ubep_layout_dispatch")


def ubep_dispatch(shape, dtype, x, pos, recv, recv_scale, ws, stream=None):
    s = _shape(shape)
    _check(lib().ubep_dispatch(C.byref(s), dtype, _ptr(x), _ptr(pos), _ptr(recv), _ptr(recv_scale),
                               _ptr(ws), _nbytes(ws), _stream(stream)), "ubep_dispatch")


def ubep_combine(shape, y, pos, topk_w, out, ws, stream=None):
    s = _shape(shape)
    _check(lib().ubep_combine(C.byref(s), _ptr(y), _ptr(pos), _ptr(topk_w), _ptr(out), _ptr(ws),
                              _nbytes(ws), _stream(stream)), "ubep_combine")


def ubep_dispatch_combine_chunked(shape, x, pos, topk_w, recv, out, chunk_order, ws,
                                  spin_limit_ns: int = 0, debug_flags: int = 0, stream=None,
                                  chunk_offset=None, rank_count=None):
    """chunk_order: a host sequence of chunk ids, or None; chunk_offset and
    rank_count (device tensors from ubep_layout): the LPT order on the device."""
    s = _shape(shape)
    order = None
    if chunk_order is not None:
        order = (C.c_int32 * len(chunk_order))(*[int(c) for c in chunk_order])
    _check(lib().ubep_dispatch_combine_chunked(
        C.byref(s), _ptr(x), _ptr(pos), _ptr(topk_w), _ptr(recv), _ptr(out),
        C.cast(order, C.c_void_p) if order is not None else None, _ptr(chunk_offset),
        _ptr(rank_count), spin_limit_ns, debug_flags, _ptr(ws), _nbytes(ws), _stream(stream)),
        "ubep_dispatch_combine_chunked")


def ubep_chunk_order_lpt(shape, chunk_offset, rank_count, order, stream=None):
    s = _shape(shape)
    _check(lib().ubep_chunk_order_lpt(C.byref(s), _ptr(chunk_offset), _ptr(rank_count), _ptr(order),
                                      _stream(stream)), "ubep_chunk_order_lpt")


def ubep_dispatch_combine_sentinel(shape, x, pos, topk_w, recv, out, ws, spin_limit_ns: int = 0,
                                   debug_flags: int = 0, stream=None):
    s = _shape(shape)
    _check(lib().ubep_dispatch_combine_sentinel(
        C.byref(s), _ptr(x), _ptr(pos), _ptr(topk_w), _ptr(recv), _ptr(out), spin_limit_ns,
        debug_flags, _ptr(ws), _nbytes(ws), _stream(stream)), "ubep_dispatch_combine_sentinel")


def ubep_recv_sentinel_init(recv, rows, H, stream=None):
    _check(lib().ubep_recv_sentinel_init(_ptr(recv), rows, H, _stream(stream)),
           "ubep_recv_sentinel_init")


def ubep_expert_linear(shape, N, expert_offset, x, w, y, ws, stream=None):
    s = _shape(shape)
    _check(lib().ubep_expert_linear(C.byref(s), int(N), _ptr(expert_offset), _ptr(x), _ptr(w),
                                    _ptr(y), _ptr(ws), _nbytes(ws), _stream(stream)),
           "ubep_expert_linear")


def ubep_expert_pack_weights(E, N, H, w, packed, stream=None):
    _check(lib().ubep_expert_pack_weights(int(E), int(N), int(H), _ptr(w), _ptr(packed),
                                          _stream(stream)), "ubep_expert_pack_weights")


def ubep_get_device_status(ws, stream=None) -> int:
    out = C.c_int(-1)
    _check(lib().ubep_get_device_status(_ptr(ws), _nbytes(ws), _stream(stream), C.byref(out)),
           "ubep_get_device_status")
    return out.value


def ubep_identity_expert_fp8(rows, H, q, scale, y, stream=None):
    _check(lib().ubep_identity_expert_fp8(rows, H, _ptr(q), _ptr(scale), _ptr(y), _stream(stream)),
           "ubep_identity_expert_fp8")


def ubep_copy(src, dst, nbytes, stream=None):
    _check(lib().ubep_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)), "ubep_copy")


def ubep_stream_probe(src, dst, n_vec, fan_in, fan_out, stream=None):
    _check(lib().ubep_stream_probe(_ptr(src), _ptr(dst), int(n_vec), int(fan_in), int(fan_out),
                                   _stream(stream)), "ubep_stream_probe")


def ubep_time_next_launch(start, stop):
    """start / stop: hipEvent_t handles (ctypes.c_void_p or int), torch.cuda.Event
    objects that have been recorded once (so that they exist), or None / None
    to clear."""
    def handle(e):
        if e is None:
            return None
        if isinstance(e, C.c_void_p):
            h = e.value
        else:
            h = e.cuda_event if hasattr(e, "cuda_event") else int(e)
        if not h:
            raise ValueError("event not created yet: record it once first")
        return h
    _check(lib().ubep_time_next_launch(handle(start), handle(stop)), "ubep_time_next_launch")


def ubep_set_layout_workers(n: int):
    _check(lib().ubep_set_layout_workers(int(n)), "ubep_set_layout_workers")

"""Device buffers for one problem shape (torch allocations, no computation)."""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _abi


@dataclass
class Buffers:
    shape: dict
    dtype: int
    topk_idx: torch.Tensor       # int32 [T, k]
    topk_w: torch.Tensor         # fp32  [T, k]
    x: torch.Tensor              # bf16  [T, H]
    pos: torch.Tensor            # int32 [T, k]
    expert_count: torch.Tensor   # int32 [E]
    rank_count: torch.Tensor     # int32 [R]
    recv_offset: torch.Tensor    # int32 [R + 1]
    send_offset: torch.Tensor    # int32 [R, R]
    chunk_offset: torch.Tensor   # int32 [C, R]
    recv_src: torch.Tensor       # int32 [T * k]
    recv: torch.Tensor           # bf16 [T*k, H] or uint8 [T*k, H]
    recv_scale: torch.Tensor | None   # fp32 [T*k, H/128] (fp8 only)
    y: torch.Tensor              # bf16 [T*k, H] combine input (aliases recv for bf16)
    out: torch.Tensor            # bf16 [T, H]
    ws: torch.Tensor             # uint8 workspace


def alloc_buffers(shape: dict, dtype: int = _abi.BF16, device="cuda", x_bits=None, topk_idx=None,
                  topk_w=None) -> Buffers:
    """Allocate every device buffer of the path for `shape`; optionally upload
    host inputs (numpy uint16 bf16 bits, int32 ids, fp32 weights)."""
    T, H, E, k, R, C = (shape[n] for n in ("T", "H", "E", "k", "R", "C"))
    rows = T * k
    dev = torch.device(device)

    def up(a, dt, shp):
        if a is None:
            return torch.zeros(shp, dtype=dt, device=dev)
        t = torch.from_numpy(a)
        if dt == torch.bfloat16:
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(dev).reshape(shp).contiguous()

    if dtype == _abi.BF16:
        recv = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
        recv_scale = None
        y = recv
    else:
        recv = torch.empty((rows, H), dtype=torch.uint8, device=dev)
        recv_scale = torch.empty((rows, H // 128), dtype=torch.float32, device=dev)
        y = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    nws = _abi.ubep_workspace_bytes(shape)
    if nws == 0:
        raise _abi.UbepError(_abi.ubep_check_shape(shape, dtype) or _abi.ERR_INVALID_ARG,
                             "alloc_buffers")
    return Buffers(
        shape=dict(shape), dtype=dtype,
        topk_idx=up(topk_idx, torch.int32, (T, k)),
        topk_w=up(topk_w, torch.float32, (T, k)),
        x=up(x_bits, torch.bfloat16, (T, H)),
        pos=torch.empty((T, k), dtype=torch.int32, device=dev),
        expert_count=torch.empty(E, dtype=torch.int32, device=dev),
        rank_count=torch.empty(R, dtype=torch.int32, device=dev),
        recv_offset=torch.empty(R + 1, dtype=torch.int32, device=dev),
        send_offset=torch.empty((R, R), dtype=torch.int32, device=dev),
        chunk_offset=torch.zeros((C, R), dtype=torch.int32, device=dev),
        recv_src=torch.empty(rows, dtype=torch.int32, device=dev),
        recv=recv, recv_scale=recv_scale, y=y,
        out=torch.empty((T, H), dtype=torch.bfloat16, device=dev),
        ws=torch.zeros(nws, dtype=torch.uint8, device=dev),
    )


def run_path(b: Buffers, stream=None, chunked: bool = False, chunk_order=None, fused: bool = False):
    """Layout, dispatch, identity expert, combine on the buffers (library calls).
    fused: layout and dispatch in one launch (bf16 payload, not chunked).
    chunk_order (chunked): a host list of chunk ids, None (index order), or
    "lpt" (the imbalance-aware order computed on the device)."""
    s = b.shape
    if fused and not chunked and b.dtype == _abi.BF16:
        _abi.ubep_layout_dispatch(s, b.topk_idx, b.x, b.pos, b.expert_count, b.rank_count,
                                  b.recv_offset, b.send_offset,
                                  b.chunk_offset if s["C"] > 1 else None, b.recv_src, b.recv,
                                  b.ws, stream)
        _abi.ubep_combine(s, b.y, b.pos, b.topk_w, b.out, b.ws, stream)
        return
    _abi.ubep_layout(s, b.topk_idx, b.pos, b.expert_count, b.rank_count, b.recv_offset,
                     b.send_offset, b.chunk_offset if s["C"] > 1 else None, b.recv_src, b.ws,
                     stream)
    if chunked:
        if isinstance(chunk_order, str) and chunk_order == "lpt":   # the device's LPT order
            _abi.ubep_dispatch_combine_chunked(s, b.x, b.pos, b.topk_w, b.recv, b.out, None, b.ws,
                                               stream=stream,
                                               chunk_offset=b.chunk_offset if s["C"] > 1 else None,
                                               rank_count=b.rank_count)
        else:
            _abi.ubep_dispatch_combine_chunked(s, b.x, b.pos, b.topk_w, b.recv, b.out, chunk_order,
                                               b.ws, stream=stream)
        return
    _abi.ubep_dispatch(s, b.dtype, b.x, b.pos, b.recv, b.recv_scale, b.ws, stream)
    if b.dtype == _abi.FP8_E4M3:
        _abi.ubep_identity_expert_fp8(s["T"] * s["k"], s["H"], b.recv, b.recv_scale, b.y, stream)
    _abi.ubep_combine(s, b.y, b.pos, b.topk_w, b.out, b.ws, stream)

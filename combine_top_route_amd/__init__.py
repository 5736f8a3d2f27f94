"""MoE token dispatch / combine for MI355X (gfx950).

The computation lives in libubep.so (hand-written HIP kernels behind the C ABI
of include/ubep.h).  This package is the Python binding (ctypes marshalling of
torch device tensors and streams) plus device-buffer helpers.
"""
from ._abi import (BF16, ERR_BAD_EXPERT_ID, ERR_BAD_POSITION, ERR_HIP, ERR_INVALID_ARG, ERR_TIMEOUT,
                   ERR_SENTINEL_DATA, ERR_UNSUPPORTED, ERR_WORKSPACE, FP8_E4M3, GATE_SIGMOID, GATE_SOFTMAX, LIB_PATH, OK, STATUS_NAMES,
                   UbepError, lib, status_str, ubep_abi_version, ubep_check_shape, ubep_combine,
                   ubep_copy, ubep_dispatch, ubep_stream_probe, ubep_gate, ubep_gate_layout, ubep_gate_shape,
                   ubep_chunk_order_lpt, ubep_dispatch_combine_chunked, ubep_dispatch_combine_sentinel, ubep_expert_linear,
                   ubep_expert_pack_weights,
                   ubep_get_device_status, ubep_recv_sentinel_init, ubep_identity_expert_fp8,
                   ubep_layout, ubep_layout_dispatch, ubep_layout_grouped, ubep_layout_noalloc,
                   ubep_set_layout_workers,
                   ubep_shape,
                   ubep_time_next_launch, ubep_workspace_bytes, ubep_workspace_init)
from .buffers import Buffers, alloc_buffers

__all__ = [n for n in dir() if not n.startswith("_")]

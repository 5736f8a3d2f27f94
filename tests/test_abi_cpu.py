"""The C-ABI library without a GPU: it loads, exports every function that
include/*.h declares, and its host-side validation rejects bad arguments
before anything is enqueued (no HIP call is reached on these paths)."""
import ctypes as C
import os
import re

import pytest

import combine_top_route_amd as ubep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = "".join(open(os.path.join(ROOT, "include", h)).read()
                  for h in sorted(os.listdir(os.path.join(ROOT, "include"))) if h.endswith(".h"))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ubep_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_path():
    names = _declared()
    for n in ("ubep_layout", "ubep_dispatch", "ubep_combine", "ubep_dispatch_combine_chunked",
              "ubep_workspace_bytes", "ubep_get_device_status"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = C.CDLL(ubep.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing
    assert ubep.ubep_abi_version() == 2


def test_shape_validation():
    ok = dict(T=4096, H=7168, E=256, k=8, R=32, C=1)
    assert ubep.ubep_check_shape(ok) == ubep.OK
    assert ubep.ubep_check_shape(ok, ubep.FP8_E4M3) == ubep.OK
    bad = [dict(ok, T=0), dict(ok, E=250), dict(ok, T=4001), dict(ok, C=3), dict(ok, H=7170),
           dict(ok, k=300, E=256), dict(ok, T=1 << 28)]
    for s in bad:
        assert ubep.ubep_check_shape(s) == ubep.ERR_INVALID_ARG, s
    assert ubep.ubep_check_shape(dict(ok, H=7168 + 64), ubep.FP8_E4M3) == ubep.ERR_INVALID_ARG
    assert ubep.ubep_check_shape(dict(ok, k=33, E=256)) == ubep.ERR_UNSUPPORTED
    assert ubep.ubep_check_shape(dict(ok, R=2048, E=4096, T=4096)) == ubep.ERR_UNSUPPORTED
    assert ubep.ubep_check_shape(dict(ok, C=512, T=8192)) == ubep.ERR_UNSUPPORTED
    assert ubep.ubep_check_shape(ok, 7) == ubep.ERR_INVALID_ARG


def test_layout_worker_cap_argument():
    with pytest.raises(ubep.UbepError) as e:
        ubep.ubep_set_layout_workers(-1)
    assert e.value.code == ubep.ERR_INVALID_ARG
    ubep.ubep_set_layout_workers(7)
    ubep.ubep_set_layout_workers(0)


def test_time_next_launch_arguments():
    with pytest.raises(ubep.UbepError) as e:       # one event of the pair missing
        ubep.ubep_time_next_launch(1234, None)
    assert e.value.code == ubep.ERR_INVALID_ARG
    ubep.ubep_time_next_launch(None, None)          # clearing is always valid


def test_workspace_size():
    s = dict(T=4096, H=7168, E=256, k=8, R=32, C=1)
    n = ubep.ubep_workspace_bytes(s)
    assert n > 0 and n % 256 == 0
    assert ubep.ubep_workspace_bytes(dict(s, E=250)) == 0
    big = ubep.ubep_workspace_bytes(dict(T=65536, H=7168, E=256, k=8, R=64, C=16))
    assert 0 < big < 64 << 20


def test_validation_happens_before_any_launch():
    L = ubep.lib()
    s = ubep.ubep_shape(8, 64, 4, 2, 2, 1)
    # null pointers, bad shapes and bad dtypes fail on the host
    assert L.ubep_layout(C.byref(s), None, None, None, None, None, None, None, None, None, 0,
                         None) == ubep.ERR_INVALID_ARG
    assert L.ubep_dispatch(C.byref(s), 3, 16, 16, 16, None, 256, 4096, None) == ubep.ERR_INVALID_ARG
    assert L.ubep_dispatch(C.byref(s), 0, 8, 16, 16, None, 256, 4096, None) == \
        ubep.ERR_INVALID_ARG                                       # x not 16-byte aligned
    assert L.ubep_combine(C.byref(ubep.ubep_shape(0, 64, 4, 2, 2, 1)), 16, 16, 16, 16, 256, 4096,
                          None) == ubep.ERR_INVALID_ARG
    assert L.ubep_workspace_init(None, 0, None) == ubep.ERR_INVALID_ARG
    assert L.ubep_copy(16, 16, 17, None) == ubep.ERR_INVALID_ARG
    assert L.ubep_identity_expert_fp8(4, 100, 16, 16, 16, None) == ubep.ERR_INVALID_ARG
    order = (C.c_int32 * 2)(0, 0)
    s2 = ubep.ubep_shape(8, 64, 4, 2, 2, 2)
    nws = L.ubep_workspace_bytes(C.byref(s2))
    assert L.ubep_dispatch_combine_chunked(C.byref(s2), 16, 16, 16, 16, 16, order, None, None, 0,
                                           0, 256, nws, None) == ubep.ERR_INVALID_ARG
    assert L.ubep_dispatch_combine_chunked(C.byref(s2), 16, 16, 16, 16, 16, None, None, None, 0, 4,
                                           256, nws, None) == ubep.ERR_INVALID_ARG  # unknown flag
    good = (C.c_int32 * 2)(1, 0)
    assert L.ubep_dispatch_combine_chunked(C.byref(s2), 16, 16, 16, 16, 16, good, 256, 256, 0, 0,
                                           256, nws, None) == ubep.ERR_INVALID_ARG  # two orders
    assert L.ubep_dispatch_combine_chunked(C.byref(s2), 16, 16, 16, 16, 16, None, None, 256, 0, 0,
                                           256, nws, None) == ubep.ERR_INVALID_ARG  # no chunk_offset
    assert L.ubep_dispatch_combine_chunked(C.byref(s2), 16, 16, 16, 16, 16, None, 256, None, 0, 0,
                                           256, nws, None) == ubep.ERR_INVALID_ARG  # no rank_count
    assert L.ubep_chunk_order_lpt(C.byref(s2), None, 256, 256, None) == ubep.ERR_INVALID_ARG
    assert L.ubep_chunk_order_lpt(C.byref(s2), 256, 256, None, None) == ubep.ERR_INVALID_ARG
    assert L.ubep_dispatch_combine_sentinel(C.byref(s2), 16, 16, 16, 16, 16, 0, 4, 256, nws,
                                            None) == ubep.ERR_INVALID_ARG  # unknown debug flag
    assert ubep.status_str(ubep.ERR_TIMEOUT) == "ready-flag wait timed out"


def test_product_path_has_no_oracle_or_fallback():
    """The package never imports the oracle or a CPU path."""
    pkg = os.path.join(ROOT, "combine_top_route_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            txt = open(os.path.join(pkg, f)).read()
            assert "import oracle" not in txt and "from oracle" not in txt, f


def test_gate_validation_without_gpu():
    """Invalid gate shapes return before any launch (dummy pointers are never used)."""
    p = 256
    cases = [dict(T=0, E=8, k=2), dict(T=4, E=8, k=9), dict(T=4, E=8, k=2, groups=3),
             dict(T=4, E=8, k=2, groups=4, keep_groups=5), dict(T=4, E=8, k=5, groups=4, keep_groups=2),
             dict(T=4, E=8, k=2, norm=2)]
    for c in cases:
        with pytest.raises(ubep.UbepError) as e:
            ubep.ubep_gate(c["T"], c["E"], c["k"], p, p, p, c.get("groups", 1), c.get("keep_groups", 1),
                           c.get("norm", 0), stream=0)
        assert e.value.code == ubep.ERR_INVALID_ARG, c
    for c in (dict(T=4, E=2048, k=2), dict(T=4, E=256, k=33), dict(T=4, E=256, k=2, groups=128)):
        with pytest.raises(ubep.UbepError) as e:
            ubep.ubep_gate(c["T"], c["E"], c["k"], p, p, p, c.get("groups", 1), c.get("keep_groups", 1), 0,
                           stream=0)
        assert e.value.code == ubep.ERR_UNSUPPORTED, c


def test_grouped_layout_validation_without_gpu():
    """ubep_layout_grouped: null outputs and LDS-exceeding expert counts fail on
    the host (dummy pointers are never used)."""
    L = ubep.lib()
    s = ubep.ubep_shape(8, 64, 4, 2, 2, 1)
    nws = L.ubep_workspace_bytes(C.byref(s))
    assert L.ubep_layout_grouped(C.byref(s), 256, 256, 256, None, 256, 256, 256, None, None, 256,
                                 nws, None) == ubep.ERR_INVALID_ARG        # no expert_offset
    big = ubep.ubep_shape(8192, 64, 8192, 2, 1, 1)                          # 8192 experts
    nws = L.ubep_workspace_bytes(C.byref(big))
    assert nws > 0
    assert L.ubep_layout_grouped(C.byref(big), 256, 256, 256, 256, 256, 256, 256, None, None, 256,
                                 nws, None) == ubep.ERR_UNSUPPORTED


def test_sentinel_pipeline_validation_without_gpu():
    L = ubep.lib()
    s = ubep.ubep_shape(8, 64, 4, 2, 2, 1)
    nws = L.ubep_workspace_bytes(C.byref(s))
    assert L.ubep_dispatch_combine_sentinel(C.byref(s), 16, 16, 16, 16, None, 0, 0, 256, nws,
                                            None) == ubep.ERR_INVALID_ARG          # no out
    assert L.ubep_dispatch_combine_sentinel(C.byref(s), 16, 16, 16, 16, 16, 0, 4, 256, nws,
                                            None) == ubep.ERR_INVALID_ARG          # unknown flag
    assert L.ubep_recv_sentinel_init(256, 4, 12, None) == ubep.ERR_INVALID_ARG   # H % 8 != 0
    assert L.ubep_recv_sentinel_init(8, 4, 16, None) == ubep.ERR_INVALID_ARG     # misaligned
    assert L.ubep_recv_sentinel_init(256, 0, 16, None) == ubep.OK                # nothing to do
    assert ubep.status_str(ubep.ERR_SENTINEL_DATA) == "input row holds the readiness sentinel word"


def test_expert_linear_validation_without_gpu():
    L = ubep.lib()
    s = ubep.ubep_shape(64, 128, 8, 2, 2, 1)
    assert L.ubep_expert_linear(C.byref(s), 100, 256, 256, 256, 256, 256, 4096,
                                None) == ubep.ERR_UNSUPPORTED           # N % 128 != 0
    s2 = ubep.ubep_shape(64, 96, 8, 2, 2, 1)
    assert L.ubep_expert_linear(C.byref(s2), 128, 256, 256, 256, 256, 256, 4096,
                                None) == ubep.ERR_UNSUPPORTED           # H % 64 != 0
    assert L.ubep_expert_linear(C.byref(s), 128, None, 256, 256, 256, 256, 4096,
                                None) == ubep.ERR_INVALID_ARG           # no expert_offset
    big = ubep.ubep_shape(2048, 128, 2048, 2, 2, 1)
    assert L.ubep_expert_linear(C.byref(big), 128, 256, 256, 256, 256, 256, 4096,
                                None) == ubep.ERR_UNSUPPORTED           # E > 1024


def test_expert_pack_validation_without_gpu():
    L = ubep.lib()
    assert L.ubep_expert_pack_weights(2, 100, 128, 256, 512, None) == ubep.ERR_UNSUPPORTED   # N
    assert L.ubep_expert_pack_weights(2, 128, 96, 256, 512, None) == ubep.ERR_UNSUPPORTED    # H
    assert L.ubep_expert_pack_weights(2, 128, 128, 256, 256, None) == ubep.ERR_INVALID_ARG   # in place
    assert L.ubep_expert_pack_weights(0, 128, 128, 256, 512, None) == ubep.ERR_INVALID_ARG

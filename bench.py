#!/usr/bin/env python3
"""MoE token dispatch + combine on one MI355X: HBM GB/s and tokens/s.

One step = the whole path over one synthetic batch already resident in HBM:
ubep_layout (counts, prefix sums, positions) -> ubep_dispatch (rows into the
R receive regions) -> identity expert (y = recv) -> ubep_combine (slot-ordered
FMA chain back to token order).  `--mode chunked` runs layout + the one-kernel
chunk pipeline instead of the two row kernels; `--order expert` takes the layout
from ubep_layout_grouped (rows of each region grouped by expert).

Throughput counts algorithmic bytes (what the path must read and write):
  layout   4Tk (ids) + 4Tk (positions)
  dispatch 2TH + 4Tk + 2TkH            (bf16)   |  2TH + 4Tk + TkH + 4TkH/128  (fp8)
  combine  2TkH + 8Tk + 2TH
  gate     4TE + 8Tk  (`--mode gated`: the step starts from router logits)
Time comes from HIP events on the stream the library launches on, only at the
two ends of K steps (an event record between kernels leaves the GPU idle for
microseconds).  The headline is the cold pass: every step follows a 512 MB read
scrub, and the K scrubs, timed alone the same way, are subtracted; the warm
(back-to-back) pass is reported beside it.  The dominant kernel's duration comes
from a separate pass in which events its own launch records time it
(ubep_time_next_launch).  The DeepSeek-V3 decode line also carries its Zipf-skewed
twin, sequential-stream ceilings measured in the same run, and the CPU oracle
pinned to one host core.

Prints one JSON line.  Only one GPU is measured: `--gpus N` with N > 1 exits
with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine HBM GB/s (% of MI355X peak) and tokens/s, 1 GPU"
HBM_PEAK_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.txt")


def algorithmic_bytes(s: dict, fp8: bool, gate: bool = False, expert_w_bytes: int = -1) -> dict:
    """expert_w_bytes >= 0: the step also runs the per-expert linear map (N = H),
    which reads the weights of the experts that received rows (that many
    bytes), the T*k receive rows, and writes T*k output rows."""
    T, H, k = s["T"], s["H"], s["k"]
    layout = 8 * T * k
    gate_b = 4 * T * s["E"] + 8 * T * k if gate else 0
    expert = expert_w_bytes + 4 * T * k * H + 4 * (s["E"] + 1) if expert_w_bytes >= 0 else 0
    if fp8:
        dispatch = 2 * T * H + 4 * T * k + T * k * H + 4 * T * k * (H // 128)
    else:
        dispatch = 2 * T * H + 4 * T * k + 2 * T * k * H
    combine = 2 * T * k * H + 8 * T * k + 2 * T * H
    return dict(gate=gate_b, layout=layout, dispatch=dispatch, combine=combine, expert=expert,
                total=gate_b + layout + dispatch + expert + combine)


# the sources each counted kernel is built from (its own file and the headers
# it includes); counters taken on other sources are not used
KERNEL_SOURCES = {
    "combine": ["combine.hip", "rows.h", "launch.h", "device_common.h", "plan.h"],
    "dispatch": ["dispatch.hip", "rows.h", "launch.h", "device_common.h", "plan.h"],
    "layout": ["layout.hip", "layout_worker.h", "launch.h", "device_common.h", "plan.h", "api.hip"],
    "expert": ["expert.hip", "rows.h", "launch.h", "device_common.h", "plan.h"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "combine_top_route_amd", "csrc")
    for f in sorted(KERNEL_SOURCES.get(kernel, os.listdir(csrc))):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def read_counters(kernel: str, workload: str):
    """HBM traffic of `kernel` from the committed rocprofv3 counter summary,
    scaled by the copy-kernel calibration; None when absent or when the
    kernel sources changed after the counters were taken."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    rows = {}
    with open(COUNTERS_FILE) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kv = dict(p.split("=", 1) for p in line.split())
            rows[(kv.get("kind"), kv.get("kernel"), kv.get("workload"))] = kv
    cal = next((v for (kind, _, _), v in rows.items() if kind == "copy"), None)
    got = rows.get(("kernel", kernel, workload))
    if cal is None or got is None or got.get("source") != source_hash(kernel):
        return None
    copy_bytes = float(cal["bytes"])
    f_scale = copy_bytes / (float(cal["fetch_kib"]) * 1024.0)
    w_scale = copy_bytes / (float(cal["write_kib"]) * 1024.0)
    return float(got["fetch_kib"]) * 1024.0 * f_scale + float(got["write_kib"]) * 1024.0 * w_scale


class HipEvents:
    """Timing events made through the HIP runtime (torch's take no flags), with
    hipEventDisableSystemFence: recording one then skips the system-scope cache
    writeback and invalidate, which would otherwise add microseconds to every
    timed step."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes as C
        self.C = C
        self.hip = C.CDLL("libamdhip64.so.7")     # the runtime torch and libubep already share
        self.hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self.hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.made = []

    def pair(self):
        out = []
        for _ in range(2):
            e = self.C.c_void_p()
            if self.hip.hipEventCreateWithFlags(self.C.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.made.append(e)
            out.append(e)
        return tuple(out)

    def record(self, e, stream):
        if self.hip.hipEventRecord(e, self.C.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_us(self, pair):
        ms = self.C.c_float()
        if self.hip.hipEventElapsedTime(self.C.byref(ms), pair[0], pair[1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1e3

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(e)
        self.made = []


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float = 10.0, min_reps: int = 3) -> dict:
    """The CPU oracle (single-threaded C) on the same batch: layout + dispatch
    + combine, outputs preallocated; this process pinned to one host core for
    the runs; median of as many runs as fit in about budget_s seconds."""
    import numpy as np

    import oracle
    s = w.shape
    fp8 = w.recipe.payload == "fp8"
    rows = s.T * s.k
    recv = np.empty((rows, s.H), np.uint16) if not fp8 else None
    out = np.empty((s.T, s.H), np.uint16)
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[0]
    os.sched_setaffinity(0, {core})
    times = []
    try:
        t_start = time.perf_counter()
        while len(times) < min_reps or time.perf_counter() - t_start < budget_s:
            t0 = time.perf_counter()
            L = oracle.layout(w.topk_idx, s.E, s.R, s.C, want_src=False)
            if fp8:
                q, sc = oracle.dispatch_fp8(w.x, L["pos"])
                t1 = time.perf_counter()
                y = oracle.identity_fp8(q, sc)         # the identity expert is not timed
                t2 = time.perf_counter()
            else:
                y = oracle.dispatch_bf16(w.x, L["pos"], recv=recv)
                t1 = t2 = time.perf_counter()
            oracle.combine(y, L["pos"], w.topk_w, out=out)
            t3 = time.perf_counter()
            times.append((t1 - t0) + (t3 - t2))
    finally:
        os.sched_setaffinity(0, set(allowed))
    med = statistics.median(times)
    nbytes = algorithmic_bytes(s.as_dict(), fp8)["total"]
    return {"value": round(nbytes / med / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"whole batch ({s.T} tokens) of the benchmarked workload, median of "
                      f"{len(times)} runs of layout+dispatch+combine (about {budget_s:.0f} s of "
                      f"CPU work), process pinned to host core {core}",
            "seconds_per_step": round(med, 4), "tokens_per_s": round(s.T / med, 1),
            "host_cores": len(allowed), "cores_used": f"1 of {len(allowed)}",
            "cpu_model": cpu_model()}


def copy_reference(nbytes: int, reps: int) -> int:
    """Time ubep_copy on `nbytes` bytes (src and dst distinct, 16-byte multiple)."""
    import torch

    import combine_top_route_amd as ubep
    nbytes -= nbytes % 16
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream()
    ubep.ubep_copy(src, dst, nbytes, st)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(st)
    for i in range(reps):
        ubep.ubep_copy(src, dst, nbytes, st)
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    us = statistics.median(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps))
    print(json.dumps({"copy_bytes": nbytes, "reps": reps, "us": round(us, 2),
                      "GBs": round(2 * nbytes / us / 1e3, 1)}), flush=True)
    return 0


def companion_of(name: str):
    """The skewed twin a bench line reports beside its workload: the DeepSeek-V3
    decode step under Zipf(1.2) routing (same shape, skewed load)."""
    return {"dsv3_decode_T4096_H7168_E256_k8_R32": "dsv3_decode_zipf_T4096_H7168_E256_k8_R32"}.get(name)


def measure(name: str, args, hev) -> dict:
    """Allocate one workload, run warm-up, an untimed calibration pass (every
    kernel timed by its own launch), then K timed steps warm and K cold.
    Returns timings and counts; raises on a device error."""
    import torch

    import combine_top_route_amd as ubep
    from combine_top_route_amd.buffers import alloc_buffers
    from workloads import make_config

    w = make_config(name)
    s = w.shape
    sd = s.as_dict()
    fp8 = w.recipe.payload == "fp8"
    dtype = ubep.FP8_E4M3 if fp8 else ubep.BF16
    order = "expert" if args.mode == "moe" else args.order
    b = alloc_buffers(sd, dtype, "cuda", x_bits=w.x, topk_idx=w.topk_idx, topk_w=w.topk_w)
    stream = torch.cuda.current_stream()
    chunk_off = b.chunk_offset if s.C > 1 else None
    expert_off = torch.empty(s.E + 1, dtype=torch.int32, device="cuda")
    scrub_buf = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    scrub_sink = torch.empty(16, dtype=torch.uint8, device="cuda")

    calls = ["layout"] + ([args.mode] if args.mode in ("chunked", "sentinel")
                          else ["dispatch", "combine"])
    if args.mode == "sentinel":
        ubep.ubep_recv_sentinel_init(b.recv, s.T * s.k, s.H)
    moe = args.mode == "moe"
    if moe:
        calls = ["layout", "dispatch", "expert", "combine"]
        gen = torch.Generator(device="cuda").manual_seed(w.recipe.seed)
        wexp = torch.randn((s.E, s.H, s.H), generator=gen, dtype=torch.bfloat16, device="cuda")
        wexp.mul_(1.0 / float(s.H) ** 0.5)
        wpacked = torch.empty_like(wexp)
        ubep.ubep_expert_pack_weights(s.E, s.H, s.H, wexp, wpacked)
        del wexp
        yexp = torch.empty((s.T * s.k, s.H), dtype=torch.bfloat16, device="cuda")
    if args.mode == "fused":
        calls = ["layout_dispatch", "combine"]
    gated = args.mode in ("gated", "gate_layout")
    if gated:
        from workloads import router_logits
        calls = (["gate"] + calls if args.mode == "gated"
                 else ["gate_layout"] + [c for c in calls if c != "layout"])
        logits = torch.from_numpy(router_logits(w.recipe)).cuda()
        grouped = w.recipe.routing == "group_zipf"
        gate_args = dict(groups=w.recipe.n_groups if grouped else 1,
                         keep_groups=w.recipe.topk_groups if grouped else 1,
                         norm=ubep.GATE_SIGMOID if w.recipe.weights == "sigmoid" else ubep.GATE_SOFTMAX)
    lpt = args.chunk_order == "lpt"

    sdc = ubep._abi._shape(sd)               # the C struct, built once (host time per call)

    def call(cname, st):
        if cname == "gate":
            ubep.ubep_gate(s.T, s.E, s.k, logits, b.topk_idx, b.topk_w, stream=st, **gate_args)
        elif cname == "gate_layout":
            ubep.ubep_gate_layout(sdc, logits, b.topk_idx, b.topk_w, b.pos, b.expert_count,
                                  b.rank_count, b.recv_offset, b.send_offset, chunk_off, None, b.ws,
                                  stream=st, **gate_args)
        elif cname == "layout" and order == "expert":
            ubep.ubep_layout_grouped(sdc, b.topk_idx, b.pos, b.expert_count, expert_off, b.rank_count,
                                     b.recv_offset, b.send_offset, chunk_off, None, b.ws, st)
        elif cname == "layout":
            ubep.ubep_layout(sdc, b.topk_idx, b.pos, b.expert_count, b.rank_count, b.recv_offset,
                             b.send_offset, chunk_off, None, b.ws, st)
        elif cname == "layout_dispatch":
            ubep.ubep_layout_dispatch(sdc, b.topk_idx, b.x, b.pos, b.expert_count, b.rank_count,
                                      b.recv_offset, b.send_offset, chunk_off, None, b.recv, b.ws,
                                      st)
        elif cname == "expert":
            ubep.ubep_expert_linear(sdc, s.H, expert_off, b.recv, wpacked, yexp, b.ws, st)
        elif cname == "sentinel":
            ubep.ubep_dispatch_combine_sentinel(sdc, b.x, b.pos, b.topk_w, b.recv, b.out, b.ws,
                                                stream=st)
        elif cname == "chunked":
            ubep.ubep_dispatch_combine_chunked(sdc, b.x, b.pos, b.topk_w, b.recv, b.out, None, b.ws,
                                               stream=st, **(dict(chunk_offset=chunk_off,
                                                                  rank_count=b.rank_count)
                                                             if lpt else {}))
        elif cname == "dispatch":
            ubep.ubep_dispatch(sdc, dtype, b.x, b.pos, b.recv, b.recv_scale, b.ws, st)
        else:
            ubep.ubep_combine(sdc, yexp if moe else b.y, b.pos, b.topk_w, b.out, b.ws, st)

    def step(timed=None):
        """One step.  `timed` maps a call name (or 'identity', the fp8 identity
        expert between dispatch and combine) to a (start, stop) event pair that
        the call's kernel launch records at its own start and end."""
        st = torch.cuda.current_stream().cuda_stream   # the capture stream while a graph records
        for cname in calls:
            if timed and cname in timed:
                ubep.ubep_time_next_launch(*timed[cname])
            call(cname, st)
            if cname == "dispatch" and fp8:
                if timed and "identity" in timed:
                    ubep.ubep_time_next_launch(*timed["identity"])
                ubep.ubep_identity_expert_fp8(s.T * s.k, s.H, b.recv, b.recv_scale, b.y, st)

    def pairs(n):
        return [hev.pair() for _ in range(n)]

    elapsed_us = hev.elapsed_us

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = ubep.ubep_get_device_status(b.ws)
    if st != ubep.OK:
        raise RuntimeError(f"{name}: device status after warm-up: {ubep.STATUS_NAMES.get(st, st)}")

    ew_bytes = -1
    if moe:    # weights of the experts that received rows are what the expert must read
        ew_bytes = int((b.expert_count > 0).sum().item()) * s.H * s.H * 2

    # untimed calibration: every kernel timed by its own launch, to find the
    # dominant one and to give each kernel's own rate
    cal = [{n: p for n, p in zip(calls, pairs(len(calls)))} for _ in range(10)]
    torch.cuda.synchronize()
    for c in cal:
        step(c)
    torch.cuda.synchronize()
    per_call = {n: statistics.median(elapsed_us(c[n]) for c in cal) for n in calls}
    dom = max((n for n in calls if n not in ("layout", "gate", "gate_layout")), key=lambda n: per_call[n])
    if dom == "layout_dispatch":
        dom = "combine"      # the fused launch also holds the layout's latency chain

    # the scrub of the cold pass: a read stream over 512 MB of unrelated data,
    # which evicts the path's arrays from the 256 MB memory-side cache and the
    # L2s and leaves clean lines behind (a write scrub would leave dirty lines
    # that the next step pays to write back)
    def scrub():
        ubep.ubep_stream_probe(scrub_buf, scrub_sink, scrub_buf.numel() // 16 // 8, 8, 0, stream)

    def region_us(body, reps):
        """Time `reps` calls of body() between two events: no event inside the
        region (each event record leaves the GPU idle for microseconds)."""
        region = hev.pair()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        hev.record(region[0], stream)
        for _ in range(reps):
            body()
        hev.record(region[1], stream)
        torch.cuda.synchronize()
        return elapsed_us(region), time.perf_counter() - t0

    def kernel_pass():
        """K steps with the dominant kernel (and the fp8 identity expert) timed
        by events their own launches record: their mean durations."""
        dom_pairs = pairs(args.steps)
        id_pairs = pairs(args.steps) if fp8 else None
        torch.cuda.synchronize()
        for i in range(args.steps):
            timed = {dom: dom_pairs[i]}
            if fp8:
                timed["identity"] = id_pairs[i]
            step(timed)
        torch.cuda.synchronize()
        dom_us = statistics.fmean(elapsed_us(p_) for p_ in dom_pairs)
        id_us = statistics.fmean(elapsed_us(p_) for p_ in id_pairs) if fp8 else 0.0
        return dom_us, id_us

    def timed_pass(cold, id_us):
        """K steps with events only at the two ends.  Warm: back to back.
        Cold: each step after a scrub; the K scrubs timed alone (same events)
        are subtracted.  The fp8 identity expert (not part of the path) is
        subtracted at its mean duration.  Returns (ms per step, wall ms per step)."""
        if not cold:
            us, wall = region_us(step, args.steps)
        else:
            def scrub_step():
                scrub()
                step()
            us_all, wall = region_us(scrub_step, args.steps)
            us_scrub, _ = region_us(scrub, args.steps)
            us = us_all - us_scrub
        us -= args.steps * id_us
        return us / args.steps / 1e3, 1e3 * wall / args.steps

    dom_us, id_us = kernel_pass()
    passes = {"warm": timed_pass(False, id_us), "cold": timed_pass(True, id_us)}
    graph_info = False
    if args.graph:
        eager = passes
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()                                   # one eager step on the capture stream
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()

        def graph_pass(cold):
            """K graph replays between two events; cold: each after a scrub,
            the K scrubs timed alone subtracted."""
            if not cold:
                us, _ = region_us(graph.replay, args.steps)
            else:
                def scrub_replay():
                    scrub()
                    graph.replay()
                us_all, _ = region_us(scrub_replay, args.steps)
                us_scrub, _ = region_us(scrub, args.steps)
                us = us_all - us_scrub
            return (us - args.steps * id_us) / args.steps / 1e3
        gw, gc = graph_pass(False), graph_pass(True)
        passes = {"warm": (gw, eager["warm"][1]), "cold": (gc, eager["cold"][1])}
        graph_info = {"eager_warm_ms_per_step": round(eager["warm"][0], 5),
                      "eager_cold_ms_per_step": round(eager["cold"][0], 5)}
    st = ubep.ubep_get_device_status(b.ws)
    if st != ubep.OK:
        raise RuntimeError(f"{name}: device status after timing: {ubep.STATUS_NAMES.get(st, st)}")
    rc = b.rank_count.cpu().numpy()
    del b, scrub_buf
    return dict(name=name, w=w, sd=sd, fp8=fp8, gated=gated, moe=moe, order=order, calls=calls,
                per_call=per_call, dom=dom, dom_ms=dom_us / 1e3, passes=passes, graph=graph_info,
                ew_bytes=ew_bytes,
                nb=algorithmic_bytes(sd, fp8, gated, ew_bytes),
                skew=round(float(rc.max() / rc.mean()), 3))


def stream_ceilings(sd: dict, reps: int = 10) -> dict:
    """Sequential-stream rates in this run, sized like the step's kernels
    (ubep_stream_probe; reps launches back to back between two events, no
    event between them, median of 3 such passes): a read stream and a write
    stream of the receive rows' bytes, and the combine's and the dispatch's
    byte mixes (eight 16-byte vectors read per vector written, and the
    reverse)."""
    import torch

    import combine_top_route_amd as ubep
    n = sd["T"] * sd["H"] // 8                       # 16-byte vectors of one token-row array
    big = torch.empty(8 * n * 16, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    small = torch.empty(n * 16, dtype=torch.uint8, device="cuda")
    small.fill_(2)
    cases = {"read": (big, small, 8, 0), "write": (small, big, 0, 8),
             "combine_mix": (big, small, 8, 1), "dispatch_mix": (small, big, 1, 8)}
    out = {}
    stream = torch.cuda.current_stream()
    for key, (src, dst, fi, fo) in cases.items():
        ubep.ubep_stream_probe(src, dst, n, fi, fo, stream)
        passes = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(reps):
                ubep.ubep_stream_probe(src, dst, n, fi, fo, stream)
            e1.record(stream)
            passes.append((e0, e1))
        torch.cuda.synchronize()
        us = statistics.median(a.elapsed_time(b) * 1e3 / reps for a, b in passes)
        nbytes = 16 * n * (fi + fo)
        out[key] = {"bytes": nbytes, "us": round(us, 2), "GBs": round(nbytes / us / 1e3, 1)}
    del big, small
    return out


def summarize(m: dict, headline: str) -> dict:
    """The numbers of one measured workload: headline pass, the other pass,
    per-kernel rates, and the dominant kernel's roofline."""
    other = "warm" if headline == "cold" else "cold"
    nb, sd = m["nb"], m["sd"]
    ms = m["passes"][headline][0]
    wall_ms = m["passes"]["warm"][1]                 # host time per back-to-back step
    dom_ms = m["dom_ms"]
    gbs = nb["total"] / (ms * 1e-3) / 1e9
    dom = m["dom"]
    dom_bytes = nb["dispatch"] + nb["combine"] if dom in ("chunked", "sentinel") else nb[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = read_counters(dom, m["name"])
    kernels = {}
    for n_, us in m["per_call"].items():
        key = {"layout_dispatch": "dispatch"}.get(n_, n_)
        by = (nb["dispatch"] + nb["combine"] if n_ in ("chunked", "sentinel")
              else nb["layout"] + nb["dispatch"] if n_ == "layout_dispatch"
              else nb["gate"] + nb["layout"] if n_ == "gate_layout" else nb.get(key, 0))
        kernels[n_] = {"us": round(us, 2), "bytes": by,
                       "GBs": round(by / (us * 1e-6) / 1e9, 1) if by else None}
    o_ms = m["passes"][other][0]
    return {
        "value": round(gbs, 2),
        "ms_per_step": round(ms, 5),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(sd["T"] / (ms * 1e-3), 1),
        "bytes_per_step": nb["total"],
        "caches": ("cold: 512 MB read between steps" if headline == "cold"
                   else "warm: back-to-back steps"),
        "ms": {"step_mean": round(ms, 5),
               "dominant_kernel_mean": round(dom_ms, 5)},
        "kernels_calibration": kernels,
        "wall_ms_per_step": round(wall_ms, 5),
        other: {"ms_per_step": round(o_ms, 5),
                "value": round(nb["total"] / (o_ms * 1e-3) / 1e9, 2),
                "pct_of_hbm_peak": round(100.0 * nb["total"] / (o_ms * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 2),
                "caches": ("cold: 512 MB read between steps" if other == "cold"
                           else "warm: back-to-back steps")},
        "rank_skew_max_over_mean": m["skew"],
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "algorithmic_bytes": dom_bytes},
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="workload name (default: DeepSeek-V3 decode)")
    ap.add_argument("--mode", choices=["unfused", "chunked", "sentinel", "gated", "gate_layout",
                                       "fused", "moe"],
                    default="unfused",
                    help="gated: the step starts from router logits (ubep_gate, then unfused); "
                         "gate_layout: the same step with ubep_gate_layout (the gate's "
                         "selections feed the layout's counts), then dispatch and combine; "
                         "fused: ubep_layout_dispatch (one launch), then combine; "
                         "sentinel: layout, then ubep_dispatch_combine_sentinel (token-granular "
                         "readiness polled in the rows); moe: expert-grouped layout, dispatch, "
                         "a per-expert H x H linear map on the matrix cores (random bf16 "
                         "weights), combine")
    ap.add_argument("--order", choices=["rank", "expert"], default="rank",
                    help="receive order inside a rank's region: (token, slot) with ubep_layout, or "
                         "expert-grouped (expert, token, slot) with ubep_layout_grouped")
    ap.add_argument("--chunk-order", choices=["identity", "lpt", "both"], default="both",
                    help="chunk pipeline (--mode chunked): chunks in index order, in LPT order "
                         "computed on the device from the layout's counts, or both (LPT reported "
                         "beside the headline identity order)")
    ap.add_argument("--warm", action="store_true",
                    help="headline the warm pass (back-to-back steps); the default headline is "
                         "the cold-cache pass, the warm one is reported beside it")
    ap.add_argument("--no-companion", action="store_true",
                    help="skip the skewed (Zipf) twin of the DeepSeek-V3 decode workload")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of CPU-oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured in a HIP graph (no host launch cost); "
                         "the dominant kernel is still timed by its launches in eager steps")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run the plain 16-byte copy kernel on this many bytes (the "
                         "reference for scaling hardware traffic counters) and exit")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the R expert-parallel ranks are regions of one "
              "GPU's HBM and no multi-GPU path is built.", file=sys.stderr, flush=True)
        return 2

    import torch

    from workloads import DEFAULT_BENCH, make_config

    if args.copy_bytes:
        return copy_reference(args.copy_bytes, max(args.steps, 1))

    name = args.workload or DEFAULT_BENCH
    payload = make_config(name).recipe.payload if args.mode != "unfused" else None
    if args.mode in ("chunked", "sentinel", "moe", "fused") and payload == "fp8":
        print("the pipelined, fused and expert modes carry a bf16 payload only", file=sys.stderr)
        return 2
    if args.mode == "fused" and args.order == "expert":
        print("the fused launch computes the rank-order layout only", file=sys.stderr)
        return 2
    if args.mode != "chunked":
        args.chunk_order = "identity"
    torch.cuda.set_device(0)
    hev = HipEvents()
    headline = "warm" if args.warm else "cold"
    try:
        orders = ["identity", "lpt"] if args.chunk_order == "both" else [args.chunk_order]
        args.chunk_order = orders[0]
        m = measure(name, args, hev)
        extra = {}
        for o in orders[1:]:
            args.chunk_order = o
            extra[o] = measure(name, args, hev)
        args.chunk_order = orders[0]
        comp_name = None if args.no_companion else companion_of(name)
        comp = measure(comp_name, args, hev) if comp_name else None
    except RuntimeError as e:
        print(str(e), file=sys.stderr, flush=True)
        return 1
    finally:
        hev.close()
    ceilings = None if args.no_ceilings else stream_ceilings(m["sd"])

    sm = summarize(m, headline)
    w = m["w"]
    line = {
        "metric": METRIC,
        "value": sm["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sm["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3+bf16" if m["fp8"] else "bf16",
        "data": "synthetic",
        "config": {"workload": name, **m["sd"], "payload": w.recipe.payload, "mode": args.mode,
                   "order": m["order"],
                   **({"chunk_order": args.chunk_order} if args.mode == "chunked" else {}),
                   "caches": sm["caches"], "seed": w.recipe.seed},
        "graph": m["graph"],
        "timing": ("steps: HIP events (hipEventDisableSystemFence) only at the two ends of "
                   "K steps (each event record idles the GPU for about 4.5 us, so none sits "
                   "inside the region); cold: K x (512 MB read scrub + step) minus K scrubs "
                   "timed alone the same way; dominant kernel: mean over a separate pass of K "
                   "steps in which events its own launch records time it (hipExtLaunchKernel); "
                   "the fp8 identity expert, timed the same way, is subtracted from the steps; "
                   "per-kernel figures: median of 10 calibration steps, every kernel timed by "
                   "its launch"),
        **{k: v for k, v in sm.items() if k not in ("value", "ms_per_step")},
        "expert": ({"flops": 2 * m["sd"]["T"] * m["sd"]["k"] * m["sd"]["H"] ** 2,
                    "ms_calibration": round(m["per_call"]["expert"] / 1e3, 5),
                    "tflops": round(2 * m["sd"]["T"] * m["sd"]["k"] * m["sd"]["H"] ** 2
                                    / (m["per_call"]["expert"] * 1e-6) / 1e12, 1),
                    "mfma_bf16_peak_tflops": 2500.0,
                    "weight_bytes": m["ew_bytes"]} if m["moe"] else None),
    }
    for o, mo in extra.items():
        so = summarize(mo, headline)
        line[f"chunk_order_{o}"] = {k: so[k] for k in ("value", "ms_per_step", "pct_of_hbm_peak",
                                                       "tokens_per_s", "warm" if headline == "cold"
                                                       else "cold", "roofline")}
    if comp is not None:
        sc = summarize(comp, headline)
        line["zipf"] = {"workload": comp["name"], **{k: sc[k] for k in (
            "value", "ms_per_step", "pct_of_hbm_peak", "tokens_per_s", "caches", "ms",
            "warm" if headline == "cold" else "cold", "rank_skew_max_over_mean",
            "kernels_calibration", "roofline")}}
    if ceilings is not None:
        kc = sm["kernels_calibration"]
        rel = {}
        for kname, ck in (("combine", "combine_mix"), ("dispatch", "dispatch_mix")):
            if kname in kc and kc[kname]["GBs"]:
                rel[kname] = {"GBs": kc[kname]["GBs"],
                              "pct_of_hbm_peak": round(100.0 * kc[kname]["GBs"] / HBM_PEAK_GBS, 2),
                              f"pct_of_{ck}_ceiling": round(100.0 * kc[kname]["GBs"]
                                                            / ceilings[ck]["GBs"], 2)}
        if "combine" in rel:
            rel["combine"]["pct_of_read_ceiling"] = round(
                100.0 * kc["combine"]["GBs"] / ceilings["read"]["GBs"], 2)
        if "dispatch" in rel:
            rel["dispatch"]["pct_of_write_ceiling"] = round(
                100.0 * kc["dispatch"]["GBs"] / ceilings["write"]["GBs"], 2)
        line["stream_ceilings"] = {
            **ceilings,
            "note": ("sequential streams of the receive rows' size in this run (ubep_stream_probe, "
                     "one 16-byte vector per thread over the whole range; warm, 10 launches back "
                     "to back, median of 3 passes): read only, write only, and the combine's (8 "
                     "read : 1 written) and dispatch's (1 : 8) byte mixes"),
            "kernels": rel}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

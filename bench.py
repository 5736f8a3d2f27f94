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
Time comes from HIP events on the stream the library launches on: two at the
ends of the timed region (marker packets between kernels would add several
microseconds per step), and, for the dominant kernel, a pair that its own
launch records (ubep_time_next_launch).

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
    "layout": ["layout.hip", "layout_worker.h", "launch.h", "device_common.h", "plan.h"],
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


def cpu_baseline(w, reps: int) -> dict:
    """The CPU oracle (single-threaded C) on the same batch: layout + dispatch
    + combine, outputs preallocated, median of `reps` runs."""
    import numpy as np

    import oracle
    s = w.shape
    fp8 = w.recipe.payload == "fp8"
    rows = s.T * s.k
    recv = np.empty((rows, s.H), np.uint16) if not fp8 else None
    out = np.empty((s.T, s.H), np.uint16)
    times = []
    for _ in range(reps):
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
    med = statistics.median(times)
    nbytes = algorithmic_bytes(s.as_dict(), fp8)["total"]
    return {"value": round(nbytes / med / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"whole batch ({s.T} tokens) of the benchmarked workload, "
                      f"median of {reps} runs of layout+dispatch+combine, one thread",
            "seconds_per_step": round(med, 4), "tokens_per_s": round(s.T / med, 1),
            "host_cores_available": len(os.sched_getaffinity(0))}


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


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="workload name (default: DeepSeek-V3 decode)")
    ap.add_argument("--mode", choices=["unfused", "chunked", "sentinel", "gated", "fused", "moe"],
                    default="unfused",
                    help="gated: the step starts from router logits (ubep_gate, then unfused); "
                         "fused: ubep_layout_dispatch (one launch), then combine; "
                         "sentinel: layout, then ubep_dispatch_combine_sentinel (token-granular "
                         "readiness polled in the rows); moe: expert-grouped layout, dispatch, "
                         "a per-expert H x H linear map on the matrix cores (random bf16 "
                         "weights), combine")
    ap.add_argument("--order", choices=["rank", "expert"], default="rank",
                    help="receive order inside a rank's region: (token, slot) with ubep_layout, or "
                         "expert-grouped (expert, token, slot) with ubep_layout_grouped")
    ap.add_argument("--cold", action="store_true",
                    help="headline the cold-cache pass (the warm one is then reported beside it)")
    ap.add_argument("--cpu-reps", type=int, default=7)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    import combine_top_route_amd as ubep
    from combine_top_route_amd.buffers import alloc_buffers
    from workloads import DEFAULT_BENCH, make_config

    if args.copy_bytes:
        return copy_reference(args.copy_bytes, max(args.steps, 1))

    name = args.workload or DEFAULT_BENCH
    w = make_config(name)
    s = w.shape
    sd = s.as_dict()
    fp8 = w.recipe.payload == "fp8"
    dtype = ubep.FP8_E4M3 if fp8 else ubep.BF16
    if args.mode == "moe":
        args.order = "expert"
    if args.mode in ("chunked", "sentinel", "moe") and fp8:
        print("the pipelined kernels carry a bf16 payload only", file=sys.stderr)
        return 2
    if args.mode == "fused" and args.order == "expert":
        print("the fused launch computes the rank-order layout only", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    b = alloc_buffers(sd, dtype, "cuda", x_bits=w.x, topk_idx=w.topk_idx, topk_w=w.topk_w)
    stream = torch.cuda.current_stream()
    chunk_off = b.chunk_offset if s.C > 1 else None
    expert_off = torch.empty(s.E + 1, dtype=torch.int32, device="cuda")
    # cold-cache pass: reading 512 MB of unrelated data between steps evicts the
    # path's arrays from the 256 MB memory-side cache and the L2s and leaves
    # clean lines behind (a write scrub would leave dirty lines that the next
    # step pays to write back)
    scrub = torch.ones(512 << 20, dtype=torch.uint8, device="cuda").view(torch.int64)

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
        if fp8:
            print("the fused launch carries a bf16 payload only", file=sys.stderr)
            return 2
        calls = ["layout_dispatch", "combine"]
    gated = args.mode == "gated"
    if gated:
        from workloads import router_logits
        calls = ["gate"] + calls
        logits = torch.from_numpy(router_logits(w.recipe)).cuda()
        grouped = w.recipe.routing == "group_zipf"
        gate_args = dict(groups=w.recipe.n_groups if grouped else 1,
                         keep_groups=w.recipe.topk_groups if grouped else 1,
                         norm=ubep.GATE_SIGMOID if w.recipe.weights == "sigmoid" else ubep.GATE_SOFTMAX)

    def call(name):
        stream = torch.cuda.current_stream()    # the capture stream while a graph records
        if name == "gate":
            ubep.ubep_gate(s.T, s.E, s.k, logits, b.topk_idx, b.topk_w, stream=stream, **gate_args)
        elif name == "layout" and args.order == "expert":
            ubep.ubep_layout_grouped(sd, b.topk_idx, b.pos, b.expert_count, expert_off, b.rank_count,
                                     b.recv_offset, b.send_offset, chunk_off, None, b.ws, stream)
        elif name == "layout":
            ubep.ubep_layout(sd, b.topk_idx, b.pos, b.expert_count, b.rank_count, b.recv_offset,
                             b.send_offset, chunk_off, None, b.ws, stream)
        elif name == "layout_dispatch":
            ubep.ubep_layout_dispatch(sd, b.topk_idx, b.x, b.pos, b.expert_count, b.rank_count,
                                      b.recv_offset, b.send_offset, chunk_off, None, b.recv, b.ws,
                                      stream)
        elif name == "expert":
            ubep.ubep_expert_linear(sd, s.H, expert_off, b.recv, wpacked, yexp, b.ws, stream)
        elif name == "sentinel":
            ubep.ubep_dispatch_combine_sentinel(sd, b.x, b.pos, b.topk_w, b.recv, b.out, b.ws,
                                                stream=stream)
        elif name == "chunked":
            ubep.ubep_dispatch_combine_chunked(sd, b.x, b.pos, b.topk_w, b.recv, b.out, None,
                                               b.ws, stream=stream)
        elif name == "dispatch":
            ubep.ubep_dispatch(sd, dtype, b.x, b.pos, b.recv, b.recv_scale, b.ws, stream)
        else:
            ubep.ubep_combine(sd, yexp if moe else b.y, b.pos, b.topk_w, b.out, b.ws, stream)

    hev = HipEvents()

    def step(timed=None):
        """One step.  `timed` maps a call name (or 'identity', the fp8 identity
        expert between dispatch and combine) to a (start, stop) event pair that
        the call's kernel launch records at its own start and end."""
        for name in calls:
            if timed and name in timed:
                ubep.ubep_time_next_launch(*timed[name])
            call(name)
            if name == "dispatch" and fp8:
                if timed and "identity" in timed:
                    ubep.ubep_time_next_launch(*timed["identity"])
                ubep.ubep_identity_expert_fp8(s.T * s.k, s.H, b.recv, b.recv_scale, b.y,
                                              torch.cuda.current_stream())

    def pairs(n):
        return [hev.pair() for _ in range(n)]

    elapsed_us = hev.elapsed_us

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = ubep.ubep_get_device_status(b.ws)
    if st != ubep.OK:
        print(f"device status after warm-up: {ubep.STATUS_NAMES.get(st, st)}", file=sys.stderr)
        return 1

    ew_bytes = -1
    if moe:    # weights of the experts that received rows are what the expert must read
        ew_bytes = int((b.expert_count > 0).sum().item()) * s.H * s.H * 2

    # untimed calibration: every kernel timed by its own launch, to find the
    # dominant one
    cal = [{n: p for n, p in zip(calls, pairs(len(calls)))} for _ in range(5)]
    torch.cuda.synchronize()
    for c in cal:
        step(c)
    torch.cuda.synchronize()
    per_call = {n: statistics.fmean(elapsed_us(c[n]) for c in cal) for n in calls}
    dom = max((n for n in calls if n not in ("layout", "gate")), key=lambda n: per_call[n])
    if dom == "layout_dispatch":
        dom = "combine"      # the fused launch also holds the layout's latency chain

    def timed_pass(cold):
        """K steps.  Warm: back to back between two events.  Cold: a read scrub
        before each step, outside per-step events.  The dominant kernel and the
        fp8 identity expert (subtracted) are timed by their own launches.
        Returns (ms per step, dominant kernel ms, wall ms per step)."""
        dom_pairs = pairs(args.steps)
        id_pairs = pairs(args.steps) if fp8 else None
        step_pairs = pairs(args.steps) if cold else None
        region = hev.pair()
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        hev.record(region[0], stream)
        for i in range(args.steps):
            timed = {dom: dom_pairs[i]}
            if fp8:
                timed["identity"] = id_pairs[i]
            if cold:
                scrub.sum()
                hev.record(step_pairs[i][0], stream)
            step(timed)
            if cold:
                hev.record(step_pairs[i][1], stream)
        hev.record(region[1], stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        per_step = [elapsed_us(p_) for p_ in step_pairs] if cold else None
        total_us = sum(per_step) if cold else elapsed_us(region)
        if fp8:
            id_us = [elapsed_us(p_) for p_ in id_pairs]
            total_us -= sum(id_us)
            if cold:
                per_step = [a_ - b_ for a_, b_ in zip(per_step, id_us)]
        return (total_us / args.steps / 1e3,
                statistics.fmean(elapsed_us(p_) for p_ in dom_pairs) / 1e3,
                1e3 * wall / args.steps, per_step)

    def copy_ceiling(nbytes):
        """A plain 16-byte copy moving about as many bytes as one step (half
        read, half written; at most 2 GiB each way), in this run: the
        achievable streaming rate that the step is compared with."""
        n = min(nbytes // 2, 2 << 30) // 16 * 16
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        reps = 10
        ubep.ubep_copy(src, dst, n, stream)
        reg = hev.pair()
        torch.cuda.synchronize()
        hev.record(reg[0], stream)
        for _ in range(reps):
            ubep.ubep_copy(src, dst, n, stream)
        hev.record(reg[1], stream)
        torch.cuda.synchronize()
        us = elapsed_us(reg) / reps
        del src, dst
        return {"bytes_moved": 2 * n, "us": round(us, 2), "GBs": round(2 * n / us / 1e3, 1)}

    passes = {"warm": timed_pass(False), "cold": timed_pass(True)}
    eager = passes
    if args.graph:
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
            """K graph replays: warm between two events, cold with a read scrub
            before each replay outside per-replay events."""
            pairs_ = pairs(args.steps) if cold else None
            region = hev.pair()
            torch.cuda.synchronize()
            hev.record(region[0], stream)
            for i in range(args.steps):
                if cold:
                    scrub.sum()
                    hev.record(pairs_[i][0], stream)
                graph.replay()
                if cold:
                    hev.record(pairs_[i][1], stream)
            hev.record(region[1], stream)
            torch.cuda.synchronize()
            per = [elapsed_us(p_) for p_ in pairs_] if cold else None
            total = sum(per) if cold else elapsed_us(region)
            return total / args.steps / 1e3, per
        (gw, _), (gc, gc_steps) = graph_pass(False), graph_pass(True)
        passes = {"warm": (gw, eager["warm"][1], eager["warm"][2], None),
                  "cold": (gc, eager["cold"][1], eager["cold"][2], gc_steps)}
    ceiling = copy_ceiling(algorithmic_bytes(sd, fp8, gated, ew_bytes)["total"])
    hev.close()
    st = ubep.ubep_get_device_status(b.ws)
    if st != ubep.OK:
        print(f"device status after timing: {ubep.STATUS_NAMES.get(st, st)}", file=sys.stderr)
        return 1
    head, other = ("cold", "warm") if args.cold else ("warm", "cold")
    ms, dom_ms, wall_ms, _ = passes[head]
    cold_steps = sorted(passes["cold"][3])

    def pct(q):
        return round(cold_steps[min(len(cold_steps) - 1, int(q * len(cold_steps)))] / 1e3, 5)

    nb = algorithmic_bytes(sd, fp8, gated, ew_bytes)
    gbs = nb["total"] / (ms * 1e-3) / 1e9
    dom_bytes = nb["dispatch"] + nb["combine"] if dom in ("chunked", "sentinel") else nb[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = read_counters(dom, name)

    rc = b.rank_count.cpu().numpy()
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3+bf16" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": name, **sd, "payload": w.recipe.payload, "mode": args.mode,
                   "order": args.order,
                   "caches": ("cold: 512 MB read between steps" if args.cold
                              else "warm: back-to-back steps"),
                   "seed": w.recipe.seed},
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "copy_ceiling": ceiling,
        "pct_of_copy_ceiling": round(100.0 * gbs / ceiling["GBs"], 2),
        "tokens_per_s": round(s.T / (ms * 1e-3), 1),
        "bytes_per_step": nb["total"],
        "ms": {"step_mean": round(ms, 5),
               "cold_step_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
               "dominant_kernel_mean": round(dom_ms, 5),
               "per_call_calibration": {n: round(v / 1e3, 5) for n, v in per_call.items()}},
        "timing": ("HIP events (hipEventDisableSystemFence) at the two ends of the timed "
                   "region (cold pass: around each step, the cache scrub outside); the "
                   "dominant kernel (and the fp8 identity expert, subtracted) timed by "
                   "events its own launch records (hipExtLaunchKernel)"),
        "wall_ms_per_step": round(wall_ms, 5),
        "graph": ({"eager_warm_ms_per_step": round(eager["warm"][0], 5),
                   "eager_cold_ms_per_step": round(eager["cold"][0], 5)} if args.graph else False),
        other: {"ms_per_step": round(passes[other][0], 5),
                "value": round(nb["total"] / (passes[other][0] * 1e-3) / 1e9, 2),
                "pct_of_hbm_peak": round(100.0 * nb["total"] / (passes[other][0] * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 2),
                "dominant_kernel_mean_ms": round(passes[other][1], 5),
                "caches": ("cold: 512 MB read between steps" if other == "cold"
                           else "warm: back-to-back steps")},
        "rank_skew_max_over_mean": round(float(rc.max() / rc.mean()), 3),
        "expert": ({"flops": 2 * s.T * s.k * s.H * s.H,
                    "ms_calibration": round(per_call["expert"] / 1e3, 5),
                    "tflops": round(2 * s.T * s.k * s.H * s.H / (per_call["expert"] * 1e-6) / 1e12, 1),
                    "mfma_bf16_peak_tflops": 2500.0,
                    "weight_bytes": ew_bytes} if moe else None),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "algorithmic_bytes": dom_bytes},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_reps)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

// C ABI (include/ubep.h): host-side validation, launch planning and status
// handling.  Every argument check happens before anything is enqueued.
#include <stdint.h>

#include "launch.h"
#include "ubep.h"
#include "ubep_testing.h"

namespace ubep {

static int bits_for(int64_t n) {   // bits needed to hold the values 0..n-1
    int b = 0;
    while (((int64_t)1 << b) < n) ++b;
    return b;
}

static int64_t gcd64(int64_t a, int64_t b) {
    while (b != 0) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// A layout tile holds whole tokens and never straddles a source-rank or chunk
// boundary: its token count divides gcd(T/R, T/C).  Take the largest such
// divisor with at most kTileRowsMax rows; with `spread`, where that leaves
// fewer than kTileTarget tiles, the largest with at most T / kTileTarget
// tokens instead, if that one still has kTileRowsMin rows and makes at most
// 2 * kTileTarget tiles.  The workspace is laid out for the spread tiling,
// which has at least as many tiles, so calls with either tiling share one
// workspace (ws_spread false: for the tiling in use only).
static int64_t largest_divisor_upto(int64_t g, int64_t cap) {
    for (int64_t d = g < cap ? g : cap; d > 1; --d)
        if (g % d == 0) return d;
    return 1;
}

void make_plan(const ubep_shape& s, Plan* p, int order, bool spread, bool ws_spread) {
    p->T = s.T;
    p->H = s.H;
    p->E = s.E;
    p->k = s.k;
    p->R = s.R;
    p->C = s.C;
    p->rows = s.T * s.k;
    p->epr = s.E / s.R;
    // floor(e / epr) == umulhi(e, ceil(2^32 / epr)) whenever e * epr < 2^32
    // (here e < E <= 8192 and epr <= 8192)
    p->epr_magic = p->epr == 1 ? 0u : (uint32_t)((((uint64_t)1 << 32) + p->epr - 1) / p->epr);
    p->tps = s.T / s.R;
    p->tpc = s.T / s.C;
    const int64_t g = gcd64(p->tps, p->tpc);
    const int64_t tt_whole = largest_divisor_upto(g, kTileRowsMax / s.k);
    const int64_t cap = s.T / kTileTarget < kTileRowsMax / s.k ? s.T / kTileTarget : kTileRowsMax / s.k;
    int64_t tt_spread = largest_divisor_upto(g, cap);
    // keep the largest tiles when the divisors of g allow no spread tiling
    // of at least kTileRowsMin rows and at most 2 * kTileTarget tiles
    if (tt_spread * s.k < kTileRowsMin || s.T / tt_spread > 2 * kTileTarget) tt_spread = tt_whole;
    const int64_t tt = spread ? tt_spread : tt_whole;
    p->tile_tokens = tt;
    p->tile_rows = tt * s.k;
    p->n_tiles = s.T / tt;
    const int64_t n_ws = s.T / (ws_spread ? tt_spread : tt);   // tiles the workspace is laid out for
    p->n_tiles_ws = n_ws;
    p->dbits = bits_for(s.R);
    p->ebits = bits_for(s.E);
    p->slots = s.R + s.E;
    p->order = order;
    p->K = order ? s.E : s.R;
    p->key_magic = order ? 0u : p->epr_magic;
    p->kbits = order ? p->ebits : p->dbits;
    p->kcol = order ? s.R : 0;
    p->gather = (p->n_tiles * p->K <= kGatherMaxWords && p->n_tiles <= kGatherMaxTiles) ? 1 : 0;
    // per-tile key arrays are sized for the larger key count (E >= R), so one
    // workspace serves both orders
    size_t off = align_up(kHdrBytes, 256);
    p->off_state = off;
    off = align_up(off + (size_t)n_ws * p->slots * 8, 256);
    p->off_excl = off;
    off = align_up(off + (size_t)n_ws * s.E * 4, 256);
    p->off_wbase = off;
    off = align_up(off + (size_t)n_ws * kLayoutWaves * s.E * 4, 256);
    p->off_flags = off;
    off = align_up(off + (size_t)s.C * kFlagStride * 4, 256);
    p->off_order = off;
    off = align_up(off + (size_t)s.C * 4, 256);
    p->off_gate_rank = off;
    off = align_up(off + (size_t)n_ws * s.R * 4, 256);
    p->off_gate_expert = off;
    off = align_up(off + (size_t)n_ws * s.E * 4, 256);
    p->ws_bytes = off;
}

}  // namespace ubep

using namespace ubep;

namespace {

constexpr int64_t kMaxTiles = 1 << 16;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

ubep_status hip_status(hipError_t e) { return e == hipSuccess ? UBEP_OK : UBEP_ERR_HIP; }

// Shape check plus the tile-count limit of the layout's workspace.
ubep_status check_and_plan(const ubep_shape* s, int dtype, Plan* p, int order = 0, bool spread = true) {
    const ubep_status st = ubep_check_shape(s, dtype);
    if (st != UBEP_OK) return st;
    make_plan(*s, p, order, spread);
    if (p->n_tiles_ws > kMaxTiles || p->n_tiles_ws * p->slots > kMaxStateWords) return UBEP_ERR_UNSUPPORTED;
    return UBEP_OK;
}

ubep_status spin_ticks_for(uint64_t ns, uint64_t* ticks) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return UBEP_ERR_HIP;
    DeviceInfo di;
    if (device_info(dev, &di) != hipSuccess) return UBEP_ERR_HIP;
    if (ns == 0) ns = 1000000000ull;
    const uint64_t t = ns / 1000ull * (uint64_t)di.wall_clock_khz / 1000ull;
    *ticks = t > 0 ? t : 1;
    return UBEP_OK;
}

}  // namespace

extern "C" {

int ubep_abi_version(void) { return UBEP_ABI_VERSION; }

const char* ubep_status_str(ubep_status s) {
    switch (s) {
        case UBEP_OK: return "ok";
        case UBEP_ERR_INVALID_ARG: return "invalid argument";
        case UBEP_ERR_UNSUPPORTED: return "unsupported shape";
        case UBEP_ERR_BAD_EXPERT_ID: return "expert id outside [0, E)";
        case UBEP_ERR_TIMEOUT: return "ready-flag wait timed out";
        case UBEP_ERR_HIP: return "HIP runtime error";
        case UBEP_ERR_BAD_POSITION: return "position outside [0, T*k)";
        case UBEP_ERR_WORKSPACE: return "workspace counters inconsistent; re-initialize the workspace";
        case UBEP_ERR_SENTINEL_DATA: return "input row holds the readiness sentinel word";
    }
    return "unknown status";
}

ubep_status ubep_check_shape(const ubep_shape* s, int dtype) {
    if (s == nullptr) return UBEP_ERR_INVALID_ARG;
    if (dtype != UBEP_BF16 && dtype != UBEP_FP8_E4M3) return UBEP_ERR_INVALID_ARG;
    if (s->T <= 0 || s->H <= 0 || s->E <= 0 || s->k <= 0 || s->R <= 0 || s->C <= 0)
        return UBEP_ERR_INVALID_ARG;
    if (s->k > s->E) return UBEP_ERR_INVALID_ARG;
    if (s->E % s->R != 0 || s->T % s->R != 0 || s->T % s->C != 0) return UBEP_ERR_INVALID_ARG;
    if (s->H % 8 != 0) return UBEP_ERR_INVALID_ARG;
    if (dtype == UBEP_FP8_E4M3 && s->H % 128 != 0) return UBEP_ERR_INVALID_ARG;
    if (s->T >= ((int64_t)1 << 30) || s->T * (int64_t)s->k >= ((int64_t)1 << 30))
        return UBEP_ERR_INVALID_ARG;
    if (s->H >= ((int64_t)1 << 30)) return UBEP_ERR_UNSUPPORTED;
    if (s->k > kMaxK || s->R > kMaxR || s->E > kMaxE || s->C > kMaxC) return UBEP_ERR_UNSUPPORTED;
    return UBEP_OK;
}

size_t ubep_workspace_bytes(const ubep_shape* s) {
    Plan p;
    if (check_and_plan(s, UBEP_BF16, &p) != UBEP_OK) return 0;
    return p.ws_bytes;
}

ubep_status ubep_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
    if (ws == nullptr || ws_bytes < kHdrBytes || ws_bytes % 4 != 0 || !aligned(ws, 256))
        return UBEP_ERR_INVALID_ARG;
    return hip_status(launch_fill_zero(ws, ws_bytes, stream));
}

ubep_status ubep_layout(const ubep_shape* s, const int32_t* topk_idx, int32_t* pos,
                        int32_t* expert_count, int32_t* rank_count, int32_t* recv_offset,
                        int32_t* send_offset, int32_t* chunk_offset, int32_t* recv_src, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
    Plan p;
    const ubep_status st = check_and_plan(s, UBEP_BF16, &p);
    if (st != UBEP_OK) return st;
    if (!topk_idx || !pos || !expert_count || !rank_count || !recv_offset || !send_offset || !ws)
        return UBEP_ERR_INVALID_ARG;
    if (ws_bytes < p.ws_bytes || !aligned(ws, 256)) return UBEP_ERR_INVALID_ARG;
    uint64_t ticks;
    const ubep_status ts = spin_ticks_for(0, &ticks);
    if (ts != UBEP_OK) return ts;
    return hip_status(launch_layout(p, topk_idx, pos, expert_count, nullptr, rank_count,
                                    recv_offset, send_offset, chunk_offset, recv_src, ws, ticks,
                                    stream));
}

ubep_status ubep_layout_noalloc(const ubep_shape* s, const int32_t* topk_idx, int32_t* pos,
                                int32_t* expert_count, int32_t* rank_count, int32_t* recv_offset,
                                int32_t* send_offset, int32_t* chunk_offset, int32_t* recv_src,
                                uint32_t* status, int reset, hipStream_t stream) {
    Plan p;
    const ubep_status st = check_and_plan(s, UBEP_BF16, &p);
    if (st != UBEP_OK) return st;
    if (!topk_idx || !pos || !expert_count || !rank_count || !recv_offset || !send_offset || !status)
        return UBEP_ERR_INVALID_ARG;
    if (!aligned(status, 4)) return UBEP_ERR_INVALID_ARG;
    if (p.ws_bytes > kScratchBytes) {
        // the spread tiling's workspace does not fit the array: the largest
        // tiles, with a workspace laid out for them alone (the array serves
        // only this entry point)
        make_plan(*s, &p, 0, false, false);
        if (p.ws_bytes > kScratchBytes) return UBEP_ERR_UNSUPPORTED;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return UBEP_ERR_HIP;
    void* ws = nullptr;
    bool first_use = false;
    if (layout_scratch(dev, &ws, &first_use) != hipSuccess) return UBEP_ERR_HIP;
    uint64_t ticks;
    const ubep_status ts = spin_ticks_for(0, &ticks);
    if (ts != UBEP_OK) return ts;
    // the array starts cleared on its first use on this device, and again
    // whenever the caller asks (after a call that reported a time-out)
    if (first_use || reset != 0) {
        const hipError_t e = launch_fill_zero(ws, first_use ? kScratchBytes : p.ws_bytes, stream);
        if (e != hipSuccess) return UBEP_ERR_HIP;
    }
    return hip_status(launch_layout(p, topk_idx, pos, expert_count, nullptr, rank_count,
                                    recv_offset, send_offset, chunk_offset, recv_src, ws, ticks,
                                    stream, status));
}

ubep_status ubep_layout_grouped(const ubep_shape* s, const int32_t* topk_idx, int32_t* pos,
                                int32_t* expert_count, int32_t* expert_offset, int32_t* rank_count,
                                int32_t* recv_offset, int32_t* send_offset, int32_t* chunk_offset,
                                int32_t* recv_src, void* ws, size_t ws_bytes, hipStream_t stream) {
    Plan p;
    const ubep_status st = check_and_plan(s, UBEP_BF16, &p, 1);
    if (st != UBEP_OK) return st;
    if (!layout_lds_fits(p)) return UBEP_ERR_UNSUPPORTED;
    if (!topk_idx || !pos || !expert_count || !expert_offset || !rank_count || !recv_offset ||
        !send_offset || !ws)
        return UBEP_ERR_INVALID_ARG;
    if (ws_bytes < p.ws_bytes || !aligned(ws, 256)) return UBEP_ERR_INVALID_ARG;
    uint64_t ticks;
    const ubep_status ts = spin_ticks_for(0, &ticks);
    if (ts != UBEP_OK) return ts;
    return hip_status(launch_layout(p, topk_idx, pos, expert_count, expert_offset, rank_count,
                                    recv_offset, send_offset, chunk_offset, recv_src, ws, ticks,
                                    stream));
}

ubep_status ubep_layout_dispatch(const ubep_shape* s, const int32_t* topk_idx, const void* x,
                                 int32_t* pos, int32_t* expert_count, int32_t* rank_count,
                                 int32_t* recv_offset, int32_t* send_offset, int32_t* chunk_offset,
                                 int32_t* recv_src, void* recv, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
    Plan p;
    // the largest tiles, so the fewest layout workgroups: with the spread
    // tiling this kernel was slower on a 4096-token decode step
    const ubep_status st = check_and_plan(s, UBEP_BF16, &p, 0, false);
    if (st != UBEP_OK) return st;
    if (!topk_idx || !x || !pos || !expert_count || !rank_count || !recv_offset || !send_offset ||
        !recv || !ws)
        return UBEP_ERR_INVALID_ARG;
    if (ws_bytes < p.ws_bytes || !aligned(ws, 256)) return UBEP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv, 16)) return UBEP_ERR_INVALID_ARG;
    uint64_t ticks;
    const ubep_status ts = spin_ticks_for(0, &ticks);
    if (ts != UBEP_OK) return ts;
    return hip_status(launch_layout_dispatch(p, topk_idx, x, pos, expert_count, rank_count,
                                             recv_offset, send_offset, chunk_offset, recv_src, recv,
                                             ws, ticks, stream));
}

static ubep_status check_gate(const ubep_gate_shape* g, const float* logits, const int32_t* topk_idx,
                              const float* topk_w) {
    if (g == nullptr || !logits || !topk_idx || !topk_w) return UBEP_ERR_INVALID_ARG;
    if (g->T <= 0 || g->E <= 0 || g->k <= 0 || g->groups <= 0 || g->keep_groups <= 0)
        return UBEP_ERR_INVALID_ARG;
    if (g->E % g->groups != 0 || g->keep_groups > g->groups) return UBEP_ERR_INVALID_ARG;
    if ((int64_t)g->k > (int64_t)g->keep_groups * (g->E / g->groups)) return UBEP_ERR_INVALID_ARG;
    if (g->norm != UBEP_GATE_SOFTMAX && g->norm != UBEP_GATE_SIGMOID) return UBEP_ERR_INVALID_ARG;
    if (g->E > kGateMaxE || g->k > kMaxK || g->groups > kGateMaxGroups) return UBEP_ERR_UNSUPPORTED;
    if (g->T * (int64_t)g->k >= ((int64_t)1 << 31) || g->T * (int64_t)g->E >= ((int64_t)1 << 40))
        return UBEP_ERR_UNSUPPORTED;
    if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4)) return UBEP_ERR_INVALID_ARG;
    return UBEP_OK;
}

ubep_status ubep_gate(const ubep_gate_shape* g, const float* logits, int32_t* topk_idx,
                      float* topk_w, hipStream_t stream) {
    const ubep_status st = check_gate(g, logits, topk_idx, topk_w);
    if (st != UBEP_OK) return st;
    return hip_status(launch_gate(*g, logits, topk_idx, topk_w, stream));
}

ubep_status ubep_gate_layout(const ubep_gate_shape* g, const ubep_shape* s, const float* logits,
                             int32_t* topk_idx, float* topk_w, int32_t* pos, int32_t* expert_count,
                             int32_t* rank_count, int32_t* recv_offset, int32_t* send_offset,
                             int32_t* chunk_offset, int32_t* recv_src, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
    ubep_status st = check_gate(g, logits, topk_idx, topk_w);
    if (st != UBEP_OK) return st;
    Plan p;
    // the largest tiles: the per-tile counts that the gate writes, and that
    // the counted layout's last workgroup clears, grow with the tile count
    st = check_and_plan(s, UBEP_BF16, &p, 0, false);
    if (st != UBEP_OK) return st;
    if (g->T != s->T || g->E != s->E || g->k != s->k) return UBEP_ERR_INVALID_ARG;
    if (!pos || !expert_count || !rank_count || !recv_offset || !send_offset || !ws)
        return UBEP_ERR_INVALID_ARG;
    if (ws_bytes < p.ws_bytes || !aligned(ws, 256)) return UBEP_ERR_INVALID_ARG;
    if (!gate_counts_fit(*g, logits, p.tile_tokens) || !layout_from_counts_fits(p)) {
        // shapes outside the counting kernels: the same results from two calls
        const hipError_t e = launch_gate(*g, logits, topk_idx, topk_w, stream);
        if (e != hipSuccess) return UBEP_ERR_HIP;
        uint64_t ticks;
        const ubep_status ts = spin_ticks_for(0, &ticks);
        if (ts != UBEP_OK) return ts;
        return hip_status(launch_layout(p, topk_idx, pos, expert_count, nullptr, rank_count,
                                        recv_offset, send_offset, chunk_offset, recv_src, ws, ticks,
                                        stream));
    }
    char* base = static_cast<char*>(ws);
    GateCountArgs c;
    c.rank_cnt = reinterpret_cast<int32_t*>(base + p.off_gate_rank);
    c.expert_cnt = reinterpret_cast<int32_t*>(base + p.off_gate_expert);
    c.tile_tokens = p.tile_tokens;
    c.R = p.R;
    c.epr_magic = p.epr_magic;
    const hipError_t e = launch_gate_counting(*g, logits, topk_idx, topk_w, &c, stream);
    if (e != hipSuccess) return UBEP_ERR_HIP;
    return hip_status(launch_layout_from_counts(p, topk_idx, pos, expert_count, rank_count,
                                                recv_offset, send_offset, chunk_offset, recv_src,
                                                ws, stream));
}

ubep_status ubep_dispatch(const ubep_shape* s, int dtype, const void* x, const int32_t* pos,
                          void* recv, float* recv_scale, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
    Plan p;
    const ubep_status st = check_and_plan(s, dtype, &p);
    if (st != UBEP_OK) return st;
    if (!x || !pos || !recv || !ws || ws_bytes < kHdrBytes) return UBEP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv, 16) || !aligned(ws, 256)) return UBEP_ERR_INVALID_ARG;
    uint32_t* status = static_cast<uint32_t*>(ws) + kHdrStatus;
    if (dtype == UBEP_BF16) {
        if (recv_scale != nullptr) return UBEP_ERR_INVALID_ARG;
        return hip_status(launch_dispatch_bf16(p, x, pos, recv, status, stream));
    }
    if (recv_scale == nullptr || !aligned(recv_scale, 4)) return UBEP_ERR_INVALID_ARG;
    return hip_status(launch_dispatch_fp8(p, x, pos, recv, recv_scale, status, stream));
}

ubep_status ubep_combine(const ubep_shape* s, const void* y, const int32_t* pos,
                         const float* topk_w, void* out, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
    Plan p;
    const ubep_status st = check_and_plan(s, UBEP_BF16, &p);
    if (st != UBEP_OK) return st;
    if (!y || !pos || !topk_w || !out || !ws || ws_bytes < kHdrBytes) return UBEP_ERR_INVALID_ARG;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(ws, 256)) return UBEP_ERR_INVALID_ARG;
    uint32_t* status = static_cast<uint32_t*>(ws) + kHdrStatus;
    return hip_status(launch_combine(p, y, pos, topk_w, out, status, stream));
}

ubep_status ubep_chunk_order_lpt(const ubep_shape* s, const int32_t* chunk_offset,
                                 const int32_t* rank_count, int32_t* order, hipStream_t stream) {
    Plan p;
    const ubep_status st = check_and_plan(s, UBEP_BF16, &p);
    if (st != UBEP_OK) return st;
    if (!rank_count || !order || (p.C > 1 && !chunk_offset)) return UBEP_ERR_INVALID_ARG;
    if (!aligned(rank_count, 4) || !aligned(order, 4) || (chunk_offset && !aligned(chunk_offset, 4)))
        return UBEP_ERR_INVALID_ARG;
    return hip_status(launch_chunk_lpt(p, chunk_offset, rank_count, order, stream));
}

ubep_status ubep_dispatch_combine_chunked(const ubep_shape* s, const void* x, const int32_t* pos,
                                          const float* topk_w, void* recv, void* out,
                                          const int32_t* chunk_order, const int32_t* chunk_offset,
                                          const int32_t* rank_count, uint64_t spin_limit_ns,
                                          uint32_t debug_flags, void* ws, size_t ws_bytes,
                                          hipStream_t stream) {
    Plan p;
    const ubep_status st = check_and_plan(s, UBEP_BF16, &p);
    if (st != UBEP_OK) return st;
    if (!x || !pos || !topk_w || !recv || !out || !ws) return UBEP_ERR_INVALID_ARG;
    // LPT policy: both layout outputs given (chunk_offset may be null for C = 1), no host order
    const bool lpt = rank_count != nullptr;
    if (lpt && (chunk_order != nullptr || (p.C > 1 && chunk_offset == nullptr)))
        return UBEP_ERR_INVALID_ARG;
    if (!lpt && chunk_offset != nullptr) return UBEP_ERR_INVALID_ARG;
    if (lpt && (!aligned(rank_count, 4) || (chunk_offset && !aligned(chunk_offset, 4))))
        return UBEP_ERR_INVALID_ARG;
    if (ws_bytes < p.ws_bytes || !aligned(ws, 256)) return UBEP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv, 16) || !aligned(out, 16)) return UBEP_ERR_INVALID_ARG;
    if (debug_flags & ~3u) return UBEP_ERR_INVALID_ARG;
    if (chunk_order != nullptr) {
        bool seen[kMaxC] = {};
        for (int32_t i = 0; i < p.C; ++i) {
            const int32_t c = chunk_order[i];
            if (c < 0 || c >= p.C || seen[c]) return UBEP_ERR_INVALID_ARG;
            seen[c] = true;
        }
    }
    uint64_t ticks;
    const ubep_status ts = spin_ticks_for(spin_limit_ns, &ticks);
    if (ts != UBEP_OK) return ts;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return UBEP_ERR_HIP;
    int32_t* dev_order = nullptr;
    if (lpt) {
        // the order kernel leaves a pending timing pair to the pipeline kernel
        const LaunchEvents ev = take_launch_events();
        dev_order = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + p.off_order);
        const hipError_t e = launch_chunk_lpt(p, chunk_offset, rank_count, dev_order, stream);
        set_launch_events(ev.start, ev.stop);
        if (e != hipSuccess) return UBEP_ERR_HIP;
    }
    return hip_status(launch_chunked(p, x, pos, topk_w, recv, out, chunk_order, dev_order, ticks,
                                     debug_flags, ws, dev, stream));
}

ubep_status ubep_dispatch_combine_sentinel(const ubep_shape* s, const void* x, const int32_t* pos,
                                           const float* topk_w, void* recv, void* out,
                                           uint64_t spin_limit_ns, uint32_t debug_flags, void* ws,
                                           size_t ws_bytes, hipStream_t stream) {
    Plan p;
    const ubep_status st = check_and_plan(s, UBEP_BF16, &p);
    if (st != UBEP_OK) return st;
    if (!x || !pos || !topk_w || !recv || !out || !ws || ws_bytes < kHdrBytes) return UBEP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv, 16) || !aligned(out, 16) || !aligned(ws, 256))
        return UBEP_ERR_INVALID_ARG;
    if (debug_flags & ~3u) return UBEP_ERR_INVALID_ARG;
    uint64_t ticks;
    const ubep_status ts = spin_ticks_for(spin_limit_ns, &ticks);
    if (ts != UBEP_OK) return ts;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return UBEP_ERR_HIP;
    return hip_status(launch_sentinel_pipeline(p, x, pos, topk_w, recv, out, ticks, debug_flags, ws,
                                               dev, stream));
}

ubep_status ubep_recv_sentinel_init(void* recv, int64_t rows, int64_t H, hipStream_t stream) {
    if (!recv || rows < 0 || H <= 0 || H % 8 != 0 || !aligned(recv, 16)) return UBEP_ERR_INVALID_ARG;
    if (rows == 0) return UBEP_OK;
    if (rows >= ((int64_t)1 << 40)) return UBEP_ERR_UNSUPPORTED;
    return hip_status(launch_sentinel_fill(recv, rows, H, stream));
}

ubep_status ubep_expert_linear(const ubep_shape* s, int64_t N, const int32_t* expert_offset,
                               const void* x, const void* w, void* y, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
    const ubep_status st = ubep_check_shape(s, UBEP_BF16);
    if (st != UBEP_OK) return st;
    if (!expert_offset || !x || !w || !y || !ws || ws_bytes < kHdrBytes) return UBEP_ERR_INVALID_ARG;
    if (N <= 0 || N % 128 != 0 || s->H % 64 != 0 || s->H > ((int64_t)1 << 22)) return UBEP_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16) || !aligned(ws, 256) ||
        !aligned(expert_offset, 4))
        return UBEP_ERR_INVALID_ARG;
    const int64_t rows = s->T * (int64_t)s->k;
    if (s->E > kExpertMaxE || (rows + 127) / 128 + s->E > kExpertMaxRowTiles || N / 128 > (1 << 30) ||
        N >= ((int64_t)1 << 30))
        return UBEP_ERR_UNSUPPORTED;
    uint32_t* status = static_cast<uint32_t*>(ws) + kHdrStatus;
    return hip_status(launch_expert_linear(s->E, s->H, N, rows, expert_offset, x, w, y, status, stream));
}

ubep_status ubep_expert_pack_weights(int32_t E, int64_t N, int64_t H, const void* w, void* packed,
                                     hipStream_t stream) {
    if (!w || !packed || E <= 0 || N <= 0 || H <= 0) return UBEP_ERR_INVALID_ARG;
    if (N % 128 != 0 || H % 64 != 0 || H > ((int64_t)1 << 22) || E > kExpertMaxE)
        return UBEP_ERR_UNSUPPORTED;
    if (!aligned(w, 16) || !aligned(packed, 16) || w == packed) return UBEP_ERR_INVALID_ARG;
    if ((int64_t)E * N * H / 8 / 256 >= ((int64_t)1 << 32)) return UBEP_ERR_UNSUPPORTED;
    return hip_status(launch_expert_pack(E, N, H, w, packed, stream));
}

ubep_status ubep_get_device_status(void* ws, size_t ws_bytes, hipStream_t stream,
                                   ubep_status* out) {
    if (ws == nullptr || out == nullptr || ws_bytes < kHdrBytes || !aligned(ws, 256))
        return UBEP_ERR_INVALID_ARG;
    uint32_t v = 0;
    uint32_t* status = static_cast<uint32_t*>(ws) + kHdrStatus;
    if (hipStreamSynchronize(stream) != hipSuccess) return UBEP_ERR_HIP;
    if (hipMemcpy(&v, status, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return UBEP_ERR_HIP;
    if (launch_clear_status(status, stream) != hipSuccess) return UBEP_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return UBEP_ERR_HIP;
    *out = (ubep_status)v;
    return UBEP_OK;
}

ubep_status ubep_identity_expert_fp8(int64_t rows, int64_t H, const uint8_t* q, const float* scale,
                                     void* y, hipStream_t stream) {
    if (rows < 0 || H <= 0 || H % 128 != 0 || !q || !scale || !y) return UBEP_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(y, 16) || !aligned(scale, 4)) return UBEP_ERR_INVALID_ARG;
    if (rows == 0) return UBEP_OK;
    return hip_status(launch_identity_fp8(rows, H, q, scale, y, stream));
}

ubep_status ubep_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    if (!src || !dst || bytes % 16 != 0 || !aligned(src, 16) || !aligned(dst, 16))
        return UBEP_ERR_INVALID_ARG;
    if (bytes == 0) return UBEP_OK;
    return hip_status(launch_copy(src, dst, bytes, stream));
}

ubep_status ubep_stream_probe(const void* src, void* dst, int64_t n_vec, int fan_in, int fan_out,
                              hipStream_t stream) {
    const bool shape_ok = (fan_in == 0 || fan_in == 1 || fan_in == 8) &&
                          (fan_out == 0 || fan_out == 1 || fan_out == 8) && fan_in + fan_out > 0;
    if (!shape_ok || n_vec < 0 || !dst || (fan_in > 0 && !src)) return UBEP_ERR_INVALID_ARG;
    if (!aligned(dst, 16) || (src && !aligned(src, 16))) return UBEP_ERR_INVALID_ARG;
    if (n_vec >= ((int64_t)1 << 36)) return UBEP_ERR_UNSUPPORTED;
    if (n_vec == 0) return UBEP_OK;
    return hip_status(launch_stream_probe(src, dst, n_vec, fan_in, fan_out, stream));
}

ubep_status ubep_time_next_launch(hipEvent_t start, hipEvent_t stop) {
    if ((start == nullptr) != (stop == nullptr)) return UBEP_ERR_INVALID_ARG;
    set_launch_events(start, stop);
    return UBEP_OK;
}

ubep_status ubep_set_layout_workers(int32_t n) {
    if (n < 0) return UBEP_ERR_INVALID_ARG;
    set_layout_worker_cap(n);
    return UBEP_OK;
}

}  // extern "C"

// Gate (router) on gfx950: fp32 logits -> the k selected experts of each
// token and their normalised weights ("NJU x Huawei UBEP: Reengineering MoE
// Expert Parallelism", opening section: each token is sent to the experts its
// gate selects).  The selection rule, group filter and weight formulas are
// the ones stated in include/ubep.h for ubep_gate.
//
// The general kernel (gate_kernel, every shape the call accepts): one wave
// per token.  Lane l holds experts l, l + 64, l + 128, ... (each
// load instruction reads 64 consecutive logits).  Groups of a power-of-two
// size up to 64 are aligned runs of lanes, whose best two logits a butterfly
// finds; other group sizes go through a copy of the row in LDS, one lane per
// group.  Every selection decision is an exact fp32 comparison: larger logit
// first, equal logits to the lower id, made by repeated wave-wide arg-max over
// (logit, id) pairs.
#include "device_common.h"
#include "launch.h"

namespace ubep {

constexpr int kGateThreads = 256;
constexpr int kGateWaves = kGateThreads / 64;

struct GateArgs {
    const float* logits;
    int32_t* idx;
    float* w;
    int64_t T;
    int32_t E, k, groups, keep, norm;
};

// (v, e) ranks before (u, f): larger value first, equal values in ascending id.
__device__ __forceinline__ bool ranks_before(float v, int32_t e, float u, int32_t f) {
    return v > u || (v == u && e < f);
}

// Wave-wide arg-max of (v, e) under ranks_before; every lane gets the winner.
__device__ __forceinline__ void wave_best(float& v, int32_t& e) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float u = __shfl_xor(v, o, 64);
        const int32_t f = __shfl_xor(e, o, 64);
        if (ranks_before(u, f, v, e)) {
            v = u;
            e = f;
        }
    }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// VPL: logits a lane holds (E <= 64 * VPL).
template <int VPL>
__global__ __launch_bounds__(kGateThreads) void gate_kernel(GateArgs a) {
    __shared__ float s_z[kGateWaves][kGateMaxE];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kGateWaves + wv;
    const bool live = t < a.T;                      // uniform across the wave
    const int32_t E = a.E, gsize = E / a.groups;
    const float* zr = a.logits + (live ? t : 0) * E;
    constexpr float kNone = -__builtin_huge_valf();
    constexpr int32_t kNoId = 0x7fffffff;

    float v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {                 // unconditional loads from valid addresses
        const int32_t e = lane + 64 * i;
        v[i] = zr[e < E ? e : 0];
    }

    // kept groups (bit g); one group keeps everything
    uint64_t kept = ~0ull;
    const bool pow2 = (gsize & (gsize - 1)) == 0 && gsize <= 64;
    if (a.groups > 1 && pow2) {
        // groups are aligned runs of gsize lanes in each row i: a butterfly
        // inside the run leaves every lane with its group's best two
        float gsc[VPL];
        int32_t gg[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int32_t e = lane + 64 * i;
            float a1 = e < E ? v[i] : kNone, a2 = kNone;
            int32_t i1 = e < E ? e : kNoId, i2 = kNoId;
            for (int o = 1; o < gsize; o <<= 1) {
                const float b1 = __shfl_xor(a1, o, 64), b2 = __shfl_xor(a2, o, 64);
                const int32_t j1 = __shfl_xor(i1, o, 64), j2 = __shfl_xor(i2, o, 64);
                if (ranks_before(b1, j1, a1, i1)) {      // the partner's best leads
                    if (ranks_before(a1, i1, b2, j2)) {
                        a2 = a1;
                        i2 = i1;
                    } else {
                        a2 = b2;
                        i2 = j2;
                    }
                    a1 = b1;
                    i1 = j1;
                } else if (ranks_before(b1, j1, a2, i2)) {
                    a2 = b1;
                    i2 = j1;
                }
            }
            gsc[i] = e < E ? (gsize == 1 ? a1 : a1 + a2) : kNone;
            gg[i] = e < E ? e / gsize : kNoId;
        }
        kept = 0;
        for (int32_t r = 0; r < a.keep; ++r) {
            float bv = kNone;
            int32_t bg = kNoId;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (ranks_before(gsc[i], gg[i], bv, bg)) {
                    bv = gsc[i];
                    bg = gg[i];
                }
            wave_best(bv, bg);
            kept |= 1ull << bg;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (gg[i] == bg) {
                    gsc[i] = kNone;
                    gg[i] = kNoId;
                }
        }
    } else if (a.groups > 1) {
        // other group sizes: the row goes to LDS and lane g scans group g
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int32_t e = lane + 64 * i;
            if (e < E) s_z[wv][e] = v[i];
        }
        __syncthreads();
        float gscore = kNone;
        int32_t gid = kNoId;
        if (lane < a.groups) {
            float b1 = kNone, b2 = kNone;
            int32_t i1 = kNoId, i2 = kNoId;
            for (int32_t e = lane * gsize; e < (lane + 1) * gsize; ++e) {
                const float z = s_z[wv][e];
                if (ranks_before(z, e, b1, i1)) {
                    b2 = b1;
                    i2 = i1;
                    b1 = z;
                    i1 = e;
                } else if (ranks_before(z, e, b2, i2)) {
                    b2 = z;
                    i2 = e;
                }
            }
            gscore = gsize == 1 ? b1 : b1 + b2;
            gid = lane;
        }
        kept = 0;
        for (int32_t r = 0; r < a.keep; ++r) {
            float bv = gscore;
            int32_t bg = gid;
            wave_best(bv, bg);
            kept |= 1ull << bg;
            if (lane == bg) {
                gscore = kNone;
                gid = kNoId;
            }
        }
    }

    // the k best experts of the kept groups
    bool open[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int32_t e = lane + 64 * i;
        open[i] = e < E && ((kept >> (e / gsize)) & 1ull);
    }
    float mine_v = kNone;                           // lane j: the j-th selected expert
    int32_t mine_e = kNoId;
    float top = kNone;
    for (int32_t j = 0; j < a.k; ++j) {
        float bv = kNone;
        int32_t be = kNoId;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int32_t e = lane + 64 * i;
            if (open[i] && ranks_before(v[i], e, bv, be)) {
                bv = v[i];
                be = e;
            }
        }
        wave_best(bv, be);
        if (j == 0) top = bv;
        if (lane == j) {
            mine_v = bv;
            mine_e = be;
        }
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (lane + 64 * i == be) open[i] = false;
    }

    // weights over the selected experts, in fp32
    const bool sel = lane < a.k;
    float u = 0.0f;
    if (sel) u = a.norm == UBEP_GATE_SOFTMAX ? expf(mine_v - top) : 1.0f / (1.0f + expf(-mine_v));
    const float sum = wave_sum(u);
    if (live && sel) {
        a.idx[t * a.k + lane] = mine_e;
        a.w[t * a.k + lane] = u / sum;
    }
}

// ---------------------------------------------------------------- row kernel
// Four tokens per wave: token r of a wave owns DPP row r (16 lanes), lane l of
// the row holds its VPL consecutive logits [l*VPL, (l+1)*VPL) (VPL/4 16-byte
// loads; a wave reads 4 rows back to back).  Each lane keeps its four best
// (logit, id) pairs, found with exact fp32 comparisons in ascending id order,
// so that a strict comparison keeps the lower id among equal logits.  Each of
// the k selection rounds finds the row's best remaining pair with two 4-step
// rotate-within-row reductions, each step one DPP max or min instruction: the
// largest logit as an order-preserving integer (-0 and +0 map to one value,
// as fp32 compares them), then the lowest id among the lanes holding it.  The
// lane that wins a round pops its best; it rescans its VPL logits below its
// last pick only after giving all four.
// Groups: a group spans `span` aligned lanes (gsize = span * VPL); the lanes'
// two best logits are merged across the span with xor shuffles, and each lane
// ranks its group's score against the row's G = 16 / span groups.
constexpr int kRowLanes = 16;
constexpr int kGateRowTokens = kGateThreads / kRowLanes;   // tokens per workgroup

// Finite fp32 -> int32 of the same order, with -0 and +0 both 0 (sign and
// magnitude to two's complement); value_of inverts it (0 -> +0).
__device__ __forceinline__ int32_t ord_of(float v) {
    const int32_t s = __float_as_int(v);
    return s < 0 ? -(s & 0x7FFFFFFF) : s;
}
__device__ __forceinline__ float value_of(int32_t o) {
    return o < 0 ? __int_as_float((-o) | (int32_t)0x80000000) : __int_as_float(o);
}

// Every lane of a 16-lane row receives the row's maximum (minimum).  DPP
// row_ror n (dpp_ctrl 0x120 + n) reads a lane of the same row for every n, so
// no lane takes the bound_ctrl fill; the compiler folds each move into the
// max (min) as one DPP instruction.
constexpr int kDppRowRor = 0x120;       // row_ror:n = 0x120 + n
constexpr int kDppRowBcast = 0x150;     // row_newbcast:n = 0x150 + n (every lane reads row lane n)
template <int CTRL>
__device__ __forceinline__ int32_t dpp_i(int32_t x) { return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true); }
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) { return __int_as_float(dpp_i<CTRL>(__float_as_int(x))); }

template <bool MAX>
__device__ __forceinline__ int32_t row_reduce(int32_t x) {
    int32_t o = dpp_i<kDppRowRor + 8>(x);
    x = MAX ? max(x, o) : min(x, o);
    o = dpp_i<kDppRowRor + 4>(x);
    x = MAX ? max(x, o) : min(x, o);
    o = dpp_i<kDppRowRor + 2>(x);
    x = MAX ? max(x, o) : min(x, o);
    o = dpp_i<kDppRowRor + 1>(x);
    return MAX ? max(x, o) : min(x, o);
}

// Insert (v, e) into a lane's sorted best four; (v, e) comes after every
// pair already held that has an equal logit (ids ascend as the lane scans).
// Four rather than three: a lane rescans its logits once it has given all it
// holds, and a wave takes the rescan's path when any of its lanes needs it,
// so the fourth pair's cost per logit buys fewer rescans (the gate of 65536
// grouped tokens: 27.9 against 30.1 us; of 4096 tokens: 5.5 against 7.4 us).
// Written out, not as a loop over arrays: that form compiled to a slower
// kernel (29.4 and 6.9 us).
__device__ __forceinline__ void insert4(float v, int32_t e, float& t1, int32_t& i1, float& t2,
                                        int32_t& i2, float& t3, int32_t& i3, float& t4, int32_t& i4) {
    const bool g1 = v > t1, g2 = v > t2, g3 = v > t3, g4 = v > t4;
    t4 = g3 ? t3 : (g4 ? v : t4);
    i4 = g3 ? i3 : (g4 ? e : i4);
    t3 = g2 ? t2 : (g3 ? v : t3);
    i3 = g2 ? i2 : (g3 ? e : i3);
    t2 = g1 ? t1 : (g2 ? v : t2);
    i2 = g1 ? i1 : (g2 ? e : i2);
    t1 = g1 ? v : t1;
    i1 = g1 ? e : i1;
}

// Per-tile counts the gate hands to the layout (ubep_gate_layout): rows per
// (layout tile, destination rank) and per (layout tile, expert).
struct GateCounts {
    int32_t* rank_cnt;       // [n_tiles][R]
    int32_t* expert_cnt;     // [n_tiles][E]
    int64_t tile_tokens;     // a multiple of the workgroup's kGateRowTokens tokens
    int32_t R;
    uint32_t epr_magic;
};

template <int VPL, bool COUNT>
__global__ __launch_bounds__(kGateThreads) void gate_rows_kernel(GateArgs a, int32_t span,
                                                                 GateCounts gc) {
    __shared__ int32_t s_rc[COUNT ? kMaxR : 1];
    __shared__ int32_t s_ec[COUNT ? kGateMaxE : 1];
    if constexpr (COUNT) {
        for (int i = threadIdx.x; i < gc.R; i += kGateThreads) s_rc[i] = 0;
        for (int i = threadIdx.x; i < a.E; i += kGateThreads) s_ec[i] = 0;
    }
    constexpr float kNone = -__builtin_huge_valf();    // an empty slot: below every finite logit
    constexpr int32_t kNoId = 0x7fffffff;
    const int lane = threadIdx.x & 63;
    const int rl = lane & (kRowLanes - 1);                  // lane within the token's row
    const int64_t t = (int64_t)blockIdx.x * kGateRowTokens + (threadIdx.x >> 4);
    const bool live = t < a.T;
    const float4* zr = reinterpret_cast<const float4*>(a.logits + (live ? t : 0) * a.E) + rl * (VPL / 4);
    float z[VPL];
#pragma unroll
    for (int i = 0; i < VPL / 4; ++i) {
        const float4 q = zr[i];
        z[4 * i] = q.x;
        z[4 * i + 1] = q.y;
        z[4 * i + 2] = q.z;
        z[4 * i + 3] = q.w;
    }
    const int32_t id0 = rl * VPL;

    // the lane's best four (its two best also give the group score)
    float t1 = kNone, t2 = kNone, t3 = kNone, t4 = kNone;
    int32_t i1 = kNoId, i2 = kNoId, i3 = kNoId, i4 = kNoId;
#pragma unroll
    for (int i = 0; i < VPL; ++i) insert4(z[i], id0 + i, t1, i1, t2, i2, t3, i3, t4, i4);
    if (a.groups > 1) {
        // the group's two best logits across its span of lanes (values only:
        // the score does not depend on which of equal logits is taken)
        float b1 = t1, b2 = t2;
        for (int o = 1; o < span; o <<= 1) {
            const float c1 = __shfl_xor(b1, o, 64), c2 = __shfl_xor(b2, o, 64);
            const float lo1 = b1 > c1 ? c1 : b1, hi2 = b2 > c2 ? b2 : c2;
            b1 = b1 > c1 ? b1 : c1;
            b2 = lo1 > hi2 ? lo1 : hi2;
        }
        const float score = b1 + b2;                        // one fp32 addition
        const int32_t G = kRowLanes / span, g = rl / span;
        const int row0 = lane & ~(kRowLanes - 1);
        int32_t rank = 0;
        for (int32_t h = 0; h < G; ++h) {
            const float sh = __shfl(score, row0 + h * span, 64);
            rank += (sh > score || (sh == score && h < g)) ? 1 : 0;
        }
        if (rank >= a.keep) t1 = t2 = t3 = t4 = kNone;          // a dropped group offers nothing
    }

    // k rounds: the row's best remaining pair; its owner pops it.  A lane that
    // has given its four may hold more (after its last pick): when any lane
    // of the wave is in that state, those lanes rescan for their next four.
    bool more = t4 != kNone;      // this lane may hold candidates past t4
    float last_v = 0.0f;          // this lane's last pick
    int32_t last_i = 0;
    int32_t mine_o = 0, mine_i = 0, top_o = 0;
    for (int32_t j = 0; j < a.k; ++j) {
        const int32_t o = ord_of(t1);
        const int32_t m = row_reduce<true>(o);
        const int32_t mi = row_reduce<false>(o == m ? i1 : kNoId);
        if (j == 0) top_o = m;
        if (rl == j) {
            mine_o = m;
            mine_i = mi;
        }
        if (o == m && i1 == mi) {
            last_v = t1;
            last_i = i1;
            t1 = t2;
            i1 = i2;
            t2 = t3;
            i2 = i3;
            t3 = t4;
            i3 = i4;
            t4 = kNone;
            i4 = kNoId;
        }
        const bool refill = more && t1 == kNone;
        if (__any(refill)) {
            if (refill) {
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const int32_t e = id0 + i;
                    const bool after = z[i] < last_v || (z[i] == last_v && e > last_i);
                    insert4(after ? z[i] : kNone, e, t1, i1, t2, i2, t3, i3, t4, i4);
                }
                more = t4 != kNone;
            }
        }
    }

    // weights over the selected experts, in fp32; the row's sum from its lane 0
    const bool sel = rl < a.k;
    const float mv = value_of(mine_o), tv = value_of(top_o);
    float u = 0.0f;
    if (sel) u = a.norm == UBEP_GATE_SOFTMAX ? expf(mv - tv) : 1.0f / (1.0f + expf(-mv));
    float sum = u;                                      // rotate-and-add within the row,
    sum += dpp_f<kDppRowRor + 8>(sum);                  // then row lane 0's total for all
    sum += dpp_f<kDppRowRor + 4>(sum);
    sum += dpp_f<kDppRowRor + 2>(sum);
    sum += dpp_f<kDppRowRor + 1>(sum);
    sum = dpp_f<kDppRowBcast + 0>(sum);
    if (live && sel) {
        a.idx[t * a.k + rl] = mine_i;
        a.w[t * a.k + rl] = u / sum;
    }
    if constexpr (COUNT) {
        // this workgroup's tokens all lie in one layout tile: count its rows
        // per rank and per expert in LDS, then add the nonzero counts to the
        // tile's rows of the workspace arrays
        __syncthreads();
        if (live && sel) {
            const uint32_t e = (uint32_t)mine_i;
            atomicAdd(&s_rc[rank_of(e, gc.epr_magic)], 1);
            atomicAdd(&s_ec[e], 1);
        }
        __syncthreads();
        const int64_t tile = (int64_t)blockIdx.x * kGateRowTokens / gc.tile_tokens;
        for (int i = threadIdx.x; i < gc.R; i += kGateThreads)
            if (s_rc[i] != 0) add_relaxed(reinterpret_cast<uint32_t*>(gc.rank_cnt + tile * gc.R + i), (uint32_t)s_rc[i]);
        for (int i = threadIdx.x; i < a.E; i += kGateThreads)
            if (s_ec[i] != 0) add_relaxed(reinterpret_cast<uint32_t*>(gc.expert_cnt + tile * a.E + i), (uint32_t)s_ec[i]);
    }
}

// The row kernel covers E = 16 * VPL with VPL in {4, 8, 16} (E in {64, 128,
// 256}), k <= 16, 16-byte aligned logits, and groups that are aligned
// power-of-two runs of whole lanes.
static int gate_row_vpl(const ubep_gate_shape& g, const float* logits) {
    if (g.k > kRowLanes || ((uintptr_t)logits % 16) != 0) return 0;
    if (g.E != 64 && g.E != 128 && g.E != 256) return 0;
    const int vpl = g.E / kRowLanes;
    if (g.groups > 1) {
        const int gsize = g.E / g.groups;
        if (gsize % vpl != 0) return 0;
        const int span = gsize / vpl;
        if ((span & (span - 1)) != 0 || span > kRowLanes) return 0;
    }
    return vpl;
}

hipError_t launch_gate(const ubep_gate_shape& g, const float* logits, int32_t* idx, float* w,
                       hipStream_t stream) {
    return launch_gate_counting(g, logits, idx, w, nullptr, stream);
}

bool gate_counts_fit(const ubep_gate_shape& g, const float* logits, int64_t tile_tokens) {
    return gate_row_vpl(g, logits) != 0 && tile_tokens % kGateRowTokens == 0;
}

hipError_t launch_gate_counting(const ubep_gate_shape& g, const float* logits, int32_t* idx,
                                float* w, const GateCountArgs* counts, hipStream_t stream) {
    GateArgs a;
    a.logits = logits;
    a.idx = idx;
    a.w = w;
    a.T = g.T;
    a.E = g.E;
    a.k = g.k;
    a.groups = g.groups;
    a.keep = g.keep_groups;
    a.norm = g.norm;
    const int rv = gate_row_vpl(g, logits);
    if (counts != nullptr && (rv == 0 || counts->tile_tokens % kGateRowTokens != 0))
        return hipErrorInvalidValue;                 // callers check gate_counts_fit first
    if (rv != 0) {
        const int32_t span = g.groups > 1 ? (g.E / g.groups) / rv : 1;
        const dim3 grid((unsigned)((g.T + kGateRowTokens - 1) / kGateRowTokens)), block(kGateThreads);
        GateCounts gc{};
        if (counts != nullptr) {
            gc.rank_cnt = counts->rank_cnt;
            gc.expert_cnt = counts->expert_cnt;
            gc.tile_tokens = counts->tile_tokens;
            gc.R = counts->R;
            gc.epr_magic = counts->epr_magic;
            if (rv == 4) return launch_kernel(gate_rows_kernel<4, true>, grid, block, 0, stream, a, span, gc);
            if (rv == 8) return launch_kernel(gate_rows_kernel<8, true>, grid, block, 0, stream, a, span, gc);
            return launch_kernel(gate_rows_kernel<16, true>, grid, block, 0, stream, a, span, gc);
        }
        if (rv == 4) return launch_kernel(gate_rows_kernel<4, false>, grid, block, 0, stream, a, span, gc);
        if (rv == 8) return launch_kernel(gate_rows_kernel<8, false>, grid, block, 0, stream, a, span, gc);
        return launch_kernel(gate_rows_kernel<16, false>, grid, block, 0, stream, a, span, gc);
    }
    const int64_t blocks = (g.T + kGateWaves - 1) / kGateWaves;
    const int vpl = (g.E + 63) / 64;
    if (vpl <= 1) return launch_kernel(gate_kernel<1>, dim3((unsigned)blocks), dim3(kGateThreads), 0, stream, a);
    if (vpl <= 2) return launch_kernel(gate_kernel<2>, dim3((unsigned)blocks), dim3(kGateThreads), 0, stream, a);
    if (vpl <= 4) return launch_kernel(gate_kernel<4>, dim3((unsigned)blocks), dim3(kGateThreads), 0, stream, a);
    if (vpl <= 8) return launch_kernel(gate_kernel<8>, dim3((unsigned)blocks), dim3(kGateThreads), 0, stream, a);
    return launch_kernel(gate_kernel<16>, dim3((unsigned)blocks), dim3(kGateThreads), 0, stream, a);
}

}  // namespace ubep

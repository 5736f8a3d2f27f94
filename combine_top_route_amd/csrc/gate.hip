// Gate (router) on gfx950: fp32 logits -> the k selected experts of each
// token and their normalised weights ("NJU x Huawei UBEP: Reengineering MoE
// Expert Parallelism", opening section: each token is sent to the experts its
// gate selects).  The selection rule, group filter and weight formulas are
// the ones stated in include/ubep.h for ubep_gate.
//
// One wave per token.  Lane l holds experts l, l + 64, l + 128, ... (each
// load instruction reads 64 consecutive logits).  Groups of a power-of-two
// size up to 64 are aligned runs of lanes, whose best two logits a butterfly
// finds; other group sizes go through a copy of the row in LDS, one lane per
// group.  Every selection decision is an exact fp32 comparison: larger logit
// first, equal logits to the lower id, made by repeated wave-wide arg-max over
// (logit, id) pairs.
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

hipError_t launch_gate(const ubep_gate_shape& g, const float* logits, int32_t* idx, float* w,
                       hipStream_t stream) {
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
    const int64_t blocks = (g.T + kGateWaves - 1) / kGateWaves;
    const int vpl = (g.E + 63) / 64;
    if (vpl <= 1) return launch_kernel(gate_kernel<1>, dim3((unsigned)blocks), dim3(kGateThreads), 0, stream, a);
    if (vpl <= 2) return launch_kernel(gate_kernel<2>, dim3((unsigned)blocks), dim3(kGateThreads), 0, stream, a);
    if (vpl <= 4) return launch_kernel(gate_kernel<4>, dim3((unsigned)blocks), dim3(kGateThreads), 0, stream, a);
    if (vpl <= 8) return launch_kernel(gate_kernel<8>, dim3((unsigned)blocks), dim3(kGateThreads), 0, stream, a);
    return launch_kernel(gate_kernel<16>, dim3((unsigned)blocks), dim3(kGateThreads), 0, stream, a);
}

}  // namespace ubep

// Combine kernel: one group of whole waves per token gathers the token's k
// expert-output rows ("NJU x Huawei UBEP: Reengineering MoE Expert
// Parallelism", opening section: outputs are gathered back to their token in
// the Combine phase) and reduces them with a slot-ordered fp32 FMA chain.
// The token's k positions and weights are uniform across its group and are
// read once through the scalar data path; each thread keeps KB slot vectors
// in flight before it runs the chain.
#include "launch.h"
#include "rows.h"

namespace ubep {

constexpr int kCombineBlock = 256;
constexpr int kSlotBatch = 8;

template <int G, int VPT>
__global__ __launch_bounds__(kCombineBlock) void combine_kernel(const u32x4* __restrict__ y,
                                                                const int32_t* __restrict__ pos,
                                                                const float* __restrict__ w,
                                                                u32x4* __restrict__ out, int64_t T,
                                                                int32_t k, int64_t nvec,
                                                                int64_t n_rows, uint32_t* status) {
    constexpr int TPB = kCombineBlock / G;
    const int64_t t = (int64_t)blockIdx.x * TPB + threadIdx.x / G;
    if (t >= T) return;
    combine_row<G, VPT, kSlotBatch>(y, pos, w, out, t, k, nvec, n_rows, threadIdx.x % G, status);
}

template <int G, int VPT>
static hipError_t launch_gv(const Plan& p, const void* y, const int32_t* pos, const float* w,
                            void* out, uint32_t* status, hipStream_t stream) {
    constexpr int TPB = kCombineBlock / G;
    const int64_t blocks = (p.T + TPB - 1) / TPB;
    hipLaunchKernelGGL((combine_kernel<G, VPT>), dim3((unsigned)blocks), dim3(kCombineBlock), 0,
                       stream, static_cast<const u32x4*>(y), pos, w, static_cast<u32x4*>(out),
                       p.T, p.k, p.H / 8, p.rows, status);
    return hipGetLastError();
}

template <int G>
static hipError_t launch_g(int vpt, const Plan& p, const void* y, const int32_t* pos,
                           const float* w, void* out, uint32_t* status, hipStream_t stream) {
    switch (vpt) {
        case 1: return launch_gv<G, 1>(p, y, pos, w, out, status, stream);
        case 2: return launch_gv<G, 2>(p, y, pos, w, out, status, stream);
        case 3: return launch_gv<G, 3>(p, y, pos, w, out, status, stream);
        case 4: return launch_gv<G, 4>(p, y, pos, w, out, status, stream);
        case 5: return launch_gv<G, 5>(p, y, pos, w, out, status, stream);
        case 6: return launch_gv<G, 6>(p, y, pos, w, out, status, stream);
        case 7: return launch_gv<G, 7>(p, y, pos, w, out, status, stream);
        default: return launch_gv<G, 8>(p, y, pos, w, out, status, stream);
    }
}

hipError_t launch_combine(const Plan& p, const void* y, const int32_t* pos, const float* topk_w,
                          void* out, uint32_t* status, hipStream_t stream) {
    const int64_t nvec = p.H / 8;
    int G = 256, VPT = 8;
    for (int g = 64; g <= 256; g *= 2) {
        if (nvec <= (int64_t)g * 8) {
            G = g;
            VPT = (int)((nvec + g - 1) / g);
            break;
        }
    }
    switch (G) {
        case 64: return launch_g<64>(VPT, p, y, pos, topk_w, out, status, stream);
        case 128: return launch_g<128>(VPT, p, y, pos, topk_w, out, status, stream);
        default: return launch_g<256>(VPT, p, y, pos, topk_w, out, status, stream);
    }
}

}  // namespace ubep

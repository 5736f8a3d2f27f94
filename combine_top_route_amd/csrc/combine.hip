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
                                                                int64_t n_rows, uint32_t* status,
                                                                uint32_t n_static) {
    constexpr int TPB = kCombineBlock / G;
    const uint32_t blk = claim_block(status + kHdrCombineTicket, n_static, status);
    const int64_t t = (int64_t)blk * TPB + threadIdx.x / G;
    if (t >= T) return;
    combine_row<G, VPT, kSlotBatch>(y, pos, w, out, t, k, nvec, n_rows, threadIdx.x % G, status);
}

// Two waves per token where the shared rule gives one wave eight vectors per
// thread (449 to 512 vectors, H = 4096 among them): two waves of four
// vectors each took 208 us against 225 us for the combine of a 16384-token
// chunk at H = 4096.  (Rows of 256 vectors stay at one wave: two waves of two
// vectors each were 15 % slower on 65536 tokens.)
static void pick_combine_group(int64_t nvec, int* G, int* VPT) {
    pick_group(nvec, G, VPT);
    if (*G == 64 && *VPT == kVptCap) {
        *G = 128;
        *VPT = (int)((nvec + 127) / 128);
    }
}

hipError_t launch_combine(const Plan& p, const void* y, const int32_t* pos, const float* topk_w,
                          void* out, uint32_t* status, hipStream_t stream) {
    int G, VPT;
    pick_combine_group(p.H / 8, &G, &VPT);
    auto go = [&]<int GG, int VV>() -> hipError_t {
        constexpr int TPB = kCombineBlock / GG;
        const int64_t blocks = (p.T + TPB - 1) / TPB;
        int64_t n_static = 0;
        const hipError_t e = resident_blocks(reinterpret_cast<const void*>(combine_kernel<GG, VV>),
                                             kCombineBlock, 0, &n_static);
        if (e != hipSuccess) return e;
        // start-order tickets only when later workgroups are many more than
        // the first resident wave (long grids drift apart across XCDs); with
        // a grid of a few waves they cost more than they save
        if (blocks < kTicketMinWaves * n_static) n_static = blocks;
        return launch_kernel(combine_kernel<GG, VV>, dim3((unsigned)blocks), dim3(kCombineBlock), 0,
                             stream, static_cast<const u32x4*>(y), pos, topk_w,
                             static_cast<u32x4*>(out), p.T, p.k, p.H / 8, p.rows, status,
                             (uint32_t)n_static);
    };
    return with_group(G, VPT, go);
}

}  // namespace ubep

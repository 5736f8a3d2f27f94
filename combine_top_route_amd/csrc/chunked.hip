// Chunked dispatch + combine in one persistent kernel ("NJU x Huawei UBEP:
// Reengineering MoE Expert Parallelism", "Kernel Decomposition": a global
// barrier is replaced by results written to global memory that consumers
// poll, so stages overlap; "The Synchronization Tax": barriers cost up to 15%
// of the time; "Data-for-Checksum": one completion signal per batch of data).
//
// Tokens form C contiguous chunks, each split into n tasks of a few tokens.
// A workgroup repeatedly takes the next ticket from one counter in HBM; the
// tickets enumerate D(o0), D(o1), C(o0), D(o2), C(o1), ..., C(o_{C-1}) for the
// host-chosen chunk order o.  A D task dispatches its tokens and then adds one
// to its chunk's ready flag (agent-scope release); a C task of chunk c waits
// until that flag reaches n (agent-scope acquire) and combines its tokens.
// Every D task of chunk c has a smaller ticket than every C task of chunk c,
// and D tasks never wait, so each awaited task is already held by a running
// workgroup: the pipeline cannot deadlock whatever the grid size.  Waits are
// bounded by a clock limit; an expired wait records UBEP_ERR_TIMEOUT and
// moves on, so every workgroup always reaches the exit.  The last workgroup
// to leave resets the ticket and the flags for the next call.
#include "launch.h"
#include "rows.h"

namespace ubep {

constexpr int kChunkBlock = 256;

struct ChunkArgs {
    const u32x4* x;
    const int32_t* pos;
    const float* w;
    u32x4* recv;
    u32x4* out;
    uint32_t* hdr;
    uint32_t* flags;
    int64_t T, nvec, n_rows, tpc;
    int32_t k, C;
    int32_t tpt;        // tokens per task
    int32_t n;          // tasks per chunk (of each kind)
    uint32_t total;     // 2 * C * n tickets
    uint64_t spin_ticks;
    uint32_t debug;
    int16_t order[kMaxC];
};

template <int G, int VPT>
__global__ __launch_bounds__(kChunkBlock) void chunked_kernel(ChunkArgs a) {
    constexpr int TPB = kChunkBlock / G;
    __shared__ uint32_t s_ticket;
    const int tid = threadIdx.x;
    const int gtid = tid % G;
    uint32_t* status = &a.hdr[kHdrStatus];

    for (;;) {
        if (tid == 0) s_ticket = add_relaxed(&a.hdr[kHdrFusedTicket], 1u);
        __syncthreads();
        const uint32_t ticket = s_ticket;
        __syncthreads();
        if (ticket >= a.total) break;

        // decode the ticket
        const uint32_t n = (uint32_t)a.n;
        bool is_d;
        int32_t c;
        uint32_t idx;
        if (ticket < n) {
            is_d = true;
            c = a.order[0];
            idx = ticket;
        } else {
            const uint32_t u = ticket - n, pair = u / (2u * n), r = u % (2u * n);
            if (pair + 1u < (uint32_t)a.C) {
                is_d = r < n;
                c = is_d ? a.order[pair + 1u] : a.order[pair];
                idx = is_d ? r : r - n;
            } else {
                is_d = false;
                c = a.order[a.C - 1];
                idx = r;
            }
        }
        const int64_t c_lo = (int64_t)c * a.tpc, c_hi = c_lo + a.tpc;
        const int64_t t_lo = c_lo + (int64_t)idx * a.tpt;
        const int64_t t_hi = t_lo + a.tpt < c_hi ? t_lo + a.tpt : c_hi;
        uint32_t* flag = a.flags + (int64_t)c * kFlagStride;

        if (is_d) {
            for (int64_t t = t_lo + tid / G; t < t_hi; t += TPB)
                dispatch_row_bf16<G, VPT, false>(a.x, a.pos, a.recv, t, a.k, a.nvec, a.n_rows, gtid,
                                                 status);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __syncthreads();
            if (tid == 0 && (a.debug & 1u) == 0u) add_release(flag, 1u);
        } else {
            if (tid == 0) {
                const uint64_t t0 = now_ticks();
                while (ld_acquire(flag) < n) {
                    if (now_ticks() - t0 > a.spin_ticks) {
                        raise_status(status, UBEP_ERR_TIMEOUT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            __syncthreads();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            for (int64_t t = t_lo + tid / G; t < t_hi; t += TPB)
                combine_row<G, VPT, 8>(a.recv, a.pos, a.w, a.out, t, a.k, a.nvec, a.n_rows, gtid,
                                       status);
        }
    }

    if (tid == 0) {
        const uint32_t done = add_acq_rel(&a.hdr[kHdrFusedDone], 1u);
        if (done == gridDim.x - 1u) {
            for (int32_t c = 0; c < a.C; ++c) st_relaxed(a.flags + (int64_t)c * kFlagStride, 0u);
            st_relaxed(&a.hdr[kHdrFusedTicket], 0u);
            st_relaxed(&a.hdr[kHdrFusedDone], 0u);
        }
    }
}

template <int G, int VPT>
static hipError_t launch_gv(ChunkArgs& a, int device, hipStream_t stream) {
    DeviceInfo di;
    hipError_t e = device_info(device, &di);
    if (e != hipSuccess) return e;
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chunked_kernel<G, VPT>, kChunkBlock, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    int64_t grid = (int64_t)di.cus * per_cu;
    if (grid > (int64_t)a.total) grid = a.total;
    hipLaunchKernelGGL((chunked_kernel<G, VPT>), dim3((unsigned)grid), dim3(kChunkBlock), 0, stream,
                       a);
    return hipGetLastError();
}

template <int G>
static hipError_t launch_g(int vpt, ChunkArgs& a, int device, hipStream_t stream) {
    switch (vpt) {
        case 1: return launch_gv<G, 1>(a, device, stream);
        case 2: return launch_gv<G, 2>(a, device, stream);
        case 3: return launch_gv<G, 3>(a, device, stream);
        case 4: return launch_gv<G, 4>(a, device, stream);
        case 5: return launch_gv<G, 5>(a, device, stream);
        case 6: return launch_gv<G, 6>(a, device, stream);
        case 7: return launch_gv<G, 7>(a, device, stream);
        default: return launch_gv<G, 8>(a, device, stream);
    }
}

hipError_t launch_chunked(const Plan& p, const void* x, const int32_t* pos, const float* topk_w,
                          void* recv, void* out, const int32_t* chunk_order, uint64_t spin_ticks,
                          uint32_t debug_flags, void* ws, int device, hipStream_t stream) {
    const int64_t nvec = p.H / 8;
    int G = 256, VPT = 8;
    for (int g = 64; g <= 256; g *= 2) {
        if (nvec <= (int64_t)g * 8) {
            G = g;
            VPT = (int)((nvec + g - 1) / g);
            break;
        }
    }
    ChunkArgs a;
    a.x = static_cast<const u32x4*>(x);
    a.pos = pos;
    a.w = topk_w;
    a.recv = static_cast<u32x4*>(recv);
    a.out = static_cast<u32x4*>(out);
    char* base = static_cast<char*>(ws);
    a.hdr = reinterpret_cast<uint32_t*>(base);
    a.flags = reinterpret_cast<uint32_t*>(base + p.off_flags);
    a.T = p.T;
    a.nvec = nvec;
    a.n_rows = p.rows;
    a.tpc = p.tpc;
    a.k = p.k;
    a.C = p.C;
    // tasks of 4 passes of the workgroup's token groups (8 tokens for 2 tokens per pass)
    const int64_t tpb = kChunkBlock / G;
    int64_t tpt = tpb * 4;
    if (tpt > p.tpc) tpt = p.tpc;
    a.tpt = (int32_t)tpt;
    a.n = (int32_t)((p.tpc + tpt - 1) / tpt);
    a.total = (uint32_t)(2 * (int64_t)p.C * a.n);
    a.spin_ticks = spin_ticks;
    a.debug = debug_flags;
    for (int i = 0; i < kMaxC; ++i) a.order[i] = (int16_t)(i < p.C ? (chunk_order ? chunk_order[i] : i) : 0);
    switch (G) {
        case 64: return launch_g<64>(VPT, a, device, stream);
        case 128: return launch_g<128>(VPT, a, device, stream);
        default: return launch_g<256>(VPT, a, device, stream);
    }
}

}  // namespace ubep

// Dispatch + combine in one persistent kernel with token-granular readiness
// carried by the data itself ("NJU x Huawei UBEP: Reengineering MoE Expert
// Parallelism", "Data-as-Flag": instead of a separate ready flag, the
// consumer polls the payload for a sentinel value that real data never
// takes; the Sentinel Polling variant).
//
// Protocol, per receive row r:
//   - between calls the first 16-byte unit of r holds the sentinel (all bits
//     set: eight bf16 NaNs; a 32-bit word of all ones never occurs in the
//     inputs' first eight channels);
//   - the producer writes units 1.. of r with device-coherent stores, waits
//     until they have completed, and only then writes unit 0 (the token's
//     first eight channels) -- the unit the consumer polls is the last to
//     arrive, since AMD GPUs make no promise about the order in which the
//     16-byte pieces of one row become visible;
//   - the consumer polls unit 0 of each of its token's k rows with
//     device-coherent loads until no 32-bit word of it holds the sentinel
//     word (a 16-byte store may become visible piecewise), reads the rows,
//     runs the combine, and writes the sentinel back into unit 0.
// So readiness is per row, there is no flag array, and the only extra
// traffic is one 16-byte poll and one 16-byte restore per row.
//
// Tasks are blocks of TPB tokens (one token per group of G threads).  Tickets
// from one counter enumerate, for a lag of L blocks,
//   D(0) .. D(L-1),  D(L) C(0),  D(L+1) C(1),  ...,  C(nb-L) .. C(nb-1)
// and a C task waits only on the D task of the same block, which has a
// smaller ticket and never waits: every awaited task is held by a running
// workgroup, whatever the grid.  Waits are clock-bounded; once any wait has
// expired (UBEP_ERR_TIMEOUT in the status word, and a give-up word in the
// header whatever error the status word already holds) later waits give up
// at once, so a withheld row costs one time limit, not one per task.  A
// token whose own first eight channels hold the sentinel word can never look
// arrived: its consumer reports UBEP_ERR_SENTINEL_DATA and does not wait.
#include "launch.h"
#include "rows.h"

namespace ubep {

constexpr int kSentBlock = 256;

struct SentArgs {
    const u32x4* x;
    const int32_t* pos;
    const float* w;
    u32x4* recv;
    u32x4* out;
    uint32_t* hdr;
    int64_t T, nvec, n_rows;
    int32_t k;
    uint32_t nb;        // token blocks
    uint32_t lag;       // blocks between a block's D task and its C task
    uint64_t spin_ticks;
    uint32_t debug;
};

// A 16-byte store need not become visible all at once, so a unit counts as
// arrived only when none of its four 32-bit words still holds the sentinel
// word (inputs never hold it: it is a pair of bf16 NaNs).
__device__ __forceinline__ bool any_sentinel_word(u32x4 v) {
    return v[0] == kRowSentinelWord || v[1] == kRowSentinelWord || v[2] == kRowSentinelWord ||
           v[3] == kRowSentinelWord;
}

// Device-coherent 16-byte load of unit 0 that the compiler may not merge
// with an earlier one (bit 31 of the cache-policy operand: volatile).
__device__ __forceinline__ u32x4 poll16_device(__amdgpu_buffer_rsrc_t r) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, kCachePolicyDevice | (int)0x80000000u);
}

// NTS: the body stores of the rows carry the non-temporal hint as well.
template <int G, int VPT, bool NTS>
__global__ __launch_bounds__(kSentBlock) void sentinel_kernel(SentArgs a) {
    constexpr int TPB = kSentBlock / G;
    __shared__ uint32_t s_ticket;
    const int tid = threadIdx.x;
    const int gtid = tid % G;
    uint32_t* status = &a.hdr[kHdrStatus];
    const uint32_t total = 2u * a.nb, L = a.lag;

    for (;;) {
        if (tid == 0) s_ticket = add_relaxed(&a.hdr[kHdrSentTicket], 1u);
        __syncthreads();
        const uint32_t ticket = s_ticket;
        __syncthreads();
        if (ticket >= total) break;
        bool is_d;
        uint32_t blk;
        if (ticket < L) {
            is_d = true;
            blk = ticket;
        } else {
            const uint32_t u = ticket - L;
            if (u / 2u < a.nb - L) {
                is_d = (u & 1u) == 0u;
                blk = is_d ? u / 2u + L : u / 2u;
            } else {
                is_d = false;
                blk = a.nb - L + (u - 2u * (a.nb - L));
            }
        }
        const int64_t t = (int64_t)blk * TPB + tid / G;   // this group's token
        const bool has_t = t < a.T;

        if (is_d) {
            if (has_t)
                dispatch_row_bf16<G, VPT, NTS, true, true>(a.x, a.pos, a.recv, t, a.k, a.nvec,
                                                             a.n_rows, gtid, status);
            wait_memory();             // every body unit of the block is at the coherent level
            __syncthreads();
            if ((a.debug & kDebugDelay) != 0u && blk % 3u == 0u) debug_delay();
            if (has_t && gtid == 0 && (a.debug & kDebugWithhold) == 0u) {
                const u32x4 head = a.x[t * a.nvec];
                if (any_sentinel_word(head)) {
                    // such a head could never signal arrival: leave the
                    // sentinel in place (the consumer does not wait for it)
                    raise_status(status, UBEP_ERR_SENTINEL_DATA);
                } else {
                    for (int32_t j = 0; j < a.k; ++j) {
                        const int32_t q = a.pos[t * a.k + j];
                        if (row_ok(q, a.n_rows))
                            store16_device(row_rsrc(a.recv + (int64_t)q * a.nvec, a.nvec * 16), 0, head);
                    }
                }
            }
        } else {
            if (has_t && gtid == 0) {
                // rows of a token whose own head holds the sentinel word never
                // look arrived: report it (the producer does too) and skip the
                // wait; only that token's output is then unspecified
                const bool own_sentinel = any_sentinel_word(a.x[t * a.nvec]);
                if (own_sentinel) raise_status(status, UBEP_ERR_SENTINEL_DATA);
                const uint64_t t0 = now_ticks();
                for (int32_t j = 0; j < a.k && !own_sentinel; ++j) {
                    const int32_t q = a.pos[t * a.k + j];
                    if (!row_ok(q, a.n_rows)) continue;
                    const __amdgpu_buffer_rsrc_t rs = row_rsrc(a.recv + (int64_t)q * a.nvec, a.nvec * 16);
                    while (any_sentinel_word(poll16_device(rs))) {
                        if (now_ticks() - t0 > a.spin_ticks || ld_relaxed(&a.hdr[kHdrSentGiveUp]) != 0u) {
                            st_relaxed(&a.hdr[kHdrSentGiveUp], 1u);
                            raise_status(status, UBEP_ERR_TIMEOUT);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
            }
            __syncthreads();
            if (has_t) {
                combine_row<G, VPT, 8, true, false>(a.recv, a.pos, a.w, a.out, t, a.k, a.nvec,
                                                    a.n_rows, gtid, status);
                if (gtid == 0) {   // this thread alone read unit 0 of the rows
                    const u32x4 sent = {kRowSentinelWord, kRowSentinelWord, kRowSentinelWord,
                                        kRowSentinelWord};
                    for (int32_t j = 0; j < a.k; ++j) {
                        const int32_t q = a.pos[t * a.k + j];
                        if (row_ok(q, a.n_rows))
                            store16_device(row_rsrc(a.recv + (int64_t)q * a.nvec, a.nvec * 16), 0, sent);
                    }
                }
            }
        }
    }

    if (tid == 0) {
        // every workgroup's final ticket claim returned before this increment
        const uint32_t done = add_relaxed(&a.hdr[kHdrSentDone], 1u);
        if (done == gridDim.x - 1u) {
            st_relaxed(&a.hdr[kHdrSentTicket], 0u);
            st_relaxed(&a.hdr[kHdrSentGiveUp], 0u);
            st_relaxed(&a.hdr[kHdrSentDone], 0u);
        }
    }
}

// Unit 0 of every receive row := the sentinel.
__global__ __launch_bounds__(256) void sentinel_fill_kernel(u32x4* recv, int64_t rows, int64_t nvec) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r < rows) {
        const u32x4 sent = {kRowSentinelWord, kRowSentinelWord, kRowSentinelWord, kRowSentinelWord};
        recv[r * nvec] = sent;
    }
}

hipError_t launch_sentinel_fill(void* recv, int64_t rows, int64_t H, hipStream_t stream) {
    const int64_t blocks = (rows + 255) / 256;
    return launch_kernel(sentinel_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                         static_cast<u32x4*>(recv), rows, H / 8);
}

hipError_t launch_sentinel_pipeline(const Plan& p, const void* x, const int32_t* pos,
                                    const float* topk_w, void* recv, void* out, uint64_t spin_ticks,
                                    uint32_t debug_flags, void* ws, int device, hipStream_t stream) {
    const int64_t nvec = p.H / 8;
    int G, VPT;
    pick_group(nvec, &G, &VPT);
    SentArgs a;
    a.x = static_cast<const u32x4*>(x);
    a.pos = pos;
    a.w = topk_w;
    a.recv = static_cast<u32x4*>(recv);
    a.out = static_cast<u32x4*>(out);
    a.hdr = static_cast<uint32_t*>(ws);
    a.T = p.T;
    a.nvec = nvec;
    a.n_rows = p.rows;
    a.k = p.k;
    const int64_t tpb = kSentBlock / G;
    a.nb = (uint32_t)((p.T + tpb - 1) / tpb);
    a.spin_ticks = spin_ticks;
    a.debug = debug_flags;
    DeviceInfo di;
    hipError_t e = device_info(device, &di);
    if (e != hipSuccess) return e;
    // Above kNtxMaxBytes of receive rows the body stores are non-temporal too:
    // the 65536-token prefill took 3.32 against 3.42 ms with them, the decode
    // step 241 against 215 us.
    const bool nts = p.rows * p.H * 2 > kNtxMaxBytes;
    auto go = [&]<int GG, int VV>() -> hipError_t {
        const auto kernel = nts ? sentinel_kernel<GG, VV, true> : sentinel_kernel<GG, VV, false>;
        int per_cu = 0;
        hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kSentBlock, 0);
        if (err != hipSuccess) return err;
        if (per_cu < 1) per_cu = 1;
        int64_t grid = (int64_t)di.cus * per_cu;
        if (grid > 2 * (int64_t)a.nb) grid = 2 * (int64_t)a.nb;
        // blocks in flight: every resident workgroup holds one task
        int64_t lag = grid;
        a.lag = (uint32_t)(lag < 1 ? 1 : (lag > a.nb ? a.nb : lag));
        return launch_kernel(kernel, dim3((unsigned)grid), dim3(kSentBlock), 0, stream, a);
    };
    return with_group(G, VPT, go);
}

}  // namespace ubep

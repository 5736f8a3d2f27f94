// Chunked dispatch + combine in one persistent kernel ("NJU x Huawei UBEP:
// Reengineering MoE Expert Parallelism", "Kernel Decomposition": a global
// barrier is replaced by results written to global memory that consumers
// poll, so stages overlap; "The Synchronization Tax": barriers cost up to 15%
// of the time; "Data-for-Checksum": one completion signal per batch of data).
//
// Tokens form C contiguous chunks, each split into n tasks of a few tokens.
// A workgroup repeatedly takes the next ticket from one counter in HBM; the
// tickets enumerate, for the host-chosen chunk order o and a lag of L chunks,
//   D(o0) .. D(o_{L-1}),  D(o_L) C(o0),  D(o_{L+1}) C(o1),  ...,  C(o_{C-L}) .. C(o_{C-1})
// so a C task is claimed about L chunks after its D tasks.  L is the number of
// chunks the resident workgroups hold in flight at once: with a smaller lag a
// claimed C task would mostly wait on a chunk still being dispatched while
// holding a workgroup slot.  A D task writes its rows with device-coherent
// stores, waits for them to complete and adds one to its chunk's ready flag;
// a C task of chunk c polls that flag until it reaches n and reads the rows
// with device-coherent loads.  No L2 write-back or invalidate is needed (an
// agent-scope release/acquire pair would write back / invalidate a whole
// XCD's L2 per task).
// Every D task of chunk c has a smaller ticket than every C task of chunk c,
// and D tasks never wait, so each awaited task is already held by a running
// workgroup: the pipeline cannot deadlock whatever the grid size.  Waits are
// bounded by a clock limit; an expired wait records UBEP_ERR_TIMEOUT, sets a
// give-up word that ends every later wait at once, and moves on, so every
// workgroup always reaches the exit.  The last workgroup
// to leave resets the ticket and the flags for the next call.
#include "launch.h"
#include "rows.h"

namespace ubep {

constexpr int kChunkBlock = 256;
constexpr uint32_t kTicketBatch = 1;

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
    int32_t lag;        // chunks between a chunk's D tasks and its C tasks
    uint32_t total;     // 2 * C * n tickets
    uint64_t spin_ticks;
    uint32_t debug;
    int16_t order[kMaxC];
    const int32_t* dev_order;   // not null: the order in device memory (LPT policy)
};

// LPT chunk order (imbalance-aware: the pages balance completion time rather
// than counts).  On one GPU every chunk moves the same bytes, so a chunk's
// load is read as its largest per-destination row count,
//   load(c) = max over d of cd(c, d),  cd(c, d) = chunk_offset[c+1][d] - chunk_offset[c][d]
// (rank_count[d] - chunk_offset[C-1][d] for the last chunk), and chunks go in
// descending load, equal loads in ascending chunk id.  One workgroup: the
// threads sweep the C x R counts (LDS max per chunk), then each chunk's place
// is the number of chunks that precede it.
__global__ __launch_bounds__(256) void chunk_lpt_kernel(const int32_t* __restrict__ chunk_offset,
                                                        const int32_t* __restrict__ rank_count,
                                                        int32_t* __restrict__ order, int32_t C,
                                                        int32_t R) {
    __shared__ int32_t s_load[kMaxC];
    for (int32_t c = threadIdx.x; c < C; c += blockDim.x) s_load[c] = 0;
    __syncthreads();
    const int64_t n = (int64_t)C * R;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        const int32_t c = (int32_t)(i / R), d = (int32_t)(i - (int64_t)c * R);
        const int32_t lo = c == 0 ? 0 : chunk_offset[i];
        const int32_t hi = c + 1 < C ? chunk_offset[i + R] : rank_count[d];
        atomicMax(&s_load[c], hi - lo);
    }
    __syncthreads();
    for (int32_t c = threadIdx.x; c < C; c += blockDim.x) {
        const int32_t lc = s_load[c];
        int32_t place = 0;
        for (int32_t o = 0; o < C; ++o) {
            const int32_t lo_ = s_load[o];
            place += (lo_ > lc || (lo_ == lc && o < c)) ? 1 : 0;
        }
        order[place] = c;
    }
}

hipError_t launch_chunk_lpt(const Plan& p, const int32_t* chunk_offset, const int32_t* rank_count,
                            int32_t* order, hipStream_t stream) {
    return launch_kernel(chunk_lpt_kernel, dim3(1), dim3(256), 0, stream, chunk_offset, rank_count,
                         order, p.C, p.R);
}

template <int G, int VPT>
__global__ __launch_bounds__(kChunkBlock) void chunked_kernel(ChunkArgs a) {
    constexpr int TPB = kChunkBlock / G;
    __shared__ uint32_t s_ticket;
    __shared__ int16_t s_order[kMaxC];
    const int tid = threadIdx.x;
    const int gtid = tid % G;
    uint32_t* status = &a.hdr[kHdrStatus];
    for (int32_t i = tid; i < a.C; i += kChunkBlock)
        s_order[i] = a.dev_order != nullptr ? (int16_t)a.dev_order[i] : a.order[i];
    __syncthreads();

    // Tickets are claimed kTicketBatch at a time and processed in order; a C
    // task in a batch waits only on smaller tickets, held by running
    // workgroups or done earlier in the same batch.  (Measured: batches of 1
    // are fastest on both the decode and the large prefill shapes.)
    uint32_t next = 0, batch_end = 0;
    for (;;) {
        if (next == batch_end) {
            if (tid == 0) s_ticket = add_relaxed(&a.hdr[kHdrFusedTicket], kTicketBatch);
            __syncthreads();
            next = s_ticket;
            batch_end = next + kTicketBatch;
            __syncthreads();
        }
        const uint32_t ticket = next++;
        if (ticket >= a.total) break;

        // decode the ticket
        const uint32_t n = (uint32_t)a.n, L = (uint32_t)a.lag, C = (uint32_t)a.C;
        bool is_d;
        int32_t c;
        uint32_t idx;
        if (ticket < L * n) {                               // the first L chunks' D tasks
            is_d = true;
            c = s_order[ticket / n];
            idx = ticket % n;
        } else {
            const uint32_t u = ticket - L * n;
            const uint32_t pair = u / (2u * n);
            if (pair < C - L) {                             // D(o_{pair+L}) then C(o_pair)
                const uint32_t r = u % (2u * n);
                is_d = r < n;
                c = is_d ? s_order[pair + L] : s_order[pair];
                idx = is_d ? r : r - n;
            } else {                                        // the last L chunks' C tasks
                const uint32_t v = u - (C - L) * 2u * n;
                is_d = false;
                c = s_order[C - L + v / n];
                idx = v % n;
            }
        }
        const int64_t c_lo = (int64_t)c * a.tpc, c_hi = c_lo + a.tpc;
        const int64_t t_lo = c_lo + (int64_t)idx * a.tpt;
        const int64_t t_hi = t_lo + a.tpt < c_hi ? t_lo + a.tpt : c_hi;
        uint32_t* flag = a.flags + (int64_t)c * kFlagStride;

        if (is_d) {
            for (int64_t t = t_lo + tid / G; t < t_hi; t += TPB)
                dispatch_row_bf16<G, VPT, false, true>(a.x, a.pos, a.recv, t, a.k, a.nvec, a.n_rows,
                                                       gtid, status);
            wait_memory();             // every row of the task is at the coherent level
            __syncthreads();
            if ((a.debug & kDebugDelay) != 0u && idx % 3u == 0u) debug_delay();
            if (tid == 0 && (a.debug & kDebugWithhold) == 0u) add_relaxed(flag, 1u);
        } else {
            if (tid == 0) {
                const uint64_t t0 = now_ticks();
                while (ld_relaxed(flag) < n) {
                    if (now_ticks() - t0 > a.spin_ticks || ld_relaxed(&a.hdr[kHdrFusedGiveUp]) != 0u) {
                        st_relaxed(&a.hdr[kHdrFusedGiveUp], 1u);
                        raise_status(status, UBEP_ERR_TIMEOUT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            __syncthreads();
            for (int64_t t = t_lo + tid / G; t < t_hi; t += TPB)
                combine_row<G, VPT, 8, true, false>(a.recv, a.pos, a.w, a.out, t, a.k, a.nvec,
                                                    a.n_rows, gtid, status);
        }
    }

    if (tid == 0) {
        // every workgroup's final ticket claim returned before this increment
        const uint32_t done = add_relaxed(&a.hdr[kHdrFusedDone], 1u);
        if (done == gridDim.x - 1u) {
            for (int32_t c = 0; c < a.C; ++c) st_relaxed(a.flags + (int64_t)c * kFlagStride, 0u);
            st_relaxed(&a.hdr[kHdrFusedTicket], 0u);
            st_relaxed(&a.hdr[kHdrFusedGiveUp], 0u);
            st_relaxed(&a.hdr[kHdrFusedDone], 0u);
        }
    }
}

hipError_t launch_chunked(const Plan& p, const void* x, const int32_t* pos, const float* topk_w,
                          void* recv, void* out, const int32_t* chunk_order,
                          const int32_t* dev_order, uint64_t spin_ticks, uint32_t debug_flags,
                          void* ws, int device, hipStream_t stream) {
    const int64_t nvec = p.H / 8;
    int G, VPT;
    pick_group(nvec, &G, &VPT);
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
    // a task is one pass of the workgroup's token groups (2 tokens when a
    // group of 128 threads covers a row)
    const int64_t tpb = kChunkBlock / G;
    int64_t tpt = tpb;
    if (tpt > p.tpc) tpt = p.tpc;
    a.tpt = (int32_t)tpt;
    a.n = (int32_t)((p.tpc + tpt - 1) / tpt);
    a.total = (uint32_t)(2 * (int64_t)p.C * a.n);
    a.spin_ticks = spin_ticks;
    a.debug = debug_flags;
    for (int i = 0; i < kMaxC; ++i) a.order[i] = (int16_t)(i < p.C ? (chunk_order ? chunk_order[i] : i) : 0);
    a.dev_order = dev_order;
    DeviceInfo di;
    hipError_t e = device_info(device, &di);
    if (e != hipSuccess) return e;
    auto go = [&]<int GG, int VV>() -> hipError_t {
        int per_cu = 0;
        hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chunked_kernel<GG, VV>,
                                                                      kChunkBlock, 0);
        if (err != hipSuccess) return err;
        if (per_cu < 1) per_cu = 1;
        int64_t grid = (int64_t)di.cus * per_cu;
        if (grid > (int64_t)a.total) grid = a.total;
        // chunks in flight: every resident workgroup holds one batch of tasks
        const int64_t window = grid * (int64_t)kTicketBatch;
        int64_t lag = (window + a.n - 1) / a.n;
        a.lag = (int32_t)(lag < 1 ? 1 : (lag > a.C ? a.C : lag));
        return launch_kernel(chunked_kernel<GG, VV>, dim3((unsigned)grid), dim3(kChunkBlock), 0, stream,
                             a);
    };
    return with_group(G, VPT, go);
}

}  // namespace ubep

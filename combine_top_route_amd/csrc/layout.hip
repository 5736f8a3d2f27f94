// Dispatch layout on gfx950: token counting, prefix sums, offsets and stable
// reorder positions ("NJU x Huawei UBEP: Reengineering MoE Expert
// Parallelism", sections "BSP Serialization" and "Kernel Decomposition").
//
// Rows (t, j) are cut into tiles of whole tokens.  Two kernels:
//
//  1. layout_scan: each workgroup takes the next tile from a ticket counter,
//     builds the tile's per-rank histogram (one per wave) and per-expert
//     histogram in LDS with wave ballots (one LDS update per distinct key per
//     wave, so hot ranks under skew cost no more than cold ones), publishes
//     the tile aggregate, and walks back over earlier tiles' published state
//     (decoupled look-back) to get, for every rank, the rows that earlier
//     tiles send there.  Tiles are handed out in order, so every tile it
//     waits on is already held by a running workgroup that publishes without
//     waiting: no grid-wide barrier and no co-residency assumption.  The last
//     tile's inclusive prefix is the per-rank total; that workgroup writes
//     rank_count and recv_offset.  Because a tile never straddles a source
//     rank or chunk boundary, a tile's exclusive prefix at such a boundary is
//     a row of send_offset / chunk_offset.
//  2. layout_positions: each tile re-reads its expert ids and ranks its rows
//     stably (wave ballot peer masks give the order among equal ranks inside
//     the wave; per-wave bases give the order across waves), adds
//     recv_offset + the tile prefix, and writes pos and recv_src.  It also
//     sums the per-tile expert histograms and clears the look-back state for
//     the next call.
#include "device_common.h"
#include "launch.h"

namespace ubep {

struct LayoutArgs {
    const int32_t* idx;
    int32_t* pos;
    int32_t* expert_count;
    int32_t* rank_count;
    int32_t* recv_offset;
    int32_t* send_offset;
    int32_t* chunk_offset;   // may be null
    int32_t* recv_src;       // may be null
    uint32_t* hdr;
    uint32_t* state;
    int32_t* excl;
    int32_t* wbase;
    int32_t* ehist;
    Plan p;
    uint64_t spin_ticks;
};

// Exclusive scan over the 256 threads of a workgroup; `s_tmp` holds 4 ints.
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* s_tmp, int32_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int32_t inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(inc, o, 64);
        if (lane >= o) inc += u;
    }
    if (lane == 63) s_tmp[w] = inc;
    __syncthreads();
    int32_t before = 0;
    for (int i = 0; i < w; ++i) before += s_tmp[i];
    *total = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
    __syncthreads();
    return before + inc - v;
}

__device__ __forceinline__ int32_t load_expert(const int32_t* idx, int64_t row, bool act,
                                               int32_t E, bool* bad) {
    int32_t e = act ? idx[row] : 0;
    if (act && (uint32_t)e >= (uint32_t)E) {
        *bad = true;
        e = 0;
    }
    return e;
}

__global__ __launch_bounds__(kLayoutThreads) void layout_scan_kernel(LayoutArgs a) {
    __shared__ int32_t s_wh[kLayoutWaves * kMaxR];   // per-wave rank histograms
    __shared__ int32_t s_eh[kMaxE];                  // tile expert histogram
    __shared__ int32_t s_tot[kMaxR];                 // per-rank totals (last tile only)
    __shared__ int32_t s_tmp[4];
    __shared__ uint32_t s_tile;

    const Plan& p = a.p;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int32_t R = p.R, E = p.E;

    if (tid == 0) s_tile = add_relaxed(&a.hdr[kHdrLayoutTicket], 1u);
    for (int i = tid; i < kLayoutWaves * R; i += kLayoutThreads) s_wh[i] = 0;
    for (int i = tid; i < E; i += kLayoutThreads) s_eh[i] = 0;
    __syncthreads();
    const int64_t tile = s_tile;
    if (tile >= p.n_tiles) {   // ticket counter not cleared: workspace was never initialised
        if (tid == 0) raise_status(&a.hdr[kHdrStatus], UBEP_ERR_INVALID_ARG);
        return;
    }
    const int64_t row0 = tile * p.tile_rows;

    // ---- histograms: wave w owns rows [lo, hi) of the tile
    const int64_t per_wave = (p.tile_rows + kLayoutWaves - 1) / kLayoutWaves;
    const int64_t lo = w * per_wave;
    const int64_t hi = lo + per_wave < p.tile_rows ? lo + per_wave : p.tile_rows;
    bool bad = false;
    for (int64_t base = lo; base < hi; base += 64) {
        const int64_t r = base + lane;
        const bool act = r < hi;
        const int32_t e = load_expert(a.idx, row0 + r, act, E, &bad);
        const uint32_t d = (uint32_t)e / (uint32_t)p.epr;
        const uint64_t am = __ballot(act);
        const uint64_t pd = peers_of(d, p.dbits, am);
        if (act && (pd & lanemask_lt()) == 0) s_wh[w * R + d] += __popcll(pd);
        const uint64_t pe = peers_of((uint32_t)e, p.ebits, am);
        if (act && (pe & lanemask_lt()) == 0) atomicAdd(&s_eh[e], (int32_t)__popcll(pe));
    }
    if (bad) raise_status(&a.hdr[kHdrStatus], UBEP_ERR_BAD_EXPERT_ID);
    __syncthreads();

    // ---- publish, look back, record offsets (one thread per rank)
    const int64_t tok0 = tile * p.tile_tokens;
    for (int32_t d = tid; d < R; d += kLayoutThreads) {
        const int32_t a0 = s_wh[d], a1 = s_wh[R + d], a2 = s_wh[2 * R + d], a3 = s_wh[3 * R + d];
        int32_t* wb = a.wbase + tile * kLayoutWaves * R;
        wb[d] = 0;
        wb[R + d] = a0;
        wb[2 * R + d] = a0 + a1;
        wb[3 * R + d] = a0 + a1 + a2;
        const int32_t agg = a0 + a1 + a2 + a3;
        uint32_t* st = a.state + tile * R + d;
        int32_t excl = 0;
        if (tile == 0) {
            st_relaxed(st, kFlagInclusive | (uint32_t)agg);
        } else {
            st_relaxed(st, kFlagAggregate | (uint32_t)agg);
            int64_t j = tile - 1;
            const uint64_t t0 = now_ticks();
            for (;;) {
                const uint32_t v = ld_relaxed(a.state + j * R + d);
                const uint32_t f = v & ~kCountMask;
                if (f == 0u) {
                    if (now_ticks() - t0 > a.spin_ticks) {
                        raise_status(&a.hdr[kHdrStatus], UBEP_ERR_TIMEOUT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                    continue;
                }
                excl += (int32_t)(v & kCountMask);
                if (f == kFlagInclusive || j == 0) break;
                --j;
            }
            st_relaxed(st, kFlagInclusive | (uint32_t)(excl + agg));
        }
        a.excl[tile * R + d] = excl;
        s_tot[d] = excl + agg;
        if (tok0 % p.tps == 0) a.send_offset[(tok0 / p.tps) * R + d] = excl;
        if (a.chunk_offset != nullptr && tok0 % p.tpc == 0)
            a.chunk_offset[(tok0 / p.tpc) * R + d] = excl;
    }
    for (int32_t e = tid; e < E; e += kLayoutThreads) a.ehist[tile * E + e] = s_eh[e];

    // ---- the last tile holds the per-rank totals: rank_count, recv_offset
    if (tile == p.n_tiles - 1) {
        __syncthreads();
        // thread i owns ranks [i*per, (i+1)*per)
        const int per = (R + kLayoutThreads - 1) / kLayoutThreads;
        int32_t mine = 0;
        for (int i = 0; i < per; ++i) {
            const int32_t d = tid * per + i;
            if (d < R) mine += s_tot[d];
        }
        int32_t total;
        int32_t run = block_exclusive_scan(mine, s_tmp, &total);
        for (int i = 0; i < per; ++i) {
            const int32_t d = tid * per + i;
            if (d < R) {
                a.rank_count[d] = s_tot[d];
                a.recv_offset[d] = run;
                run += s_tot[d];
            }
        }
        if (tid == 0) a.recv_offset[R] = total;
    }
}

__global__ __launch_bounds__(kLayoutThreads) void layout_positions_kernel(LayoutArgs a) {
    __shared__ int32_t s_base[kLayoutWaves * kMaxR];

    const Plan& p = a.p;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int32_t R = p.R, E = p.E;
    const int64_t tile = blockIdx.x;
    const int64_t row0 = tile * p.tile_rows;

    for (int i = tid; i < kLayoutWaves * R; i += kLayoutThreads) {
        const int32_t d = i % R;
        s_base[i] = a.recv_offset[d] + a.excl[tile * R + d] + a.wbase[tile * kLayoutWaves * R + i];
    }
    __syncthreads();

    const int64_t per_wave = (p.tile_rows + kLayoutWaves - 1) / kLayoutWaves;
    const int64_t lo = w * per_wave;
    const int64_t hi = lo + per_wave < p.tile_rows ? lo + per_wave : p.tile_rows;
    bool bad = false, bad_pos = false;
    for (int64_t base = lo; base < hi; base += 64) {
        const int64_t r = base + lane;
        const bool act = r < hi;
        const int32_t e = load_expert(a.idx, row0 + r, act, E, &bad);
        const uint32_t d = (uint32_t)e / (uint32_t)p.epr;
        const uint64_t pd = peers_of(d, p.dbits, __ballot(act));
        const uint64_t before = pd & lanemask_lt();
        if (act) {
            const int32_t b = s_base[w * R + d];
            const int32_t q = b + (int32_t)__popcll(before);
            a.pos[row0 + r] = q;
            // q is in range whenever the scan completed; guard the scatter anyway
            if ((uint64_t)(int64_t)q < (uint64_t)p.rows) {
                if (a.recv_src != nullptr) a.recv_src[q] = (int32_t)(row0 + r);
            } else {
                bad_pos = true;
            }
            if (before == 0) s_base[w * R + d] = b + (int32_t)__popcll(pd);
        }
    }

    if (bad_pos) raise_status(&a.hdr[kHdrStatus], UBEP_ERR_BAD_POSITION);

    // expert totals: sum of the per-tile histograms
    for (int64_t e = (int64_t)blockIdx.x * kLayoutThreads + tid; e < E;
         e += (int64_t)gridDim.x * kLayoutThreads) {
        int32_t s = 0;
        for (int64_t t = 0; t < p.n_tiles; ++t) s += a.ehist[t * E + e];
        a.expert_count[e] = s;
    }
    // clear this tile's look-back state and the ticket for the next call
    for (int32_t d = tid; d < R; d += kLayoutThreads) st_relaxed(a.state + tile * R + d, 0u);
    if (tile == 0 && tid == 0) st_relaxed(&a.hdr[kHdrLayoutTicket], 0u);
}

hipError_t launch_layout(const Plan& p, const int32_t* idx, int32_t* pos, int32_t* expert_count,
                         int32_t* rank_count, int32_t* recv_offset, int32_t* send_offset,
                         int32_t* chunk_offset, int32_t* recv_src, void* ws, uint64_t spin_ticks,
                         hipStream_t stream) {
    LayoutArgs a;
    a.idx = idx;
    a.pos = pos;
    a.expert_count = expert_count;
    a.rank_count = rank_count;
    a.recv_offset = recv_offset;
    a.send_offset = send_offset;
    a.chunk_offset = p.C > 1 ? chunk_offset : nullptr;
    a.recv_src = recv_src;
    char* base = static_cast<char*>(ws);
    a.hdr = reinterpret_cast<uint32_t*>(base);
    a.state = reinterpret_cast<uint32_t*>(base + p.off_state);
    a.excl = reinterpret_cast<int32_t*>(base + p.off_excl);
    a.wbase = reinterpret_cast<int32_t*>(base + p.off_wbase);
    a.ehist = reinterpret_cast<int32_t*>(base + p.off_ehist);
    a.p = p;
    a.spin_ticks = spin_ticks;
    hipLaunchKernelGGL(layout_scan_kernel, dim3((unsigned)p.n_tiles), dim3(kLayoutThreads), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(layout_positions_kernel, dim3((unsigned)p.n_tiles), dim3(kLayoutThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace ubep

// Dispatch layout on gfx950: token counting, prefix sums, offsets and stable
// reorder positions ("NJU x Huawei UBEP: Reengineering MoE Expert
// Parallelism", sections "BSP Serialization" and "Kernel Decomposition").
//
// One persistent kernel, with no memory fences: every value one workgroup
// passes to another travels inside a self-contained 64-bit state word
// (call epoch | flag | count) written and read with agent-scope atomics.
// Rows (t, j) are cut into tiles of whole tokens; a tile never straddles a
// source-rank or chunk boundary.  Each tile has R + E "digits": one per
// destination rank and one per expert.
//
// Phase A -- each workgroup takes tiles from a ticket counter, in order:
//   * each wave loads all of its ids in one burst, then builds per-wave rank
//     counts and the tile's expert counts in LDS with wave ballots (one LDS
//     update per distinct key per wave, so a hot rank under skewed routing
//     costs no more than a cold one);
//   * publishes the tile's per-digit aggregate, then looks back over earlier
//     tiles' published words, 32 predecessors per round (decoupled look-back),
//     and publishes the inclusive count.  Tiles are handed out in order, so
//     every awaited tile is held by a running workgroup that publishes its
//     aggregate without waiting: no grid barrier, no co-residency assumption;
//   * a tile's exclusive prefix at a source-rank / chunk boundary is a row of
//     send_offset / chunk_offset.
// Phase B -- after the ticket counter runs dry, each workgroup waits for the
//   last tile's inclusive words (the totals; everything awaited is already
//   claimed), scans the rank totals into recv_offset, and re-ranks its own
//   tiles stably (ballot peer masks inside a wave, per-wave bases across
//   waves) to write pos / recv_src.  Workgroup 0 also writes the expert
//   totals.  Words of an older epoch read as "not yet published", so nothing
//   is cleared between calls; the last workgroup out resets the ticket and
//   advances the epoch.
//
// Small problems (the decode shapes) take a one-workgroup kernel instead:
// 16 waves own contiguous runs of tiles, keep their ids in registers, and do
// the tile counts, the prefix sums over tiles and ranks, and the ranking in
// LDS.  With no value crossing workgroups it avoids the device-memory round
// trips (ticket, publish, look-back, totals) that bound the persistent
// kernel's latency.
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
    uint64_t* state;         // [n_tiles][R + E]
    int32_t* excl;           // [n_tiles][R]
    int32_t* wbase;          // [n_tiles][4][R]
    Plan p;
    uint64_t spin_ticks;
};

// Rows of the tile owned by wave w: [lo, hi), at most kRowsPerLane * 64.
__device__ __forceinline__ void wave_rows(const Plan& p, int w, int64_t* lo, int64_t* hi) {
    const int64_t per_wave = (p.tile_rows + kLayoutWaves - 1) / kLayoutWaves;
    *lo = w * per_wave;
    *hi = *lo + per_wave < p.tile_rows ? *lo + per_wave : p.tile_rows;
}

// Load the wave's expert ids in one burst: ev[i] holds row lo + 64 i + lane
// (loads are unconditional, from clamped rows, so all are in flight at once;
// entries past the wave's rows are unused).  Ids outside [0, E) are reported
// and treated as expert 0.
__device__ __forceinline__ void load_ids(const LayoutArgs& a, int64_t tile, int32_t (&ev)[kRowsPerLane]) {
    const Plan& p = a.p;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int64_t lo, hi;
    wave_rows(p, w, &lo, &hi);
    const int32_t* src = a.idx + tile * p.tile_rows;
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
        const int64_t r = lo + 64 * i + lane;
        ev[i] = src[r < p.tile_rows ? r : p.tile_rows - 1];
    }
}

__device__ __forceinline__ void check_ids(const Plan& p, int32_t (&ev)[kRowsPerLane], bool* bad) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int64_t lo, hi;
    wave_rows(p, w, &lo, &hi);
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
        if ((uint32_t)ev[i] >= (uint32_t)p.E) {
            if (lo + 64 * i + lane < hi) *bad = true;
            ev[i] = 0;
        }
    }
}

// s_wh[w*R + d] = rows of wave w with rank d; s_eh[e] = rows of the tile with
// expert e.  Counting needs no order, so plain LDS atomics do it (a hot key
// under skew only serialises its own lanes).
__device__ __forceinline__ void tile_histograms(const Plan& p, const int32_t (&ev)[kRowsPerLane],
                                                int32_t* s_wh, int32_t* s_eh) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int64_t lo, hi;
    wave_rows(p, w, &lo, &hi);
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
        if (lo + 64 * i >= hi) break;                      // uniform across the wave
        if (lo + 64 * i + lane < hi) {
            const uint32_t e = (uint32_t)ev[i];
            atomicAdd(&s_wh[w * p.R + rank_of(e, p.epr_magic)], 1);
            atomicAdd(&s_eh[e], 1);
        }
    }
}

// Stable ranking inside a tile: s_base[w*R + d] holds the value of wave w's
// first row with rank d; every row gets s_base + (rows before it in the wave
// with rank d), and s_base advances.  Ballot peer masks give the order among
// equal ranks inside a 64-row step; steps run in row order.
__device__ __forceinline__ void tile_ranks(const Plan& p, const int32_t (&ev)[kRowsPerLane],
                                           int32_t* s_base, int32_t (&rank)[kRowsPerLane]) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int64_t lo, hi;
    wave_rows(p, w, &lo, &hi);
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
        rank[i] = 0;
        if (lo + 64 * i >= hi) continue;                   // uniform across the wave
        const bool act = lo + 64 * i + lane < hi;
        const uint32_t d = rank_of((uint32_t)ev[i], p.epr_magic);
        const uint64_t pd = peers_of_n<10>(d, p.dbits, __ballot(act));
        const uint64_t before = pd & lanemask_lt();
        if (act) {
            const int32_t b = s_base[w * p.R + d];
            rank[i] = b + (int32_t)__popcll(before);
            if (before == 0) s_base[w * p.R + d] = b + (int32_t)__popcll(pd);
        }
    }
}

// pos (and recv_src) of the tile's rows from their receive rows.
__device__ __forceinline__ void store_positions(const LayoutArgs& a, int64_t tile,
                                                const int32_t (&q)[kRowsPerLane], bool* bad_pos) {
    const Plan& p = a.p;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row0 = tile * p.tile_rows;
    int64_t lo, hi;
    wave_rows(p, w, &lo, &hi);
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
        const int64_t r = lo + 64 * i + lane;
        if (r >= hi) continue;
        a.pos[row0 + r] = q[i];
        // q is in range whenever the scan completed; guard the scatter anyway
        if ((uint32_t)q[i] < (uint32_t)p.rows) {
            if (a.recv_src != nullptr) a.recv_src[q[i]] = (int32_t)(row0 + r);
        } else {
            *bad_pos = true;
        }
    }
}

__device__ __forceinline__ uint64_t state_word(uint32_t epoch, uint32_t flag, int32_t count) {
    return ((uint64_t)epoch << 32) | flag | (uint32_t)count;
}

// Count of digit `slot` in tiles before `tile`: walk back over published
// words, a window of predecessors per round, adding aggregates until an
// inclusive count is found.  A predecessor that has not published yet stalls
// the walk at that point until it does (bounded by spin_ticks).
__device__ __forceinline__ int32_t look_back(const LayoutArgs& a, int64_t tile, int32_t slot,
                                             uint32_t epoch, bool* timed_out) {
    const int32_t S = a.p.slots;
    int32_t excl = 0;
    int64_t j = tile - 1;
    const uint64_t t0 = now_ticks();
    while (j >= 0) {
        uint64_t v[kLookbackWindow];
#pragma unroll
        for (int i = 0; i < kLookbackWindow; ++i)
            v[i] = (j - i >= 0) ? ld_relaxed64(a.state + (j - i) * S + slot) : 0ull;
        int consumed = 0;
        bool done = false, stall = false;
#pragma unroll
        for (int i = 0; i < kLookbackWindow; ++i) {
            if (done || stall) continue;
            if (j - i < 0) {
                done = true;
                continue;
            }
            const uint32_t tag = (uint32_t)(v[i] >> 32), lo = (uint32_t)v[i];
            const uint32_t f = lo & ~kCountMask;
            if (tag != epoch || f == 0u) {
                stall = true;
                continue;
            }
            excl += (int32_t)(lo & kCountMask);
            consumed = i + 1;
            if (f == kFlagInclusive) done = true;
        }
        j -= consumed;
        if (done) break;
        if (stall) {
            if (now_ticks() - t0 > a.spin_ticks) {
                *timed_out = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    return excl;
}

// Wait for the inclusive word of digit `slot` of the last tile.
__device__ __forceinline__ int32_t wait_total(const LayoutArgs& a, int32_t slot, uint32_t epoch,
                                              bool* timed_out) {
    const uint64_t* w = a.state + (a.p.n_tiles - 1) * a.p.slots + slot;
    const uint64_t t0 = now_ticks();
    for (;;) {
        const uint64_t v = ld_relaxed64(w);
        if ((uint32_t)(v >> 32) == epoch && ((uint32_t)v & ~kCountMask) == kFlagInclusive)
            return (int32_t)((uint32_t)v & kCountMask);
        if (now_ticks() - t0 > a.spin_ticks) {
            *timed_out = true;
            return 0;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

__global__ __launch_bounds__(kLayoutThreads) void layout_kernel(LayoutArgs a) {
    __shared__ int32_t s_wh[kLayoutWaves * kMaxR];   // per-wave rank counts, then running bases
    __shared__ int32_t s_eh[kMaxE];                  // tile expert counts
    __shared__ int32_t s_cnt[kMaxR];                 // tile rank counts, then rank totals
    __shared__ int32_t s_excl[kMaxR];                // rows to rank d before the last claimed tile
    __shared__ int32_t s_off[kMaxR];                 // recv_offset
    __shared__ uint32_t s_tiles[kMaxTilesPerGroup];
    __shared__ int32_t s_tmp[kLayoutWaves];
    __shared__ uint32_t s_ticket;

    const Plan& p = a.p;
    const int tid = threadIdx.x;
    const int32_t R = p.R, E = p.E, S = p.slots;
    const uint32_t epoch = ld_relaxed(&a.hdr[kHdrLayoutEpoch]);
    bool bad = false, bad_pos = false, timed_out = false;
    uint32_t n_mine = 0;
    int32_t ev[kRowsPerLane];                        // ids of the last claimed tile
    int32_t lrank[kRowsPerLane];                     // their ranks inside the tile

    // ---------------- phase A: counts, in-tile ranks and look-back, tile by tile
    // (grid * kMaxTilesPerGroup >= n_tiles; a full tile list stops claiming)
    for (;;) {
        if (n_mine >= (uint32_t)kMaxTilesPerGroup) break;
        if (tid == 0) s_ticket = add_relaxed(&a.hdr[kHdrLayoutTicket], 1u);
        // the first ticket is usually blockIdx.x: fetch that tile's ids while
        // the ticket is in flight, refetch below if the guess was wrong
        const uint32_t guess = blockIdx.x + n_mine * gridDim.x;
        int32_t nv[kRowsPerLane];
        if (guess < (uint64_t)p.n_tiles) load_ids(a, guess, nv);
        for (int i = tid; i < kLayoutWaves * R; i += kLayoutThreads) s_wh[i] = 0;
        for (int i = tid; i < E; i += kLayoutThreads) s_eh[i] = 0;
        __syncthreads();
        const uint32_t tile = s_ticket;
        if (tile >= (uint64_t)p.n_tiles) break;
        if (tile != guess) load_ids(a, tile, nv);
#pragma unroll
        for (int i = 0; i < kRowsPerLane; ++i) ev[i] = nv[i];
        check_ids(p, ev, &bad);
        if (tid == 0) s_tiles[n_mine] = tile;
        ++n_mine;
        tile_histograms(p, ev, s_wh, s_eh);
        __syncthreads();

        // wave bases (kept for a later re-rank), tile aggregates, publish
        int32_t* wb = a.wbase + (int64_t)tile * kLayoutWaves * R;
        for (int32_t d = tid; d < R; d += kLayoutThreads) {
            int32_t run = 0;
#pragma unroll
            for (int v = 0; v < kLayoutWaves; ++v) {
                const int32_t c = s_wh[v * R + d];
                s_wh[v * R + d] = run;
                wb[v * R + d] = run;
                run += c;
            }
            s_cnt[d] = run;
        }
        __syncthreads();
        uint64_t* st = a.state + (int64_t)tile * S;
        for (int32_t s = tid; s < S; s += kLayoutThreads) {
            const int32_t c = s < R ? s_cnt[s] : s_eh[s - R];
            st_relaxed64(st + s, state_word(epoch, tile == 0 ? kFlagInclusive : kFlagAggregate, c));
        }
        // in-tile ranks now, while predecessors publish
        tile_ranks(p, ev, s_wh, lrank);
        const int64_t tok0 = (int64_t)tile * p.tile_tokens;
        for (int32_t s = tid; s < S; s += kLayoutThreads) {
            const int32_t c = s < R ? s_cnt[s] : s_eh[s - R];
            const int32_t excl = tile == 0 ? 0 : look_back(a, tile, s, epoch, &timed_out);
            if (tile != 0) st_relaxed64(st + s, state_word(epoch, kFlagInclusive, excl + c));
            if (s < R) {
                s_excl[s] = excl;
                a.excl[(int64_t)tile * R + s] = excl;
                if (tok0 % p.tps == 0) a.send_offset[(tok0 / p.tps) * R + s] = excl;
                if (a.chunk_offset != nullptr && tok0 % p.tpc == 0)
                    a.chunk_offset[(tok0 / p.tpc) * R + s] = excl;
            }
        }
        __syncthreads();
    }

    // ---------------- phase B: totals, recv_offset, positions
    for (int32_t d = tid; d < R; d += kLayoutThreads) s_cnt[d] = wait_total(a, d, epoch, &timed_out);
    if (blockIdx.x == 0)
        for (int32_t e = tid; e < E; e += kLayoutThreads)
            a.expert_count[e] = wait_total(a, R + e, epoch, &timed_out);
    __syncthreads();
    {   // exclusive scan of the rank totals; thread i owns a run of ranks
        const int per = (R + kLayoutThreads - 1) / kLayoutThreads;
        int32_t mine = 0;
        for (int i = 0; i < per; ++i) {
            const int32_t d = tid * per + i;
            if (d < R) mine += s_cnt[d];
        }
        const int lane = tid & 63, w = tid >> 6;
        int32_t inc = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t u = __shfl_up(inc, o, 64);
            if (lane >= o) inc += u;
        }
        if (lane == 63) s_tmp[w] = inc;
        __syncthreads();
        int32_t run = inc - mine;
        for (int i = 0; i < w; ++i) run += s_tmp[i];
        for (int i = 0; i < per; ++i) {
            const int32_t d = tid * per + i;
            if (d < R) {
                s_off[d] = run;
                run += s_cnt[d];
            }
        }
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int32_t d = tid; d < R; d += kLayoutThreads) {
            a.rank_count[d] = s_cnt[d];
            a.recv_offset[d] = s_off[d];
        }
        if (tid == 0) a.recv_offset[R] = s_off[R - 1] + s_cnt[R - 1];
    }
    for (uint32_t m = 0; m < n_mine; ++m) {
        const int64_t tile = s_tiles[m];
        int32_t q[kRowsPerLane];
        if (m + 1 == n_mine) {     // the last claimed tile: ids and in-tile ranks in registers
#pragma unroll
            for (int i = 0; i < kRowsPerLane; ++i) {
                const uint32_t d = rank_of((uint32_t)ev[i], p.epr_magic);
                q[i] = s_off[d] + s_excl[d] + lrank[i];
            }
        } else {                   // an earlier tile of this workgroup: rebuild from its state
            int32_t ids[kRowsPerLane];
            load_ids(a, tile, ids);
            bool ignore = false;
            check_ids(p, ids, &ignore);
            __syncthreads();
            for (int i = tid; i < kLayoutWaves * R; i += kLayoutThreads) {
                const int32_t d = i % R;
                s_wh[i] = s_off[d] + a.excl[tile * R + d] + a.wbase[tile * kLayoutWaves * R + i];
            }
            __syncthreads();
            tile_ranks(p, ids, s_wh, q);
        }
        store_positions(a, tile, q, &bad_pos);
    }

    if (bad) raise_status(&a.hdr[kHdrStatus], UBEP_ERR_BAD_EXPERT_ID);
    if (timed_out) raise_status(&a.hdr[kHdrStatus], UBEP_ERR_TIMEOUT);
    if (bad_pos) raise_status(&a.hdr[kHdrStatus], UBEP_ERR_BAD_POSITION);

    // The last workgroup out resets the ticket and advances the epoch.  Every
    // workgroup's final ticket claim returned before its increment below.
    __syncthreads();
    if (tid == 0) {
        const uint32_t done = add_relaxed(&a.hdr[kHdrLayoutDone], 1u);
        if (done == gridDim.x - 1u) {
            st_relaxed(&a.hdr[kHdrLayoutTicket], 0u);
            st_relaxed(&a.hdr[kHdrLayoutDone], 0u);
            st_relaxed(&a.hdr[kHdrLayoutEpoch], epoch + 1u);
        }
    }
}

// ---------------------------------------------------------------- one-workgroup layout
constexpr int kSingleThreads = 1024;
constexpr int kSingleWaves = kSingleThreads / 64;
constexpr int kSingleSteps = 64;                 // 64-row steps a wave may own
constexpr int64_t kSingleMaxRows = (int64_t)kSingleWaves * kSingleSteps * 64;
constexpr int kSingleMaxR = 256;
constexpr int kSingleMaxE = 4096;
constexpr int kSingleMaxTiles = 256;
constexpr int kSingleMaxTileCounts = 8192;       // n_tiles * R

// Only tiny problems: above a few thousand rows one CU's ballot and LDS work
// costs more than the persistent kernel's memory round trips.
constexpr int64_t kSingleUseRows = 4096;

bool layout_fits_one_group(const Plan& p) {
    const int64_t tiles_per_wave = (p.n_tiles + kSingleWaves - 1) / kSingleWaves;
    return p.rows <= kSingleUseRows && p.rows <= kSingleMaxRows && p.tile_rows % 64 == 0 && p.n_tiles <= kSingleMaxTiles &&
           p.n_tiles * p.R <= kSingleMaxTileCounts && p.R <= kSingleMaxR && p.E <= kSingleMaxE &&
           tiles_per_wave * p.tile_rows <= (int64_t)kSingleSteps * 64;
}

template <int STEPS>
__global__ __launch_bounds__(kSingleThreads) void layout_single_kernel(LayoutArgs a) {
    __shared__ int32_t s_tc[kSingleMaxTileCounts];  // [tile][rank]: counts, then row bases
    __shared__ int32_t s_eh[kSingleMaxE];           // expert counts
    __shared__ int32_t s_tot[kSingleMaxR];          // rank totals
    __shared__ int32_t s_off[kSingleMaxR];          // recv_offset
    __shared__ int32_t s_tmp[kSingleWaves];

    const Plan& p = a.p;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int32_t R = p.R, E = p.E;
    for (int i = tid; i < p.n_tiles * R; i += kSingleThreads) s_tc[i] = 0;
    for (int i = tid; i < E; i += kSingleThreads) s_eh[i] = 0;

    // wave w owns tiles [t_lo, t_hi): rows [r_lo, r_lo + 64 steps)
    const int32_t tpw = (int32_t)((p.n_tiles + kSingleWaves - 1) / kSingleWaves);
    const int32_t n_tiles = (int32_t)p.n_tiles;
    const int32_t t_lo = w * tpw < n_tiles ? w * tpw : n_tiles;
    const int32_t t_hi = t_lo + tpw < n_tiles ? t_lo + tpw : n_tiles;
    const int32_t steps_per_tile = (int32_t)(p.tile_rows / 64);
    const int32_t steps = (t_hi - t_lo) * steps_per_tile;
    const int64_t r_lo = (int64_t)t_lo * p.tile_rows;
    int32_t ev[STEPS];
    bool bad = false, bad_pos = false;
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
        // unconditional loads from clamped (always valid) rows, so that all of
        // them are in flight together; steps past the wave's rows are unused
        const int64_t r = r_lo + 64 * i + lane;
        ev[i] = a.idx[r < p.rows ? r : p.rows - 1];
    }
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
        if ((uint32_t)ev[i] >= (uint32_t)E) {
            if (i < steps) bad = true;
            ev[i] = 0;
        }
    }
    __syncthreads();

    // pass 1: per-tile rank counts and expert counts (order-free: LDS atomics)
    {
        int32_t tile = t_lo, in_tile = 0;
#pragma unroll
        for (int i = 0; i < STEPS; ++i) {
            if (i >= steps) break;                           // uniform across the wave
            const uint32_t e = (uint32_t)ev[i];
            atomicAdd(&s_tc[tile * R + rank_of(e, p.epr_magic)], 1);
            atomicAdd(&s_eh[e], 1);
            if (++in_tile == steps_per_tile) {
                in_tile = 0;
                ++tile;
            }
        }
    }
    __syncthreads();

    // exclusive prefix over tiles for every rank; the totals
    for (int32_t d = tid; d < R; d += kSingleThreads) {
        int32_t run = 0;
        for (int32_t t = 0; t < n_tiles; ++t) {
            const int32_t c = s_tc[t * R + d];
            s_tc[t * R + d] = run;
            run += c;
        }
        s_tot[d] = run;
    }
    __syncthreads();
    {   // exclusive scan of the totals over ranks (R <= 1024: one rank per thread)
        const int32_t mine = tid < R ? s_tot[tid] : 0;
        int32_t inc = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t u = __shfl_up(inc, o, 64);
            if (lane >= o) inc += u;
        }
        if (lane == 63) s_tmp[tid >> 6] = inc;
        __syncthreads();
        int32_t before = 0;
        for (int i = 0; i < (tid >> 6); ++i) before += s_tmp[i];
        if (tid < R) s_off[tid] = before + inc - mine;
    }
    __syncthreads();
    for (int32_t d = tid; d < R; d += kSingleThreads) {
        a.rank_count[d] = s_tot[d];
        a.recv_offset[d] = s_off[d];
    }
    if (tid == 0) a.recv_offset[R] = (int32_t)p.rows;
    for (int32_t e = tid; e < E; e += kSingleThreads) a.expert_count[e] = s_eh[e];
    // send / chunk offsets are the tile prefixes at source-rank / chunk boundaries
    const int32_t tiles_per_source = (int32_t)(p.tps / p.tile_tokens);
    const int32_t tiles_per_chunk = (int32_t)(p.tpc / p.tile_tokens);
    for (int32_t i = tid; i < R * R; i += kSingleThreads)
        a.send_offset[i] = s_tc[(i / R) * tiles_per_source * R + i % R];
    if (a.chunk_offset != nullptr)
        for (int32_t i = tid; i < p.C * R; i += kSingleThreads)
            a.chunk_offset[i] = s_tc[(i / R) * tiles_per_chunk * R + i % R];
    __syncthreads();
    for (int32_t i = tid; i < n_tiles * R; i += kSingleThreads) s_tc[i] += s_off[i % R];
    __syncthreads();

    // pass 2: stable ranks -> positions (ballot peer masks give the order
    // among equal ranks inside a step; steps run in row order)
    {
        int32_t tile = t_lo, in_tile = 0;
#pragma unroll
        for (int i = 0; i < STEPS; ++i) {
            if (i >= steps) break;                           // uniform across the wave
            const int64_t row = r_lo + 64 * i + lane;
            const uint32_t d = rank_of((uint32_t)ev[i], p.epr_magic);
            const uint64_t pd = peers_of_n<8>(d, p.dbits, ~0ull);
            const uint64_t before = pd & lanemask_lt();
            const int32_t b = s_tc[tile * R + d];
            const int32_t q = b + (int32_t)__popcll(before);
            a.pos[row] = q;
            if ((uint32_t)q < (uint32_t)p.rows) {
                if (a.recv_src != nullptr) a.recv_src[q] = (int32_t)row;
            } else {
                bad_pos = true;
            }
            if (before == 0) s_tc[tile * R + d] = b + (int32_t)__popcll(pd);
            if (++in_tile == steps_per_tile) {
                in_tile = 0;
                ++tile;
            }
        }
    }
    if (bad) raise_status(&a.hdr[kHdrStatus], UBEP_ERR_BAD_EXPERT_ID);
    if (bad_pos) raise_status(&a.hdr[kHdrStatus], UBEP_ERR_BAD_POSITION);
}

hipError_t launch_layout(const Plan& p, const int32_t* idx, int32_t* pos, int32_t* expert_count,
                         int32_t* rank_count, int32_t* recv_offset, int32_t* send_offset,
                         int32_t* chunk_offset, int32_t* recv_src, void* ws, uint64_t spin_ticks,
                         hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    DeviceInfo di;
    e = device_info(dev, &di);
    if (e != hipSuccess) return e;
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
    a.state = reinterpret_cast<uint64_t*>(base + p.off_state);
    a.excl = reinterpret_cast<int32_t*>(base + p.off_excl);
    a.wbase = reinterpret_cast<int32_t*>(base + p.off_wbase);
    a.p = p;
    a.spin_ticks = spin_ticks;
    if (layout_fits_one_group(p)) {
        const int64_t tpw = (p.n_tiles + kSingleWaves - 1) / kSingleWaves;
        const int64_t steps = tpw * p.tile_rows / 64;
        if (steps <= 16)
            hipLaunchKernelGGL(layout_single_kernel<16>, dim3(1), dim3(kSingleThreads), 0, stream, a);
        else if (steps <= 32)
            hipLaunchKernelGGL(layout_single_kernel<32>, dim3(1), dim3(kSingleThreads), 0, stream, a);
        else
            hipLaunchKernelGGL(layout_single_kernel<64>, dim3(1), dim3(kSingleThreads), 0, stream, a);
        return hipGetLastError();
    }
    // enough workgroups to fill the chip, never more than tiles, and few
    // enough tiles per workgroup for the LDS tile list
    int64_t grid = 2 * (int64_t)di.cus;
    const int64_t need = (p.n_tiles + kMaxTilesPerGroup - 1) / kMaxTilesPerGroup;
    if (grid < need) grid = need;
    if (grid > p.n_tiles) grid = p.n_tiles;
    hipLaunchKernelGGL(layout_kernel, dim3((unsigned)grid), dim3(kLayoutThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ubep

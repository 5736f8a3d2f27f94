// The multi-workgroup dispatch layout ("NJU x Huawei UBEP: Reengineering MoE
// Expert Parallelism", sections "BSP Serialization" and "Kernel
// Decomposition"), as a device-side worker that a kernel runs in some or all
// of its workgroups.  NW is the number of waves per workgroup.
//
// No memory fences: every value one workgroup passes to another travels
// inside a self-contained 64-bit state word (call epoch | flag | count),
// written and read with agent-scope atomics.  Rows (t, j) are cut into tiles
// of whole tokens; a tile never straddles a source-rank or chunk boundary.
// Each tile has R + E "digits": one per destination rank, one per expert.
// Positions are ranked by "key": the destination rank (rank order) or the
// expert (expert order, rows grouped by expert inside each region); the key
// digits are the rank digits or the expert digits.  All per-key arrays below
// have K = R or K = E entries.
//
// Phase A -- the worker takes tiles from a ticket counter, in order, and
//   claims its next tile while it works on the current one:
//   * each wave loads all of its ids in one burst, then counts per-wave rank
//     histograms and the tile's expert histogram with LDS atomics;
//   * publishes the tile's per-digit aggregate and computes the in-tile
//     stable ranks (ballot peer masks per 64-row step, per-wave bases across
//     waves);
//   * look-back mode only: looks back over earlier tiles' published words,
//     32 predecessors per round (decoupled look-back), and publishes the
//     inclusive count.  Tiles are handed out in order, so every awaited tile
//     is held by a running workgroup that publishes its aggregate without
//     waiting: no grid barrier, no co-residency assumption.  A tile's
//     exclusive prefix at a source-rank / chunk boundary is a row of
//     send_offset / chunk_offset.
// Phase B -- after the ticket counter runs dry (so every tile is held by a
//   running workgroup whose phase A does not wait on this one):
//   * look-back mode: the worker waits for the last tile's inclusive words
//     (the totals);
//   * gather mode (few tiles): the worker reads every tile's rank aggregates
//     once, which gives both its own tiles' exclusive prefixes and the
//     totals in a single round of loads, and sums one slice of the expert
//     aggregates into expert_count;
//   then it scans the rank totals into recv_offset and writes pos / recv_src
//   for its tiles.  Workgroup 0 of the workers writes the rank totals.
// Words of an older epoch read as "not yet published", so nothing is cleared
// between calls; the kernel's last workgroup resets the tickets and advances
// the epoch.
#pragma once

#include "device_common.h"

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
    int32_t* excl;           // [n_tiles][K]
    int32_t* wbase;          // [n_tiles][NW][K]
    Plan p;
    uint64_t spin_ticks;
    int32_t* expert_offset;  // [E+1], expert order only (may be null)
    uint32_t* status;        // device status word (first error wins)
};

// LDS of one worker, carved from the kernel's dynamic shared memory.
struct LayoutLds {
    int32_t* wh;      // [NW][K] per-wave key counts, then running bases
    int32_t* eh;      // [E]     tile expert counts
    int32_t* cnt;     // [K]     tile key counts, then key totals
    int32_t* excl;    // [K]     rows with key q before the last claimed tile
    int32_t* off;     // [K]     exclusive scan of the key totals
    uint32_t* tiles;  // [kMaxTilesPerGroup] tiles this workgroup claimed
    int32_t* tmp;     // [NW]
    uint32_t* ticket; // [1]
    int32_t* bins;    // gather mode: [kGatherMaxMine + 1][K] key counts binned by own tiles
};

// Tiles one worker may claim.
__host__ __device__ inline int64_t layout_claim_limit(const Plan& p) {
    return p.gather ? kGatherMaxMine : kMaxTilesPerGroup;
}

inline int64_t layout_lds_bytes(const Plan& p, int nw) {
    const int64_t bins = p.gather ? (int64_t)(kGatherMaxMine + 1) * p.K : 0;
    return 4 * ((int64_t)nw * p.K + p.E + 3 * (int64_t)p.K + kMaxTilesPerGroup + nw + 1 + bins);
}

template <bool EORD = false>
__device__ __forceinline__ LayoutLds carve_lds(int32_t* base, const Plan& p, int nw) {
    const int32_t K = EORD ? p.K : p.R;
    LayoutLds L;
    L.wh = base;
    L.eh = L.wh + nw * K;
    L.cnt = L.eh + p.E;
    L.excl = L.cnt + K;
    L.off = L.excl + K;
    L.tiles = reinterpret_cast<uint32_t*>(L.off + K);
    L.tmp = reinterpret_cast<int32_t*>(L.tiles + kMaxTilesPerGroup);
    L.ticket = reinterpret_cast<uint32_t*>(L.tmp + nw);
    L.bins = reinterpret_cast<int32_t*>(L.ticket + 1);
    return L;
}

// LR: ids a lane holds for one tile (tiles of at most NW * 64 * LR rows);
// the default covers kTileRowsMax.
template <int NW>
constexpr int max_lane_rows() { return (int)(kTileRowsMax / NW / 64); }

// Rows of the tile owned by wave w: [lo, hi).
template <int NW>
__device__ __forceinline__ void wave_rows(const Plan& p, int w, int64_t* lo, int64_t* hi) {
    const int64_t per_wave = (p.tile_rows + NW - 1) / NW;
    *lo = w * per_wave;
    *hi = *lo + per_wave < p.tile_rows ? *lo + per_wave : p.tile_rows;
}

// Load the wave's expert ids in one burst: ev[i] holds row lo + 64 i + lane
// (loads are unconditional, from clamped rows, so all are in flight at once;
// entries past the wave's rows are unused).
template <int NW, int LR>
__device__ __forceinline__ void load_ids(const LayoutArgs& a, int64_t tile, int32_t (&ev)[LR]) {
    const Plan& p = a.p;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int64_t lo, hi;
    wave_rows<NW>(p, w, &lo, &hi);
    const int32_t* src = a.idx + tile * p.tile_rows;
#pragma unroll
    for (int i = 0; i < LR; ++i) {
        const int64_t r = lo + 64 * i + lane;
        ev[i] = src[r < p.tile_rows ? r : p.tile_rows - 1];
    }
}

// Ids outside [0, E) are reported and treated as expert 0.
template <int NW, int LR>
__device__ __forceinline__ void check_ids(const Plan& p, int32_t (&ev)[LR], bool* bad) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int64_t lo, hi;
    wave_rows<NW>(p, w, &lo, &hi);
#pragma unroll
    for (int i = 0; i < LR; ++i) {
        if ((uint32_t)ev[i] >= (uint32_t)p.E) {
            if (lo + 64 * i + lane < hi) *bad = true;
            ev[i] = 0;
        }
    }
}

// wh[w*K + q] = rows of wave w with key q; eh[e] = rows of the tile with
// expert e (rank order only: in expert order the key counts are the expert
// counts).  Counting needs no order, so plain LDS atomics do it (a hot key
// under skew only serialises its own lanes).
template <int NW, int LR, bool EORD>
__device__ __forceinline__ void tile_histograms(const Plan& p, const int32_t (&ev)[LR],
                                                int32_t* wh, int32_t* eh) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int64_t lo, hi;
    wave_rows<NW>(p, w, &lo, &hi);
#pragma unroll
    for (int i = 0; i < LR; ++i) {
        if (lo + 64 * i >= hi) break;                      // uniform across the wave
        if (lo + 64 * i + lane < hi) {
            const uint32_t e = (uint32_t)ev[i];
            atomicAdd(&wh[w * (EORD ? p.K : p.R) + (EORD ? e : rank_of(e, p.epr_magic))], 1);
            if constexpr (!EORD) atomicAdd(&eh[e], 1);
        }
    }
}

// Stable ranking inside a tile: base[w*K + q] holds the value of wave w's
// first row with key q; every row gets base + (rows before it in the wave
// with key q), and base advances.  Ballot peer masks give the order among
// equal ranks inside a 64-row step; steps run in row order.
template <int NW, int LR, bool EORD>
__device__ __forceinline__ void tile_ranks(const Plan& p, const int32_t (&ev)[LR],
                                           int32_t* base, int32_t (&rank)[LR]) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int64_t lo, hi;
    wave_rows<NW>(p, w, &lo, &hi);
#pragma unroll
    for (int i = 0; i < LR; ++i) {
        rank[i] = 0;
        if (lo + 64 * i >= hi) continue;                   // uniform across the wave
        const bool act = lo + 64 * i + lane < hi;
        const uint32_t d = EORD ? (uint32_t)ev[i] : rank_of((uint32_t)ev[i], p.epr_magic);
        const uint64_t pd = peers_of_n<EORD ? 13 : 10>(d, EORD ? p.ebits : p.dbits, __ballot(act));
        const uint64_t before = pd & lanemask_lt();
        if (act) {
            const int32_t K = EORD ? p.K : p.R;
            const int32_t b = base[w * K + d];
            rank[i] = b + (int32_t)__popcll(before);
            if (before == 0) base[w * K + d] = b + (int32_t)__popcll(pd);
        }
    }
}

// pos (and recv_src) of the tile's rows.  COH: pos is written with
// device-coherent stores, for consumers in other workgroups of this kernel.
template <int NW, int LR, bool COH>
__device__ __forceinline__ void store_positions(const LayoutArgs& a, int64_t tile,
                                                const int32_t (&q)[LR], bool* bad_pos) {
    const Plan& p = a.p;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row0 = tile * p.tile_rows;
    int64_t lo, hi;
    wave_rows<NW>(p, w, &lo, &hi);
#pragma unroll
    for (int i = 0; i < LR; ++i) {
        const int64_t r = lo + 64 * i + lane;
        if (r >= hi) continue;
        if constexpr (COH)
            __hip_atomic_store(a.pos + row0 + r, q[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
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
// words, a window of W predecessors per round, adding aggregates until an
// inclusive count is found.  A predecessor that has not published yet stalls
// the walk at that point until it does (bounded by spin_ticks).
template <int W>
__device__ __forceinline__ int32_t look_back(const LayoutArgs& a, int64_t tile, int32_t slot,
                                             uint32_t epoch, bool* timed_out) {
    const int32_t S = a.p.slots;
    int32_t excl = 0;
    int64_t j = tile - 1;
    const uint64_t t0 = now_ticks();
    while (j >= 0) {
        uint64_t v[W];
#pragma unroll
        for (int i = 0; i < W; ++i)
            v[i] = (j - i >= 0) ? ld_relaxed64(a.state + (j - i) * S + slot) : 0ull;
        int consumed = 0;
        bool done = false, stall = false;
#pragma unroll
        for (int i = 0; i < W; ++i) {
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

// Count of a published state word; spins on the word until its tile has
// published in this epoch (bounded by spin_ticks).
__device__ __forceinline__ int32_t settle(const uint64_t* w, uint64_t v, uint32_t epoch,
                                          uint64_t spin_ticks, bool* timed_out) {
    const auto published = [epoch](uint64_t x) {
        return (uint32_t)(x >> 32) == epoch && ((uint32_t)x & ~kCountMask) != 0u;
    };
    if (!published(v)) {
        const uint64_t t0 = now_ticks();
        for (;;) {
            __builtin_amdgcn_s_sleep(1);
            v = ld_relaxed64(w);
            if (published(v)) break;
            if (now_ticks() - t0 > spin_ticks) {
                *timed_out = true;
                return 0;
            }
        }
    }
    return (int32_t)((uint32_t)v & kCountMask);
}

// Gather mode: the aggregates of `n_cols` digits starting at `col0` for every
// tile, pair q = tile * n_cols + column, kGatherBurst loads in flight per
// thread (clamped to the first pair past the end, so all are valid), each
// passed to f(tile, column, count) once published.
template <int NT, typename F>
__device__ __forceinline__ void gather_aggregates(const LayoutArgs& a, int32_t col0, int32_t n_cols,
                                                  uint32_t epoch, bool* timed_out, F&& f) {
    const int32_t S = a.p.slots;
    const int32_t n = (int32_t)a.p.n_tiles * n_cols;
    for (int32_t q0 = 0; q0 < n; q0 += NT * kGatherBurst) {
        uint64_t v[kGatherBurst];
        const uint64_t* w[kGatherBurst];
#pragma unroll
        for (int u = 0; u < kGatherBurst; ++u) {
            const int32_t q_raw = q0 + u * NT + (int32_t)threadIdx.x;
            const int32_t q = q_raw < n ? q_raw : 0;
            const int32_t j = q / n_cols, c = q - j * n_cols;
            w[u] = a.state + (int64_t)j * S + col0 + c;
            v[u] = ld_relaxed64(w[u]);
        }
#pragma unroll
        for (int u = 0; u < kGatherBurst; ++u) {
            const int32_t q = q0 + u * NT + (int32_t)threadIdx.x;
            if (q < n) {
                const int32_t j = q / n_cols, c = q - j * n_cols;
                f(j, c, settle(w[u], v[u], epoch, a.spin_ticks, timed_out));
            }
        }
    }
}

// One worker workgroup (worker `wid` of `nw_workers`): phases A and B for
// the tiles it claims.  Worker 0 writes the totals.  Returns once this
// workgroup's pos / recv_src are stored (COH_POS: with device-coherent stores).
// done (thread 0, may be null): counts the workgroup on the done counter once
// it has its totals -- its last ticket claim has returned long before, and it
// touches no ticket, counter or epoch word after that -- and receives the
// counter's old value (its round trip overlaps the scan and the stores).
template <int NW, int LR, bool COH_POS, int W = kLookbackWindow, bool EORD = false>
__device__ __forceinline__ void layout_worker(const LayoutArgs& a, const LayoutLds& L, uint32_t epoch,
                                              uint32_t wid, uint32_t nw_workers,
                                              uint32_t* done = nullptr) {
    const bool leader = wid == 0;
    constexpr int T_ = NW * 64;
    const Plan& p = a.p;
    const int tid = threadIdx.x;
    constexpr bool eord = EORD;   // expert order (p.order == 1)
    const int32_t R = p.R, E = p.E, S = p.slots, epr = p.epr;
    const int32_t K = eord ? p.K : p.R, kcol = eord ? p.kcol : 0;
    bool bad = false, bad_pos = false, timed_out = false;
    uint32_t n_mine = 0;
    int32_t ev[LR];                                  // ids of the last claimed tile
    int32_t lrank[LR];                               // their ranks inside the tile

    // ---------------- phase A: counts, in-tile ranks (and look-back), tile by tile
    // (the launch guarantees workers * claim limit >= n_tiles; at its limit a
    // worker stops claiming)
    const bool gather = p.gather != 0;
    const uint32_t cap = (uint32_t)layout_claim_limit(p);
    uint32_t claim = 0;                              // thread 0: the claim in flight
    if (tid == 0) claim = add_relaxed(&a.hdr[kHdrLayoutTicket], 1u);
    // the first ticket is usually the worker's own index: fetch that tile's
    // ids while the claim is in flight, refetch below if it is another
    int32_t nv[LR];
    if (wid < (uint64_t)p.n_tiles) load_ids<NW, LR>(a, wid, nv);
    for (;;) {
        if (tid == 0) *L.ticket = claim;
        for (int i = tid; i < NW * K; i += T_) L.wh[i] = 0;
        if (!eord)
            for (int i = tid; i < E; i += T_) L.eh[i] = 0;
        __syncthreads();
        const uint32_t tile = *L.ticket;
        if (tile >= (uint64_t)p.n_tiles) break;
        if (n_mine > 0 || tile != wid) load_ids<NW, LR>(a, tile, nv);
#pragma unroll
        for (int i = 0; i < LR; ++i) ev[i] = nv[i];
        check_ids<NW, LR>(p, ev, &bad);
        if (tid == 0) L.tiles[n_mine] = tile;
        ++n_mine;
        tile_histograms<NW, LR, EORD>(p, ev, L.wh, L.eh);
        __syncthreads();
        // claim the next tile now, after the barrier (so that the ids are in
        // registers: a claim issued before they arrived would be waited on
        // with them); its round trip overlaps the rest of this tile's work.
        // At the claim limit claim nothing and stop after this tile.
        if (tid == 0) claim = n_mine < cap ? add_relaxed(&a.hdr[kHdrLayoutTicket], 1u) : 0xFFFFFFFFu;

        // wave bases (kept for a later re-rank), tile aggregates, publish
        int32_t* wb = a.wbase + (int64_t)tile * NW * K;
        for (int32_t d = tid; d < K; d += T_) {
            int32_t run = 0;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const int32_t c = L.wh[v * K + d];
                L.wh[v * K + d] = run;
                wb[v * K + d] = run;
                run += c;
            }
            L.cnt[d] = run;
        }
        __syncthreads();
        // the tile's count of digit s: a rank (s < R) or an expert
        const auto digit_count = [&](int32_t s) -> int32_t {
            if (!eord) return s < R ? L.cnt[s] : L.eh[s - R];
            if (s >= R) return L.cnt[s - R];
            int32_t c = 0;
            for (int32_t e = s * epr; e < (s + 1) * epr; ++e) c += L.cnt[e];
            return c;
        };
        uint64_t* st = a.state + (int64_t)tile * S;
        for (int32_t s = tid; s < S; s += T_) {
            const int32_t c = digit_count(s);
            st_relaxed64(st + s, state_word(epoch, tile == 0 ? kFlagInclusive : kFlagAggregate, c));
        }
        // in-tile ranks now, while the other tiles publish
        tile_ranks<NW, LR, EORD>(p, ev, L.wh, lrank);
        if (!gather) {
            const int64_t tok0 = (int64_t)tile * p.tile_tokens;
            for (int32_t s = tid; s < S; s += T_) {
                const int32_t c = digit_count(s);
                const int32_t excl = tile == 0 ? 0 : look_back<W>(a, tile, s, epoch, &timed_out);
                if (tile != 0) st_relaxed64(st + s, state_word(epoch, kFlagInclusive, excl + c));
                const int32_t q = s - kcol;
                if ((uint32_t)q < (uint32_t)K) {
                    L.excl[q] = excl;
                    a.excl[(int64_t)tile * K + q] = excl;
                }
                if (s < R) {
                    if (tok0 % p.tps == 0) a.send_offset[(tok0 / p.tps) * R + s] = excl;
                    if (a.chunk_offset != nullptr && tok0 % p.tpc == 0)
                        a.chunk_offset[(tok0 / p.tpc) * R + s] = excl;
                }
            }
        }
        __syncthreads();
    }

    // ---------------- phase B: totals, recv_offset, positions
    const int32_t n_m = (int32_t)n_mine;
    int32_t e_lo = 0, n_e = 0;      // gather mode: this worker's slice of expert_count
    if (gather) {
        // bins[b][d]: rows to rank d in the tiles j with b of this worker's
        // tiles at or before j.  A tile j lies before tiles[m] exactly when
        // fewer than m + 1 of them are at or before j, so the running sum
        // over b up to m is the exclusive prefix of tiles[m], and up to
        // n_mine the total.
        for (int i = tid; i < (n_m + 1) * K; i += T_) L.bins[i] = 0;
        if (!eord) {   // in expert order the key totals are the expert counts
            const int32_t e_per = (E + (int32_t)nw_workers - 1) / (int32_t)nw_workers;
            e_lo = (int64_t)wid * e_per < E ? (int32_t)wid * e_per : E;
            n_e = E - e_lo < e_per ? E - e_lo : e_per;
        }
        for (int i = tid; i < n_e; i += T_) L.eh[i] = 0;
        __syncthreads();
        gather_aggregates<T_>(a, kcol, K, epoch, &timed_out, [&](int32_t j, int32_t d, int32_t c) {
            int32_t b = 0;
            for (int32_t m = 0; m < n_m; ++m) b += (int32_t)L.tiles[m] <= j ? 1 : 0;
            atomicAdd(&L.bins[b * K + d], c);
        });
        if (n_e > 0)
            gather_aggregates<T_>(a, R + e_lo, n_e, epoch, &timed_out,
                                  [&](int32_t, int32_t e, int32_t c) { atomicAdd(&L.eh[e], c); });
        __syncthreads();
        for (int32_t d = tid; d < K; d += T_) {
            int32_t run = 0;
            for (int32_t m = 0; m <= n_m; ++m) {
                run += L.bins[m * K + d];
                L.bins[m * K + d] = run;   // prefix of tiles[m] (m < n_mine), total (m = n_mine)
            }
            L.cnt[d] = run;
            if (n_m > 0) L.excl[d] = L.bins[(n_m - 1) * K + d];
        }
    } else {
        for (int32_t d = tid; d < K; d += T_) L.cnt[d] = wait_total(a, kcol + d, epoch, &timed_out);
    }
    // this workgroup touches no ticket, counter or epoch word from here on
    if (done != nullptr && tid == 0) *done = add_relaxed(&a.hdr[kHdrLayoutDone], 1u);
    __syncthreads();
    {   // exclusive scan of the key totals; thread i owns a run of keys
        const int per = (K + T_ - 1) / T_;
        int32_t mine = 0;
        for (int i = 0; i < per; ++i) {
            const int32_t d = tid * per + i;
            if (d < K) mine += L.cnt[d];
        }
        const int lane = tid & 63, w = tid >> 6;
        int32_t inc = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t u = __shfl_up(inc, o, 64);
            if (lane >= o) inc += u;
        }
        if (lane == 63) L.tmp[w] = inc;
        __syncthreads();
        int32_t run = inc - mine;
        for (int i = 0; i < w; ++i) run += L.tmp[i];
        for (int i = 0; i < per; ++i) {
            const int32_t d = tid * per + i;
            if (d < K) {
                L.off[d] = run;
                run += L.cnt[d];
            }
        }
    }
    __syncthreads();
    for (uint32_t m = 0; m < n_mine; ++m) {
        const int64_t tile = L.tiles[m];
        int32_t q[LR];
        if (m + 1 == n_mine) {     // the last claimed tile: ids and in-tile ranks in registers
#pragma unroll
            for (int i = 0; i < LR; ++i) {
                const uint32_t d = eord ? (uint32_t)ev[i] : rank_of((uint32_t)ev[i], p.epr_magic);
                q[i] = L.off[d] + L.excl[d] + lrank[i];
            }
        } else {                   // an earlier tile of this workgroup: rebuild from its state
            int32_t ids[LR];
            load_ids<NW, LR>(a, tile, ids);
            bool ignore = false;
            check_ids<NW, LR>(p, ids, &ignore);
            __syncthreads();
            for (int i = tid; i < NW * K; i += T_) {
                const int32_t d = i % K;
                const int32_t excl = gather ? L.bins[m * K + d] : a.excl[tile * K + d];
                L.wh[i] = L.off[d] + excl + a.wbase[tile * NW * K + i];
            }
            __syncthreads();
            tile_ranks<NW, LR, EORD>(p, ids, L.wh, q);
        }
        store_positions<NW, LR, COH_POS>(a, tile, q, &bad_pos);
    }

    // outputs that nothing in this kernel reads, stored last so that no wait
    // above covers them
    // rows with a key of rank d in a per-key array v (rank order: v[d])
    const auto rank_sum = [&](const int32_t* v, int32_t d) -> int32_t {
        if (!eord) return v[d];
        int32_t c = 0;
        for (int32_t e = d * epr; e < (d + 1) * epr; ++e) c += v[e];
        return c;
    };
    if (gather) {
        for (int32_t d = tid; d < R; d += T_) {
            for (int32_t m = 0; m < n_m; ++m) {
                const int64_t tok0 = (int64_t)L.tiles[m] * p.tile_tokens;
                if (tok0 % p.tps == 0) a.send_offset[(tok0 / p.tps) * R + d] = rank_sum(L.bins + m * K, d);
                if (a.chunk_offset != nullptr && tok0 % p.tpc == 0)
                    a.chunk_offset[(tok0 / p.tpc) * R + d] = rank_sum(L.bins + m * K, d);
            }
        }
        for (int i = tid; i < n_e; i += T_) a.expert_count[e_lo + i] = L.eh[i];
    } else if (leader && !eord) {
        for (int32_t e = tid; e < E; e += T_) a.expert_count[e] = wait_total(a, R + e, epoch, &timed_out);
    }
    if (leader) {
        for (int32_t d = tid; d < R; d += T_) {
            a.rank_count[d] = rank_sum(L.cnt, d);
            a.recv_offset[d] = L.off[eord ? d * epr : d];
        }
        if (tid == 0) a.recv_offset[R] = L.off[K - 1] + L.cnt[K - 1];
        if (eord) {    // key totals and their scan are the expert counts and offsets
            for (int32_t e = tid; e < E; e += T_) {
                a.expert_count[e] = L.cnt[e];
                if (a.expert_offset != nullptr) a.expert_offset[e] = L.off[e];
            }
            if (tid == 0 && a.expert_offset != nullptr) a.expert_offset[E] = L.off[E - 1] + L.cnt[E - 1];
        }
    }

    if (bad) raise_status(a.status, UBEP_ERR_BAD_EXPERT_ID);
    if (timed_out) raise_status(a.status, UBEP_ERR_TIMEOUT);
    if (bad_pos) raise_status(a.status, UBEP_ERR_BAD_POSITION);
}

// Reset the tickets and counters and advance the epoch (done by the last
// workgroup to count itself done).
__device__ __forceinline__ void layout_reset(const LayoutArgs& a, uint32_t epoch) {
    st_relaxed(&a.hdr[kHdrLayoutTicket], 0u);
    st_relaxed(&a.hdr[kHdrRoleTicket], 0u);
    st_relaxed(&a.hdr[kHdrPosReady], 0u);
    st_relaxed(&a.hdr[kHdrLayoutDone], 0u);
    st_relaxed(&a.hdr[kHdrLayoutEpoch], epoch + 1u);
}

// End of a kernel that ran layout workers (and possibly workgroups that poll
// the header until they end): the last workgroup out resets.  Every
// workgroup's final ticket claim returned before its increment here.
__device__ __forceinline__ void layout_finish(const LayoutArgs& a, uint32_t epoch) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t done = add_relaxed(&a.hdr[kHdrLayoutDone], 1u);
        if (done == gridDim.x - 1u) layout_reset(a, epoch);
    }
}

}  // namespace ubep

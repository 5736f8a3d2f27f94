// Dispatch layout on gfx950: token counting, prefix sums, offsets and stable
// reorder positions ("NJU x Huawei UBEP: Reengineering MoE Expert
// Parallelism", sections "BSP Serialization" and "Kernel Decomposition").
//
// The persistent multi-workgroup layout is the worker in layout_worker.h
// (no memory fences; decoupled look-back over epoch-tagged state words); the
// standalone kernel below runs it in every workgroup.
//
// Tiny problems take a one-workgroup kernel instead:
// 16 waves own contiguous runs of tiles, keep their ids in registers, and do
// the tile counts, the prefix sums over tiles and ranks, and the ranking in
// LDS.  With no value crossing workgroups it avoids the device-memory round
// trips (ticket, publish, look-back, totals) that bound the persistent
// kernel's latency.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "launch.h"
#include "layout_worker.h"

namespace ubep {

// Every workgroup is a worker and counts itself done as soon as it has its
// totals (the round trip overlaps the rest of phase B); the last one resets.
// LR: ids a lane holds (tiles of at most kLayoutThreads * LR rows).
// EORD: expert order (a.p.order == 1).
template <int LR, bool EORD>
__global__ __launch_bounds__(kLayoutThreads) void layout_kernel(LayoutArgs a) {
    extern __shared__ int32_t dyn_lds[];
    const uint32_t epoch = ld_relaxed(&a.hdr[kHdrLayoutEpoch]);
    const LayoutLds L = carve_lds<EORD>(dyn_lds, a.p, kLayoutWaves);
    uint32_t done = 0;
    layout_worker<kLayoutWaves, LR, false, kLookbackWindow, EORD>(a, L, epoch, blockIdx.x, gridDim.x,
                                                                 &done);
    if (threadIdx.x == 0 && done == gridDim.x - 1u) layout_reset(a, epoch);
}

static std::atomic<int32_t> g_worker_cap{0};

void set_layout_worker_cap(int32_t n) { g_worker_cap.store(n, std::memory_order_relaxed); }

// No worker cap set (a cap asks for the persistent kernel, whose tiles it spreads).
static bool g_worker_cap_default() { return g_worker_cap.load(std::memory_order_relaxed) == 0; }

// ---------------------------------------------------------------- one-workgroup layout
constexpr int kSingleThreads = 1024;
constexpr int kSingleWaves = kSingleThreads / 64;
constexpr int kSingleSteps = 64;                 // 64-row steps a wave may own
constexpr int64_t kSingleMaxRows = (int64_t)kSingleWaves * kSingleSteps * 64;
constexpr int kSingleMaxK = 256;
constexpr int kSingleMaxE = 4096;
constexpr int kSingleMaxTiles = 256;
constexpr int kSingleMaxTileCounts = 8192;       // n_tiles * K

// Only tiny problems: above a few thousand rows one CU's ballot and LDS work
// costs more than the persistent kernel's memory round trips.
constexpr int64_t kSingleUseRows = 4096;

bool layout_fits_one_group(const Plan& p) {
    const int64_t tiles_per_wave = (p.n_tiles + kSingleWaves - 1) / kSingleWaves;
    return p.rows <= kSingleUseRows && p.rows <= kSingleMaxRows && p.tile_rows % 64 == 0 && p.n_tiles <= kSingleMaxTiles &&
           p.n_tiles * p.K <= kSingleMaxTileCounts && p.K <= kSingleMaxK && p.E <= kSingleMaxE &&
           tiles_per_wave * p.tile_rows <= (int64_t)kSingleSteps * 64;
}

template <int STEPS>
__global__ __launch_bounds__(kSingleThreads) void layout_single_kernel(LayoutArgs a) {
    __shared__ int32_t s_tc[kSingleMaxTileCounts];  // [tile][key]: counts, then row bases
    __shared__ int32_t s_eh[kSingleMaxE];           // expert counts
    __shared__ int32_t s_tot[kSingleMaxK];          // key totals
    __shared__ int32_t s_off[kSingleMaxK];          // exclusive scan of the key totals
    __shared__ int32_t s_tmp[kSingleWaves];

    const Plan& p = a.p;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int32_t R = p.R, E = p.E, K = p.K, epr = p.epr;
    const bool eord = p.order != 0;
    // rows with a key of rank d in a per-key array v (rank order: v[d])
    const auto rank_sum = [&](const int32_t* v, int32_t d) -> int32_t {
        if (!eord) return v[d];
        int32_t c = 0;
        for (int32_t e = d * epr; e < (d + 1) * epr; ++e) c += v[e];
        return c;
    };
    for (int i = tid; i < p.n_tiles * K; i += kSingleThreads) s_tc[i] = 0;
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

    // pass 1: per-tile key counts and expert counts (order-free: LDS atomics)
    {
        int32_t tile = t_lo, in_tile = 0;
#pragma unroll
        for (int i = 0; i < STEPS; ++i) {
            if (i >= steps) break;                           // uniform across the wave
            const uint32_t e = (uint32_t)ev[i];
            atomicAdd(&s_tc[tile * K + rank_of(e, p.key_magic)], 1);
            atomicAdd(&s_eh[e], 1);
            if (++in_tile == steps_per_tile) {
                in_tile = 0;
                ++tile;
            }
        }
    }
    __syncthreads();

    // exclusive prefix over tiles for every key; the totals
    for (int32_t d = tid; d < K; d += kSingleThreads) {
        int32_t run = 0;
        for (int32_t t = 0; t < n_tiles; ++t) {
            const int32_t c = s_tc[t * K + d];
            s_tc[t * K + d] = run;
            run += c;
        }
        s_tot[d] = run;
    }
    __syncthreads();
    {   // exclusive scan of the totals over keys (K <= 1024: one key per thread)
        const int32_t mine = tid < K ? s_tot[tid] : 0;
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
        if (tid < K) s_off[tid] = before + inc - mine;
    }
    __syncthreads();
    for (int32_t d = tid; d < R; d += kSingleThreads) {
        a.rank_count[d] = rank_sum(s_tot, d);
        a.recv_offset[d] = s_off[eord ? d * epr : d];
    }
    if (tid == 0) a.recv_offset[R] = (int32_t)p.rows;
    for (int32_t e = tid; e < E; e += kSingleThreads) a.expert_count[e] = s_eh[e];
    if (eord && a.expert_offset != nullptr) {
        for (int32_t e = tid; e < E; e += kSingleThreads) a.expert_offset[e] = s_off[e];
        if (tid == 0) a.expert_offset[E] = (int32_t)p.rows;
    }
    // send / chunk offsets are the tile prefixes at source-rank / chunk boundaries
    const int32_t tiles_per_source = (int32_t)(p.tps / p.tile_tokens);
    const int32_t tiles_per_chunk = (int32_t)(p.tpc / p.tile_tokens);
    for (int32_t i = tid; i < R * R; i += kSingleThreads)
        a.send_offset[i] = rank_sum(s_tc + (i / R) * tiles_per_source * K, i % R);
    if (a.chunk_offset != nullptr)
        for (int32_t i = tid; i < p.C * R; i += kSingleThreads)
            a.chunk_offset[i] = rank_sum(s_tc + (i / R) * tiles_per_chunk * K, i % R);
    __syncthreads();
    for (int32_t i = tid; i < n_tiles * K; i += kSingleThreads) s_tc[i] += s_off[i % K];
    __syncthreads();

    // pass 2: stable ranks -> positions (ballot peer masks give the order
    // among equal ranks inside a step; steps run in row order)
    {
        int32_t tile = t_lo, in_tile = 0;
#pragma unroll
        for (int i = 0; i < STEPS; ++i) {
            if (i >= steps) break;                           // uniform across the wave
            const int64_t row = r_lo + 64 * i + lane;
            const uint32_t d = rank_of((uint32_t)ev[i], p.key_magic);
            const uint64_t pd = peers_of_n<8>(d, p.kbits, ~0ull);
            const uint64_t before = pd & lanemask_lt();
            const int32_t b = s_tc[tile * K + d];
            const int32_t q = b + (int32_t)__popcll(before);
            a.pos[row] = q;
            if ((uint32_t)q < (uint32_t)p.rows) {
                if (a.recv_src != nullptr) a.recv_src[q] = (int32_t)row;
            } else {
                bad_pos = true;
            }
            if (before == 0) s_tc[tile * K + d] = b + (int32_t)__popcll(pd);
            if (++in_tile == steps_per_tile) {
                in_tile = 0;
                ++tile;
            }
        }
    }
    if (bad) raise_status(a.status, UBEP_ERR_BAD_EXPERT_ID);
    if (bad_pos) raise_status(a.status, UBEP_ERR_BAD_POSITION);
}

// LDS of the persistent layout's workgroup within what a CU offers (the
// expert order keeps per-wave counts for every expert).
bool layout_lds_fits(const Plan& p) {
    return layout_fits_one_group(p) || layout_lds_bytes(p, kLayoutWaves) <= kLdsBytesPerCu;
}


// Workers of the persistent layout: enough to fill the chip (or the cap set
// by ubep_set_layout_workers), never more than tiles, and few enough tiles
// per worker for its claim limit.
int64_t layout_workers(const Plan& p, int cus) {
    int64_t n = 2 * (int64_t)cus;
    const int32_t user = g_worker_cap.load(std::memory_order_relaxed);
    if (user > 0 && user < n) n = user;
    const int64_t cap = layout_claim_limit(p);
    const int64_t need = (p.n_tiles + cap - 1) / cap;
    if (n < need) n = need;
    if (n > p.n_tiles) n = p.n_tiles;
    return n;
}

// ---------------------------------------------------------------- replicated layout
// Small problems with several tiles (up to kRepMaxRows rows, e.g. a
// 4096-token decode step of 32768 rows): every workgroup owns one tile and
// sweeps ALL the ids itself (a few hundred KB, read from L2), counting per
// expert the rows before its tile and the rest (per-rank counts are sums over
// the rank's experts).  That gives its tile's exclusive prefixes and the key
// totals with no value crossing workgroups: no tickets,
// no published words, no polling -- the round trips through device memory
// that bound the persistent kernel at this size -- at the price of the ids
// being read once per workgroup.  Then it ranks its own tile as the
// persistent kernel does (per-wave counts, ballot peer masks).  Under skewed
// routing many lanes of one atomic hit the same hot expert and serialise, so
// for up to 256 experts the counts go to four copies (by lane), summed after.
constexpr int64_t kRepMaxRows = 32768;
constexpr int kRepMaxK = 1024;
constexpr int kRepMaxSlice = 1024;
constexpr int kRepMaxTiles = 256;

bool layout_replicates(const Plan& p, const int32_t* idx) {
    return g_worker_cap_default() && p.rows <= kRepMaxRows && p.rows % 4 == 0 &&
           ((uintptr_t)idx % 16) == 0 && p.n_tiles >= 2 && p.n_tiles <= kRepMaxTiles &&
           p.E <= kRepMaxK;                              // the sweep's keys are experts (E >= R)
}

template <int LR, int NV, bool EORD>
__global__ __launch_bounds__(kLayoutThreads) void layout_replicated_kernel(LayoutArgs a) {
    // [copy][0][e]: rows to expert e before this tile; [copy][1][e]: the others
    __shared__ int32_t s_hist[2 * kRepMaxK];
    __shared__ int32_t s_rk[2 * kRepMaxK];         // rank order: the same two halves per rank
    __shared__ int32_t s_off[kRepMaxK];            // exclusive scan of the key totals
    __shared__ int32_t s_wh[kLayoutWaves * kRepMaxK];   // this tile's per-wave key counts, then row bases
    __shared__ int32_t s_tmp[kLayoutWaves];
    constexpr int T_ = kLayoutThreads;
    const Plan& p = a.p;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t tile = blockIdx.x;
    const int64_t t_start = tile * p.tile_rows;
    const int32_t R = p.R, E = p.E, epr = p.epr;
    const int32_t K = EORD ? E : R;                        // the layout's keys
    const int32_t copies = E <= kRepMaxK / 4 ? 4 : 1;      // both fit s_hist
    const int32_t my_copy = (tid & (copies - 1)) * 2 * E;

    // this tile's ids first, then the sweep over every row (int4 loads, all in
    // flight together; clamped, so every address is valid)
    int32_t ev[LR];
    load_ids<kLayoutWaves, LR>(a, tile, ev);
    const int4* src = reinterpret_cast<const int4*>(a.idx);
    const int64_t n4 = p.rows / 4;
    int4 v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int64_t i = tid + (int64_t)j * T_;
        v[j] = src[i < n4 ? i : n4 - 1];
    }
    for (int i = tid; i < 2 * E * copies; i += T_) s_hist[i] = 0;
    for (int i = tid; i < kLayoutWaves * K; i += T_) s_wh[i] = 0;
    __syncthreads();

    // The sweep counts experts, one LDS atomic per row; a rank's counts are
    // the sums over its experts, taken once afterwards.  Ids outside [0, E)
    // count as expert 0, as in the other modes (reported below).
    const auto count = [&](int32_t* h, int32_t e) {
        atomicAdd(&h[(uint32_t)e < (uint32_t)E ? e : 0], 1);
    };
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int64_t i = tid + (int64_t)j * T_;
        if (i < n4) {
            const int64_t r0 = 4 * i;
            int32_t* h = s_hist + my_copy + (r0 < t_start ? 0 : E);
            if (r0 < t_start && r0 + 4 > t_start) {          // the one vector astride the tile start
                int32_t* g = s_hist + my_copy + E;
                count(r0 + 0 < t_start ? h : g, v[j].x);
                count(r0 + 1 < t_start ? h : g, v[j].y);
                count(r0 + 2 < t_start ? h : g, v[j].z);
                count(r0 + 3 < t_start ? h : g, v[j].w);
            } else {
                count(h, v[j].x);
                count(h, v[j].y);
                count(h, v[j].z);
                count(h, v[j].w);
            }
        }
    }
    // this tile's per-wave key counts
    bool bad = false, bad_pos = false;
    check_ids<kLayoutWaves, LR>(p, ev, &bad);
    {
        int64_t lo, hi;
        wave_rows<kLayoutWaves>(p, w, &lo, &hi);
#pragma unroll
        for (int i = 0; i < LR; ++i) {
            if (lo + 64 * i + lane < hi) {
                const uint32_t e = (uint32_t)ev[i];
                atomicAdd(&s_wh[w * K + (EORD ? (int32_t)e : (int32_t)rank_of(e, p.epr_magic))], 1);
            }
        }
    }
    __syncthreads();
    if (copies > 1) {
        for (int i = tid; i < 2 * E; i += T_)
            s_hist[i] += s_hist[2 * E + i] + s_hist[4 * E + i] + s_hist[6 * E + i];
        __syncthreads();
    }
    // kh[q]: rows with key q before this tile; kh[K + q]: the others
    const int32_t* kh = s_hist;
    if (!EORD) {
        for (int i = tid; i < 2 * R; i += T_) {
            const int32_t half = i < R ? 0 : E, d = i < R ? i : i - R;
            int32_t c = 0;
            for (int32_t e = d * epr; e < (d + 1) * epr; ++e) c += s_hist[half + e];
            s_rk[i] = c;
        }
        __syncthreads();
        kh = s_rk;
    }

    {   // exclusive scan of the key totals; thread i owns a run of keys
        const int per = (K + T_ - 1) / T_;
        int32_t mine = 0;
        for (int i = 0; i < per; ++i) {
            const int32_t d = tid * per + i;
            if (d < K) mine += kh[d] + kh[K + d];
        }
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
            if (d < K) {
                s_off[d] = run;
                run += kh[d] + kh[K + d];
            }
        }
    }
    __syncthreads();
    // row bases of each wave of this tile: region start + rows in earlier
    // tiles + rows of earlier waves of this tile
    for (int32_t d = tid; d < K; d += T_) {
        int32_t run = s_off[d] + kh[d];
#pragma unroll
        for (int v_ = 0; v_ < kLayoutWaves; ++v_) {
            const int32_t c = s_wh[v_ * K + d];
            s_wh[v_ * K + d] = run;
            run += c;
        }
    }
    __syncthreads();
    int32_t q[LR];
    tile_ranks<kLayoutWaves, LR, EORD>(p, ev, s_wh, q);
    store_positions<kLayoutWaves, LR, false>(a, tile, q, &bad_pos);

    // rows to rank d before this tile (half 0) or in total (half 1)
    const auto rank_rows = [&](int32_t d, bool total) -> int32_t {
        if (!EORD) return s_rk[d] + (total ? s_rk[R + d] : 0);
        int32_t c = 0;
        for (int32_t e = d * epr; e < (d + 1) * epr; ++e) c += s_hist[e] + (total ? s_hist[E + e] : 0);
        return c;
    };
    const int64_t tok0 = tile * p.tile_tokens;
    if (tok0 % p.tps == 0)
        for (int32_t d = tid; d < R; d += T_) a.send_offset[(tok0 / p.tps) * R + d] = rank_rows(d, false);
    if (a.chunk_offset != nullptr && tok0 % p.tpc == 0)
        for (int32_t d = tid; d < R; d += T_) a.chunk_offset[(tok0 / p.tpc) * R + d] = rank_rows(d, false);
    {   // each workgroup writes a slice of the expert totals
        const int32_t e_per = (E + (int32_t)gridDim.x - 1) / (int32_t)gridDim.x;
        const int32_t e_lo = (int64_t)tile * e_per < E ? (int32_t)tile * e_per : E;
        const int32_t e_hi = E - e_lo < e_per ? E : e_lo + e_per;
        for (int32_t e = e_lo + tid; e < e_hi; e += T_) a.expert_count[e] = s_hist[e] + s_hist[E + e];
    }
    if (tile == 0) {
        for (int32_t d = tid; d < R; d += T_) {
            a.rank_count[d] = rank_rows(d, true);
            a.recv_offset[d] = s_off[EORD ? d * epr : d];
        }
        if (tid == 0) a.recv_offset[R] = (int32_t)p.rows;
        if (EORD && a.expert_offset != nullptr) {
            for (int32_t e = tid; e < E; e += T_) a.expert_offset[e] = s_off[e];
            if (tid == 0) a.expert_offset[E] = (int32_t)p.rows;
        }
    }
    if (bad) raise_status(a.status, UBEP_ERR_BAD_EXPERT_ID);
    if (bad_pos) raise_status(a.status, UBEP_ERR_BAD_POSITION);
}

// ---------------------------------------------------------------- layout from gate counts
// The second half of ubep_gate_layout: the gate has already counted its
// selections per (tile, rank) and per (tile, expert) into the workspace, so a
// workgroup per tile needs no sweep of the ids and no word from another
// workgroup of this kernel: one round of loads of the counts gives its tile's
// exclusive prefixes and the totals, and it ranks its own tile as the other
// layouts do.  The last workgroup to finish clears the counts for the next
// call (the workspace starts zero-filled).
bool layout_from_counts_fits(const Plan& p) {
    const int64_t e_per = (p.E + p.n_tiles - 1) / p.n_tiles;
    return p.R <= kRepMaxK && e_per <= kRepMaxSlice && p.n_tiles <= 65535;
}

template <int LR>
__global__ __launch_bounds__(kLayoutThreads) void layout_counts_kernel(LayoutArgs a,
                                                                       int32_t* rank_cnt,
                                                                       int32_t* expert_cnt) {
    __shared__ int32_t s_before[kRepMaxK];     // rows to rank d in earlier tiles
    __shared__ int32_t s_total[kRepMaxK];      // rows to rank d
    __shared__ int32_t s_off[kRepMaxK];        // exclusive scan of the totals
    __shared__ int32_t s_wh[kLayoutWaves * kRepMaxK];
    __shared__ int32_t s_eh[kRepMaxSlice];
    __shared__ int32_t s_tmp[kLayoutWaves];
    constexpr int T_ = kLayoutThreads;
    const Plan& p = a.p;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t tile = blockIdx.x;
    const int32_t R = p.R, E = p.E;
    const int32_t n_tiles = (int32_t)p.n_tiles;
    const int32_t e_per = (E + n_tiles - 1) / n_tiles;
    const int32_t e_lo = (int64_t)tile * e_per < E ? (int32_t)tile * e_per : E;
    const int32_t n_e = E - e_lo < e_per ? E - e_lo : e_per;

    int32_t ev[LR];
    load_ids<kLayoutWaves, LR>(a, tile, ev);
    for (int i = tid; i < R; i += T_) s_before[i] = s_total[i] = 0;
    for (int i = tid; i < kLayoutWaves * R; i += T_) s_wh[i] = 0;
    for (int i = tid; i < n_e; i += T_) s_eh[i] = 0;
    __syncthreads();
    // every tile's rank counts and this workgroup's slice of expert counts
    const int64_t nr = (int64_t)n_tiles * R;
    for (int64_t i = tid; i < nr; i += T_) {
        const int32_t tau = (int32_t)(i / R), d = (int32_t)(i - (int64_t)tau * R);
        const int32_t c = rank_cnt[i];
        atomicAdd(&s_total[d], c);
        if (tau < tile) atomicAdd(&s_before[d], c);
    }
    const int64_t ne = (int64_t)n_tiles * n_e;
    for (int64_t i = tid; i < ne; i += T_) {
        const int32_t tau = (int32_t)(i / n_e), e = (int32_t)(i - (int64_t)tau * n_e);
        atomicAdd(&s_eh[e], expert_cnt[(int64_t)tau * E + e_lo + e]);
    }
    bool bad = false, bad_pos = false;
    check_ids<kLayoutWaves, LR>(p, ev, &bad);
    {
        int64_t lo, hi;
        wave_rows<kLayoutWaves>(p, w, &lo, &hi);
#pragma unroll
        for (int i = 0; i < LR; ++i)
            if (lo + 64 * i + lane < hi) atomicAdd(&s_wh[w * R + (int32_t)rank_of((uint32_t)ev[i], p.epr_magic)], 1);
    }
    __syncthreads();
    // every count has been read: count this workgroup out; the last one
    // clears the counts for the next call
    if (tid == 0) {
        const uint32_t done = add_relaxed(&a.hdr[kHdrGateLayoutDone], 1u);
        s_tmp[0] = done == gridDim.x - 1u ? 1 : 0;
    }
    __syncthreads();
    if (s_tmp[0] != 0) {
        for (int64_t i = tid; i < nr; i += T_) rank_cnt[i] = 0;
        for (int64_t i = tid; i < (int64_t)n_tiles * E; i += T_) expert_cnt[i] = 0;
        if (tid == 0) st_relaxed(&a.hdr[kHdrGateLayoutDone], 0u);
    }
    __syncthreads();
    {   // exclusive scan of the rank totals; thread i owns a run of ranks
        const int per = (R + T_ - 1) / T_;
        int32_t mine = 0;
        for (int i = 0; i < per; ++i) {
            const int32_t d = tid * per + i;
            if (d < R) mine += s_total[d];
        }
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
                run += s_total[d];
            }
        }
    }
    __syncthreads();
    for (int32_t d = tid; d < R; d += T_) {
        int32_t run = s_off[d] + s_before[d];
#pragma unroll
        for (int v_ = 0; v_ < kLayoutWaves; ++v_) {
            const int32_t c = s_wh[v_ * R + d];
            s_wh[v_ * R + d] = run;
            run += c;
        }
    }
    __syncthreads();
    int32_t q[LR];
    tile_ranks<kLayoutWaves, LR, false>(p, ev, s_wh, q);
    store_positions<kLayoutWaves, LR, false>(a, tile, q, &bad_pos);
    const int64_t tok0 = tile * p.tile_tokens;
    if (tok0 % p.tps == 0)
        for (int32_t d = tid; d < R; d += T_) a.send_offset[(tok0 / p.tps) * R + d] = s_before[d];
    if (a.chunk_offset != nullptr && tok0 % p.tpc == 0)
        for (int32_t d = tid; d < R; d += T_) a.chunk_offset[(tok0 / p.tpc) * R + d] = s_before[d];
    for (int i = tid; i < n_e; i += T_) a.expert_count[e_lo + i] = s_eh[i];
    if (tile == 0) {
        for (int32_t d = tid; d < R; d += T_) {
            a.rank_count[d] = s_total[d];
            a.recv_offset[d] = s_off[d];
        }
        if (tid == 0) a.recv_offset[R] = (int32_t)p.rows;
    }
    if (bad) raise_status(a.status, UBEP_ERR_BAD_EXPERT_ID);
    if (bad_pos) raise_status(a.status, UBEP_ERR_BAD_POSITION);
}

hipError_t launch_layout_from_counts(const Plan& p, const int32_t* idx, int32_t* pos,
                                     int32_t* expert_count, int32_t* rank_count,
                                     int32_t* recv_offset, int32_t* send_offset,
                                     int32_t* chunk_offset, int32_t* recv_src, void* ws,
                                     hipStream_t stream) {
    LayoutArgs a{};
    a.idx = idx;
    a.pos = pos;
    a.expert_count = expert_count;
    a.rank_count = rank_count;
    a.recv_offset = recv_offset;
    a.send_offset = send_offset;
    a.chunk_offset = p.C > 1 ? chunk_offset : nullptr;
    a.recv_src = recv_src;
    a.expert_offset = nullptr;
    char* base = static_cast<char*>(ws);
    a.hdr = reinterpret_cast<uint32_t*>(base);
    a.p = p;
    a.status = a.hdr + kHdrStatus;
    int32_t* rc = reinterpret_cast<int32_t*>(base + p.off_gate_rank);
    int32_t* ec = reinterpret_cast<int32_t*>(base + p.off_gate_expert);
    const int64_t lane_rows = (p.tile_rows + kLayoutThreads - 1) / kLayoutThreads;
    const dim3 g((unsigned)p.n_tiles), b(kLayoutThreads);
    if (lane_rows <= 1) return launch_kernel(layout_counts_kernel<1>, g, b, 0, stream, a, rc, ec);
    if (lane_rows <= 2) return launch_kernel(layout_counts_kernel<2>, g, b, 0, stream, a, rc, ec);
    if (lane_rows <= 4) return launch_kernel(layout_counts_kernel<4>, g, b, 0, stream, a, rc, ec);
    return launch_kernel(layout_counts_kernel<8>, g, b, 0, stream, a, rc, ec);
}

// ---------------------------------------------------------------- allocation-free layout
// The workspace of ubep_layout_noalloc: one array per device for the life of
// the process, shared by every such call on that device.  Host code never
// uses its name as an address (on the host it names a stand-in): the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t layout_scratch(int device, void** out, bool* first_use) {
    static std::mutex mu;
    static void* ptr[kScratchMaxDevices] = {};
    if (device < 0 || device >= kScratchMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    *first_use = false;
    if (ptr[device] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        ptr[device] = p;
        *first_use = true;
    }
    *out = ptr[device];
    return hipSuccess;
}

hipError_t launch_layout(const Plan& p, const int32_t* idx, int32_t* pos, int32_t* expert_count,
                         int32_t* expert_offset, int32_t* rank_count, int32_t* recv_offset,
                         int32_t* send_offset, int32_t* chunk_offset, int32_t* recv_src, void* ws,
                         uint64_t spin_ticks, hipStream_t stream, uint32_t* status) {
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
    a.expert_offset = expert_offset;
    char* base = static_cast<char*>(ws);
    a.hdr = reinterpret_cast<uint32_t*>(base);
    a.state = reinterpret_cast<uint64_t*>(base + p.off_state);
    a.excl = reinterpret_cast<int32_t*>(base + p.off_excl);
    a.wbase = reinterpret_cast<int32_t*>(base + p.off_wbase);
    a.p = p;
    a.spin_ticks = spin_ticks;
    a.status = status != nullptr ? status : a.hdr + kHdrStatus;
    if (layout_fits_one_group(p)) {
        const int64_t tpw = (p.n_tiles + kSingleWaves - 1) / kSingleWaves;
        const int64_t steps = tpw * p.tile_rows / 64;
        if (steps <= 16)
            return launch_kernel(layout_single_kernel<16>, dim3(1), dim3(kSingleThreads), 0, stream, a);
        if (steps <= 32)
            return launch_kernel(layout_single_kernel<32>, dim3(1), dim3(kSingleThreads), 0, stream, a);
        return launch_kernel(layout_single_kernel<64>, dim3(1), dim3(kSingleThreads), 0, stream, a);
    }
    const int64_t lane_rows = (p.tile_rows + kLayoutThreads - 1) / kLayoutThreads;
    if (layout_replicates(p, idx)) {
        const int64_t nv = (p.rows / 4 + kLayoutThreads - 1) / kLayoutThreads;
        const auto rep = [&](auto lr_tag) -> hipError_t {
            constexpr int LR_ = decltype(lr_tag)::value;
            const dim3 g((unsigned)p.n_tiles), b(kLayoutThreads);
            if (p.order != 0) {
                if (nv <= 4) return launch_kernel(layout_replicated_kernel<LR_, 4, true>, g, b, 0, stream, a);
                if (nv <= 8) return launch_kernel(layout_replicated_kernel<LR_, 8, true>, g, b, 0, stream, a);
                return launch_kernel(layout_replicated_kernel<LR_, 16, true>, g, b, 0, stream, a);
            }
            if (nv <= 4) return launch_kernel(layout_replicated_kernel<LR_, 4, false>, g, b, 0, stream, a);
            if (nv <= 8) return launch_kernel(layout_replicated_kernel<LR_, 8, false>, g, b, 0, stream, a);
            return launch_kernel(layout_replicated_kernel<LR_, 16, false>, g, b, 0, stream, a);
        };
        static_assert(kRepMaxRows / 4 <= 16 * kLayoutThreads, "vectors per thread");
        if (lane_rows <= 1) return rep(std::integral_constant<int, 1>{});
        if (lane_rows <= 2) return rep(std::integral_constant<int, 2>{});
        if (lane_rows <= 4) return rep(std::integral_constant<int, 4>{});
        return rep(std::integral_constant<int, 8>{});
    }
    const int64_t lds = layout_lds_bytes(p, kLayoutWaves);
    const auto go = [&](void (*kernel)(LayoutArgs)) -> hipError_t {
        if (lds > 64 * 1024) {
            const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (err != hipSuccess) return err;
        }
        return launch_kernel(kernel, dim3((unsigned)layout_workers(p, di.cus)), dim3(kLayoutThreads),
                             (size_t)lds, stream, a);
    };
    static_assert(max_lane_rows<kLayoutWaves>() == 8, "tile rows per lane");
    if (p.order != 0) {
        if (lane_rows <= 1) return go(layout_kernel<1, true>);
        if (lane_rows <= 2) return go(layout_kernel<2, true>);
        if (lane_rows <= 4) return go(layout_kernel<4, true>);
        return go(layout_kernel<8, true>);
    }
    if (lane_rows <= 1) return go(layout_kernel<1, false>);
    if (lane_rows <= 2) return go(layout_kernel<2, false>);
    if (lane_rows <= 4) return go(layout_kernel<4, false>);
    return go(layout_kernel<8, false>);
}

}  // namespace ubep

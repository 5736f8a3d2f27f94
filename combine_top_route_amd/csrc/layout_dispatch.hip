// Layout and bf16 dispatch in one launch ("NJU x Huawei UBEP: Reengineering
// MoE Expert Parallelism", "Kernel Decomposition": a few cores compute the
// metadata -- token counts, prefix sums, offsets -- and publish it to global
// memory while the other cores move token data, polling that memory and
// starting the reorder as soon as the metadata is there, with no global
// barrier between the stages).
//
// Every workgroup moves the rows of one block of tokens (its block index for
// the workgroups that start together, the next block ticket for later ones).
// The first n_workers workgroups to find layout roles left also run the layout
// worker (layout_worker.h) first: a workgroup reads the role counter with a
// plain load and takes a role with an atomic only while the count is below
// n_workers, so the other workgroups never queue on that word.  Layout
// workers write pos with device-coherent stores and bump a "positions ready"
// counter; every workgroup loads its tokens' rows of x (data-only workgroups
// while the layout runs), polls the counter, reads its positions with
// device-coherent loads and stores the rows into the receive regions.
// A workgroup is data-only only once all n_workers roles are taken, by
// workgroups that were running when they took them and whose layout work
// never waits on row movement: no deadlock for any grid of at least n_workers
// workgroups.  The result equals ubep_layout followed by
// ubep_dispatch(UBEP_BF16).
#include "launch.h"
#include "layout_worker.h"
#include "rows.h"

namespace ubep {

constexpr int kFusedThreads = 256;
constexpr int kFusedWaves = kFusedThreads / 64;
constexpr int64_t kFusedLdsMax = 24 * 1024;     // keep data workers at full occupancy
constexpr int kFusedWindow = 32;                 // look-back window of the layout workers

// NTX: x read with non-temporal loads; row blocks from nt_from on store
// non-temporally (the dispatch kernel's policy, rows.h).
template <int G, int VPT, int LR, bool NTX>
__global__ __launch_bounds__(kFusedThreads) void layout_dispatch_kernel(LayoutArgs la,
                                                                       const u32x4* __restrict__ x,
                                                                       u32x4* __restrict__ recv,
                                                                       uint32_t n_workers,
                                                                       uint32_t n_static,
                                                                       uint32_t nt_from) {
    extern __shared__ int32_t dyn_lds[];
    __shared__ uint32_t s_role;
    __shared__ int32_t s_pos[kFusedThreads / 64 * kMaxK];
    const Plan& p = la.p;
    const int tid = threadIdx.x;
    uint32_t* status = &la.hdr[kHdrStatus];
    const uint32_t epoch = ld_relaxed(&la.hdr[kHdrLayoutEpoch]);
    if (tid == 0) {
        uint32_t role = 0xFFFFFFFFu;
        if (ld_relaxed(&la.hdr[kHdrRoleTicket]) < n_workers) {
            const uint32_t r = add_relaxed(&la.hdr[kHdrRoleTicket], 1u);
            if (r < n_workers) role = r;
        }
        s_role = role;
    }
    __syncthreads();
    const uint32_t role = s_role;
    const bool worker = role < n_workers;

    if (worker) {
        const LayoutLds L = carve_lds(dyn_lds, p, kFusedWaves);
        layout_worker<kFusedWaves, LR, true, kFusedWindow>(la, L, epoch, role, n_workers);
        wait_memory();                 // this workgroup's positions are at the coherent level
        __syncthreads();
        if (tid == 0) add_relaxed(&la.hdr[kHdrPosReady], 1u);
    }

    constexpr int TPB = kFusedThreads / G;
    const int grp = tid / G, gtid = tid % G;
    const uint32_t blk = claim_block(&la.hdr[kHdrFusedBlockTicket], n_static, status);
    const int64_t t = (int64_t)blk * TPB + grp;
    const bool live = t < p.T;
    const int64_t nvec = p.H / 8;
    const u32x4* xr = x + (live ? t : 0) * nvec;
    // the first pass of the row (loaded while the layout runs, for data-only
    // workgroups)
    u32x4 buf[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int64_t v = gtid + (int64_t)i * G;
        if (live && v < nvec) buf[i] = NTX ? __builtin_nontemporal_load(xr + v) : xr[v];
    }
    if (tid == 0) {
        const uint64_t t0 = now_ticks();
        while (ld_relaxed(&la.hdr[kHdrPosReady]) < n_workers) {
            if (now_ticks() - t0 > la.spin_ticks) {
                raise_status(status, UBEP_ERR_TIMEOUT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
    if (live && gtid < p.k)
        s_pos[grp * kMaxK + gtid] = __hip_atomic_load(la.pos + t * p.k + gtid, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (live) {
        for (int64_t v0 = 0; v0 < nvec; v0 += (int64_t)G * VPT) {
            if (v0 > 0) {
#pragma unroll
                for (int i = 0; i < VPT; ++i) {
                    const int64_t v = v0 + gtid + (int64_t)i * G;
                    if (v < nvec) buf[i] = NTX ? __builtin_nontemporal_load(xr + v) : xr[v];
                }
            }
            for (int32_t j = 0; j < p.k; ++j) {
                const int32_t q = s_pos[grp * kMaxK + j];
                if (!row_ok(q, p.rows)) {
                    if (gtid == 0 && v0 == 0) raise_status(status, UBEP_ERR_BAD_POSITION);
                    continue;
                }
                u32x4* dst = recv + (int64_t)q * nvec;
#pragma unroll
                for (int i = 0; i < VPT; ++i) {
                    const int64_t v = v0 + gtid + (int64_t)i * G;
                    if (v < nvec) {
                        if (blk >= nt_from) __builtin_nontemporal_store(buf[i], dst + v);
                        else dst[v] = buf[i];
                    }
                }
            }
        }
    }
    layout_finish(la, epoch);
}

bool layout_dispatch_fuses(const Plan& p) {
    return layout_lds_bytes(p, kFusedWaves) <= kFusedLdsMax &&
           p.tile_rows <= (int64_t)kFusedWaves * 64 * 16;
}

hipError_t launch_layout_dispatch(const Plan& p, const int32_t* idx, const void* x, int32_t* pos,
                                  int32_t* expert_count, int32_t* rank_count, int32_t* recv_offset,
                                  int32_t* send_offset, int32_t* chunk_offset, int32_t* recv_src,
                                  void* recv, void* ws, uint64_t spin_ticks, hipStream_t stream) {
    uint32_t* status = static_cast<uint32_t*>(ws) + kHdrStatus;
    if (!layout_dispatch_fuses(p)) {   // two launches, same result
        hipError_t e = launch_layout(p, idx, pos, expert_count, nullptr, rank_count, recv_offset,
                                     send_offset, chunk_offset, recv_src, ws, spin_ticks, stream);
        if (e != hipSuccess) return e;
        return launch_dispatch_bf16(p, x, pos, recv, status, stream);
    }
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
    a.expert_offset = nullptr;
    char* base = static_cast<char*>(ws);
    a.hdr = reinterpret_cast<uint32_t*>(base);
    a.state = reinterpret_cast<uint64_t*>(base + p.off_state);
    a.excl = reinterpret_cast<int32_t*>(base + p.off_excl);
    a.wbase = reinterpret_cast<int32_t*>(base + p.off_wbase);
    a.p = p;
    a.spin_ticks = spin_ticks;
    a.status = status;
    const uint32_t n_workers = (uint32_t)layout_workers(p, di.cus);
    const unsigned lds = (unsigned)layout_lds_bytes(p, kFusedWaves);
    int G, VPT;
    pick_group(p.H / 8, &G, &VPT);
    const int64_t lane_need = (p.tile_rows + kFusedWaves * 64 - 1) / (kFusedWaves * 64);
    auto go = [&]<int GG, int VV>() -> hipError_t {
        constexpr int TPB = kFusedThreads / GG;
        int64_t grid = (p.T + TPB - 1) / TPB;     // one block of tokens per workgroup
        if (grid < (int64_t)n_workers) grid = n_workers;
        const int64_t data_blocks = (p.T + TPB - 1) / TPB;
        const int64_t block_bytes = (int64_t)TPB * p.k * p.H * 2;   // receive rows a block writes
        const int64_t nt_blocks = (kNtTailBytes + block_bytes - 1) / block_bytes;
        const int64_t nt_from = data_blocks > nt_blocks ? data_blocks - nt_blocks : 0;
        const auto one = [&](auto kernel) -> hipError_t {
            int64_t n_static = 0;
            const hipError_t err = resident_blocks(reinterpret_cast<const void*>(kernel), kFusedThreads,
                                                   lds, &n_static);
            if (err != hipSuccess) return err;
            if (n_static > grid) n_static = grid;
            return launch_kernel(kernel, dim3((unsigned)grid), dim3(kFusedThreads), lds, stream, a,
                                 static_cast<const u32x4*>(x), static_cast<u32x4*>(recv), n_workers,
                                 (uint32_t)n_static, (uint32_t)nt_from);
        };
        const bool ntx = p.rows * p.H * 2 <= kNtxMaxBytes;
        if (lane_need <= 4)
            return ntx ? one(layout_dispatch_kernel<GG, VV, 4, true>) : one(layout_dispatch_kernel<GG, VV, 4, false>);
        if (lane_need <= 8)
            return ntx ? one(layout_dispatch_kernel<GG, VV, 8, true>) : one(layout_dispatch_kernel<GG, VV, 8, false>);
        return ntx ? one(layout_dispatch_kernel<GG, VV, 16, true>) : one(layout_dispatch_kernel<GG, VV, 16, false>);
    };
    return with_group(G, VPT, go);
}

}  // namespace ubep

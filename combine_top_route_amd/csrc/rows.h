// Per-token row routines for dispatch and combine.  A "group" of G threads
// (G a multiple of 64, so whole waves) handles one token; each thread moves
// VPT 16-byte vectors per pass, so one pass covers G*VPT vectors of the row.
#pragma once

#include "device_common.h"

namespace ubep {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ void store16(u32x4* p, u32x4 v) {
    if constexpr (NT) {
        __builtin_nontemporal_store(v, p);
    } else {
        *p = v;
    }
}

// Group size G (64, 128 or 256 threads: whole waves) and vectors per thread
// VPT for a row of `nvec` 16-byte vectors: the smallest group that covers the
// row in at most kVptCap vectors per thread; longer rows take several passes.
constexpr int kVptCap = 8;

inline void pick_group(int64_t nvec, int* G, int* VPT) {
    for (int g = 64; g <= 256; g *= 2) {
        if (nvec <= (int64_t)g * kVptCap) {
            *G = g;
            *VPT = (int)((nvec + g - 1) / g);
            return;
        }
    }
    *G = 256;
    *VPT = kVptCap;
}

// Calls F.template operator()<G, VPT>() for the runtime (G, VPT).
template <typename F>
inline hipError_t with_group(int G, int VPT, F&& f) {
#define UBEP_VPT_CASES(GG)                                                    \
    switch (VPT) {                                                            \
        case 1: return f.template operator()<GG, 1>();                        \
        case 2: return f.template operator()<GG, 2>();                        \
        case 3: return f.template operator()<GG, 3>();                        \
        case 4: return f.template operator()<GG, 4>();                        \
        case 5: return f.template operator()<GG, 5>();                        \
        case 6: return f.template operator()<GG, 6>();                        \
        case 7: return f.template operator()<GG, 7>();                        \
        default: return f.template operator()<GG, kVptCap>();                 \
    }
    switch (G) {
        case 64: UBEP_VPT_CASES(64)
        case 128: UBEP_VPT_CASES(128)
        default: UBEP_VPT_CASES(256)
    }
#undef UBEP_VPT_CASES
}

// ---- device-coherent row access for producer/consumer hand-offs inside one
// kernel.  A buffer resource spans exactly one row (hardware bounds check:
// stores past it are dropped, loads past it read zero).  Cache policy sc1
// (device scope) makes a store write through this XCD's L2 to the
// device-coherent level and makes a load bypass non-coherent cached copies --
// the same policy the compiler gives agent-scope atomics -- so a hand-off
// needs only "stores complete, then flag" on one side and "flag, then loads"
// on the other, with no L2 write-back or invalidate.
constexpr int kCachePolicyDevice = 16;   // sc1
constexpr int kCachePolicyNt = 2;        // nt: streaming, read once
constexpr int kBufferWord3 = 0x00020000; // raw 32-bit data format (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row, int64_t bytes) {
    // the row address is uniform across the wave; make that explicit for the
    // scalar resource registers
    const uint64_t a = (uint64_t)row;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* base = (void*)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, kBufferWord3);
}

__device__ __forceinline__ void store16_device(__amdgpu_buffer_rsrc_t r, int64_t v, u32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)(v * 16), 0, kCachePolicyDevice);
}

// The same with the non-temporal hint as well (rows nothing reads soon).
__device__ __forceinline__ void store16_device_nt(__amdgpu_buffer_rsrc_t r, int64_t v, u32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)(v * 16), 0, kCachePolicyDevice | kCachePolicyNt);
}

// The loads also carry the non-temporal hint (the rows are read once): on
// the 4096-token decode step the chunk pipeline took 399 against 427 us with
// it and the sentinel pipeline 215 against 261 us; at the 65536-token prefill
// 3.33 against 3.38 ms and 3.42 against 3.40 ms.  (Non-temporal device stores
// as well: 394 us, 241 us, 3.34 ms and 3.32 ms.)
__device__ __forceinline__ u32x4 load16_device(__amdgpu_buffer_rsrc_t r, int64_t v) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)(v * 16), 0, kCachePolicyDevice | kCachePolicyNt);
}

// Wait until this thread's memory operations have completed.
__device__ __forceinline__ void wait_memory() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Debug aid of the pipelines (debug flag bit 1): hold a producer back for
// about 25 us before it publishes, so that consumers find their data late.
// A fixed number of sleeps: it always ends.
constexpr uint32_t kDebugWithhold = 1u;   // bit 0: never publish (forces the time-out path)
constexpr uint32_t kDebugDelay = 2u;      // bit 1: publish late
__device__ __forceinline__ void debug_delay() {
#pragma unroll 1
    for (int i = 0; i < 8; ++i) __builtin_amdgcn_s_sleep(127);
}

__device__ __forceinline__ bool row_ok(int32_t q, int64_t n_rows) {
    return (uint64_t)(int64_t)q < (uint64_t)n_rows;
}

// Dispatch (and the fused layout + dispatch launch): the workgroups from
// nt_from on (the last ones to start) write their rows with
// non-temporal stores: the rows written last would otherwise still sit dirty
// in the L2s when the kernel ends, and the next kernel's loads would pay for
// writing them back.  The tail is 160 MB, five times the L2s' 32 MB, written
// while the grid drains and HBM has room.  On the 4096-token decode step (a
// step of layout, dispatch and combine from a cold cache) 128 MB took 178.2
// us against 182.0 (64 MB), 180.1 (192 MB) and 185.9 us (256 MB); with x
// read non-temporally as well, 160 MB took 176.5 us against 176.8 (128 MB)
// and 179.1 us (192 MB).
constexpr int64_t kNtTailBytes = 160ll << 20;

// Up to this many bytes of receive rows, x is read with non-temporal loads
// too: on the decode step that, with the tail above, left the combine that
// follows fewer lines to evict (step 177.5 -> 176.5 us cold, Zipf warm 184.0
// -> 180.0 us), while from 32768 tokens of H = 7168 (3.8 GB of rows) it made
// the dispatch itself 1.5 % slower; at 16384 tokens (1.9 GB) it changed
// nothing.  In the fused launch the two together took the decode step from
// 205.4 to 201.5 us cold; at the 65536-token prefill the tail alone changed
// nothing and non-temporal x reads cost 1.2 %.
constexpr int64_t kNtxMaxBytes = 2ll << 30;

// recv[pos[t][j]] = x[t] for j = 0..k-1 (bf16 bit copy, no relay buffer).
// NT: non-temporal stores (device-coherent ones too with COH).
// COH: write the rows with device-coherent stores (see above).  SKIP0: leave
// each row's first 16-byte unit unwritten (the caller stores it last).  NTX:
// read x with non-temporal loads.
template <int G, int VPT, bool NT, bool COH = false, bool SKIP0 = false, bool NTX = false>
__device__ __forceinline__ void dispatch_row_bf16(const u32x4* __restrict__ x,
                                                  const int32_t* __restrict__ pos,
                                                  u32x4* __restrict__ recv, int64_t t, int32_t k,
                                                  int64_t nvec, int64_t n_rows, int gtid,
                                                  uint32_t* status) {
    const int64_t tu = __builtin_amdgcn_readfirstlane((int32_t)t);   // uniform across the wave
    const u32x4* xr = x + tu * nvec;
    const int32_t* pr = pos + tu * k;
    for (int64_t v0 = 0; v0 < nvec; v0 += (int64_t)G * VPT) {
        u32x4 buf[VPT];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int64_t v = v0 + gtid + (int64_t)i * G;
            if (v < nvec) buf[i] = NTX ? __builtin_nontemporal_load(xr + v) : xr[v];
        }
        for (int32_t j = 0; j < k; ++j) {
            const int32_t q = pr[j];
            if (!row_ok(q, n_rows)) {
                if (gtid == 0 && v0 == 0) raise_status(status, UBEP_ERR_BAD_POSITION);
                continue;
            }
            u32x4* dst = recv + (int64_t)q * nvec;
            if constexpr (COH) {
                const __amdgpu_buffer_rsrc_t rs = row_rsrc(dst, nvec * 16);
#pragma unroll
                for (int i = 0; i < VPT; ++i) {
                    const int64_t v = v0 + gtid + (int64_t)i * G;
                    if (v < nvec && !(SKIP0 && v == 0)) {
                        if constexpr (NT) store16_device_nt(rs, v, buf[i]);
                        else store16_device(rs, v, buf[i]);
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < VPT; ++i) {
                    const int64_t v = v0 + gtid + (int64_t)i * G;
                    if (v < nvec) store16<NT>(dst + v, buf[i]);
                }
            }
        }
    }
}

// fp8 payload: each thread owns 16 channels (two 16-byte loads of bf16, one
// 16-byte store of codes); the 8 threads of a 128-channel block reduce amax
// with xor shuffles.  s = amax / 448 and x / s are IEEE fp32 divisions.
template <int G>
__device__ __forceinline__ void dispatch_row_fp8(const u32x4* __restrict__ x,
                                                 const int32_t* __restrict__ pos,
                                                 u32x4* __restrict__ recv8,
                                                 float* __restrict__ recv_scale, int64_t t,
                                                 int32_t k, int64_t H, int64_t n_rows, int gtid,
                                                 uint32_t* status) {
    const int64_t ng = H / 16;          // 16-channel groups per row
    const int64_t nb = H / 128;         // scale blocks per row
    const int64_t tu = __builtin_amdgcn_readfirstlane((int32_t)t);   // uniform across the wave
    const u32x4* xr = x + tu * (H / 8);
    const int32_t* pr = pos + tu * k;
    for (int64_t g = gtid; g < ng; g += G) {
        const u32x4 lo = xr[2 * g], hi = xr[2 * g + 1];
        float f[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(lo[i] << 16);
            f[2 * i + 1] = __uint_as_float(lo[i] & 0xFFFF0000u);
            f[8 + 2 * i] = __uint_as_float(hi[i] << 16);
            f[8 + 2 * i + 1] = __uint_as_float(hi[i] & 0xFFFF0000u);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
        const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
        u32x4 code;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            code[i] = f32_to_e4m3(f[4 * i] / s) | (f32_to_e4m3(f[4 * i + 1] / s) << 8) |
                      (f32_to_e4m3(f[4 * i + 2] / s) << 16) | (f32_to_e4m3(f[4 * i + 3] / s) << 24);
        }
        const bool leader = (g & 7) == 0;
        const int64_t b = g >> 3;
        for (int32_t j = 0; j < k; ++j) {
            const int32_t q = pr[j];
            if (!row_ok(q, n_rows)) {
                if (g == 0) raise_status(status, UBEP_ERR_BAD_POSITION);
                continue;
            }
            recv8[(int64_t)q * (H / 16) + g] = code;
            if (leader) recv_scale[(int64_t)q * nb + b] = s;
        }
    }
}

// out[t] = bf16(fma chain over slots 0..k-1 of topk_w[t][j] * y[pos[t][j]])
// in fp32 from +0.0f.  Slots are taken KB at a time: the KB row loads are
// issued together, unconditionally, from addresses that are always valid (a
// slot past k or with a position outside [0, T*k) reads row 0 and is skipped
// in the chain), so no load waits behind another.  The rows of y are read
// once, so they are loaded non-temporally (they need not displace other lines
// from the caches).  COH: read them with device-coherent loads instead.
// Slot metadata of one batch: the receive row to read (always valid) and
// whether the slot takes part in the chain.
template <int KB>
__device__ __forceinline__ void slot_batch(const int32_t* pr, int32_t j0, int32_t k, int64_t n_rows,
                                           int64_t (&row)[KB], bool (&use)[KB], bool* bad) {
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
        const int32_t j = j0 + jj;
        const int32_t q = pr[j < k ? j : k - 1];
        const bool ok = row_ok(q, n_rows);
        *bad |= (j < k) && !ok;
        use[jj] = (j < k) && ok;
        row[jj] = ok ? (int64_t)q : 0;
    }
}

// The KB rows' vectors v of one batch, loaded together.
template <int KB, bool COH>
__device__ __forceinline__ void load_batch(const u32x4* __restrict__ y, int64_t nvec, int64_t v,
                                           const int64_t (&row)[KB], u32x4 (&r)[KB]) {
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
        if constexpr (COH)
            r[jj] = load16_device(row_rsrc(y + row[jj] * nvec, nvec * 16), v);
        else
            r[jj] = __builtin_nontemporal_load(y + row[jj] * nvec + v);
    }
}

// acc[c] = fma(w_j, r_j channel c, acc[c]) for the used slots of a batch, in
// slot order.
template <int KB>
__device__ __forceinline__ void fma_batch(const u32x4 (&r)[KB], const bool (&use)[KB],
                                          const float* wr, float (&acc)[8]) {
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
        if (!use[jj]) continue;
        const float wj = wr[jj];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            acc[2 * c] = __builtin_fmaf(wj, __uint_as_float(r[jj][c] << 16), acc[2 * c]);
            acc[2 * c + 1] = __builtin_fmaf(wj, __uint_as_float(r[jj][c] & 0xFFFF0000u), acc[2 * c + 1]);
        }
    }
}

__device__ __forceinline__ u32x4 pack_bf16x8(const float (&acc)[8]) {
    u32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = f32_to_bf16(acc[2 * c]) | (f32_to_bf16(acc[2 * c + 1]) << 16);
    return o;
}

// PIPE: when k <= KB, software-pipeline the thread's vectors (kPipeDepth * KB
// more registers of loads in flight).
constexpr int kPipeDepth = 2;
template <int G, int VPT, int KB, bool COH = false, bool PIPE = true>
__device__ __forceinline__ void combine_row(const u32x4* __restrict__ y,
                                            const int32_t* __restrict__ pos,
                                            const float* __restrict__ w, u32x4* __restrict__ out,
                                            int64_t t_in, int32_t k, int64_t nvec, int64_t n_rows,
                                            int gtid, uint32_t* status) {
    // a group is whole waves, so the token is uniform across the wave: say so,
    // which turns the slot metadata reads into scalar loads
    const int64_t t = __builtin_amdgcn_readfirstlane((int32_t)t_in);
    const int32_t* pr = pos + t * k;
    const float* wr = w + t * k;
    bool bad = false;
    int64_t row0[KB];
    bool use0[KB];
    slot_batch<KB>(pr, 0, k, n_rows, row0, use0, &bad);
    if (PIPE && k <= KB) {
        // one batch holds every slot: software-pipeline the thread's vectors,
        // so the loads of the next kPipeDepth vectors are in flight while
        // this one is reduced
        constexpr int D = kPipeDepth;
        for (int64_t v0 = 0; v0 < nvec; v0 += (int64_t)G * VPT) {
            u32x4 r[D + 1][KB];
#pragma unroll
            for (int i = 0; i < D && i < VPT; ++i) {
                const int64_t v_raw = v0 + gtid + (int64_t)i * G;
                load_batch<KB, COH>(y, nvec, v_raw < nvec ? v_raw : 0, row0, r[i]);
            }
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                if (i + D < VPT) {
                    const int64_t v_raw = v0 + gtid + (int64_t)(i + D) * G;
                    load_batch<KB, COH>(y, nvec, v_raw < nvec ? v_raw : 0, row0, r[(i + D) % (D + 1)]);
                }
                float acc[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
                fma_batch<KB>(r[i % (D + 1)], use0, wr, acc);
                const int64_t v = v0 + gtid + (int64_t)i * G;
                if (v < nvec) out[t * nvec + v] = pack_bf16x8(acc);
            }
        }
    } else {
        for (int64_t v0 = 0; v0 < nvec; v0 += (int64_t)G * VPT) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int64_t v_raw = v0 + gtid + (int64_t)i * G;
                const bool v_ok = v_raw < nvec;
                const int64_t v = v_ok ? v_raw : 0;
                float acc[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
                u32x4 r[KB];
                load_batch<KB, COH>(y, nvec, v, row0, r);
                fma_batch<KB>(r, use0, wr, acc);
                for (int32_t j0 = KB; j0 < k; j0 += KB) {     // later batches
                    int64_t row[KB];
                    bool use[KB];
                    slot_batch<KB>(pr, j0, k, n_rows, row, use, &bad);
                    load_batch<KB, COH>(y, nvec, v, row, r);
                    fma_batch<KB>(r, use, wr + j0, acc);
                }
                if (v_ok) out[t * nvec + v] = pack_bf16x8(acc);
            }
        }
    }
    if (bad && gtid == 0) raise_status(status, UBEP_ERR_BAD_POSITION);
}

}  // namespace ubep

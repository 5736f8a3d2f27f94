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

__device__ __forceinline__ bool row_ok(int32_t q, int64_t n_rows) {
    return (uint64_t)(int64_t)q < (uint64_t)n_rows;
}

// recv[pos[t][j]] = x[t] for j = 0..k-1 (bf16 bit copy, no relay buffer).
template <int G, int VPT, bool NT>
__device__ __forceinline__ void dispatch_row_bf16(const u32x4* __restrict__ x,
                                                  const int32_t* __restrict__ pos,
                                                  u32x4* __restrict__ recv, int64_t t, int32_t k,
                                                  int64_t nvec, int64_t n_rows, int gtid,
                                                  uint32_t* status) {
    const u32x4* xr = x + t * nvec;
    const int32_t* pr = pos + t * k;
    for (int64_t v0 = 0; v0 < nvec; v0 += (int64_t)G * VPT) {
        u32x4 buf[VPT];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int64_t v = v0 + gtid + (int64_t)i * G;
            if (v < nvec) buf[i] = xr[v];
        }
        for (int32_t j = 0; j < k; ++j) {
            const int32_t q = pr[j];
            if (!row_ok(q, n_rows)) {
                if (gtid == 0 && v0 == 0) raise_status(status, UBEP_ERR_BAD_POSITION);
                continue;
            }
            u32x4* dst = recv + (int64_t)q * nvec;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int64_t v = v0 + gtid + (int64_t)i * G;
                if (v < nvec) store16<NT>(dst + v, buf[i]);
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
    const u32x4* xr = x + t * (H / 8);
    const int32_t* pr = pos + t * k;
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
// in fp32 from +0.0f.  Slots are loaded KB at a time so their loads are in
// flight together; the FMAs then run in slot order.
template <int G, int VPT, int KB>
__device__ __forceinline__ void combine_row(const u32x4* __restrict__ y,
                                            const int32_t* __restrict__ pos,
                                            const float* __restrict__ w, u32x4* __restrict__ out,
                                            int64_t t, int32_t k, int64_t nvec, int64_t n_rows,
                                            int gtid, uint32_t* status) {
    const int32_t* pr = pos + t * k;
    const float* wr = w + t * k;
    for (int64_t v0 = 0; v0 < nvec; v0 += (int64_t)G * VPT) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int64_t v = v0 + gtid + (int64_t)i * G;
            if (v >= nvec) continue;
            float acc[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
            for (int32_t j0 = 0; j0 < k; j0 += KB) {
                u32x4 r[KB];
                bool ok[KB];
#pragma unroll
                for (int jj = 0; jj < KB; ++jj) {
                    const int32_t j = j0 + jj;
                    ok[jj] = false;
                    if (j < k) {
                        const int32_t q = pr[j];
                        ok[jj] = row_ok(q, n_rows);
                        if (ok[jj]) r[jj] = y[(int64_t)q * nvec + v];
                        else if (v == gtid) raise_status(status, UBEP_ERR_BAD_POSITION);
                    }
                }
#pragma unroll
                for (int jj = 0; jj < KB; ++jj) {
                    if (!ok[jj]) continue;
                    const float wj = wr[j0 + jj];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        acc[2 * c] = __builtin_fmaf(wj, __uint_as_float(r[jj][c] << 16), acc[2 * c]);
                        acc[2 * c + 1] =
                            __builtin_fmaf(wj, __uint_as_float(r[jj][c] & 0xFFFF0000u), acc[2 * c + 1]);
                    }
                }
            }
            u32x4 o;
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] = f32_to_bf16(acc[2 * c]) | (f32_to_bf16(acc[2 * c + 1]) << 16);
            out[t * nvec + v] = o;
        }
    }
}

}  // namespace ubep

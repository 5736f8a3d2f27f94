// Device-side helpers for the gfx950 dispatch / combine kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace ubep {

// ---------------------------------------------------------------- wave64 helpers
__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

// Lanes of the wave whose `key` equals this lane's key, restricted to
// `active`.  One ballot per key bit (a wave-level multisplit): the result for
// a lane is the AND over bits b of (ballot(bit b) if this lane's bit b is set,
// else its complement).  Every lane of the wave must call this.
__device__ __forceinline__ uint64_t peers_of(uint32_t key, int bits, uint64_t active) {
    uint64_t m = active;
    for (int b = 0; b < bits; ++b) {
        const uint32_t bit = (key >> b) & 1u;
        const uint64_t bal = __ballot(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

// peers_of with the bit loop unrolled to MAXB (bits <= MAXB, uniform).
template <int MAXB>
__device__ __forceinline__ uint64_t peers_of_n(uint32_t key, int bits, uint64_t active) {
    uint64_t m = active;
#pragma unroll
    for (int b = 0; b < MAXB; ++b) {
        if (b < bits) {
            const uint32_t bit = (key >> b) & 1u;
            const uint64_t bal = __ballot(bit);
            m &= bit ? bal : ~bal;
        }
    }
    return m;
}

// Destination rank of expert e: floor(e / epr) by multiply-high with the
// host-computed magic ceil(2^32 / epr) (exact for e * epr < 2^32).
__device__ __forceinline__ uint32_t rank_of(uint32_t e, uint32_t magic) {
    return magic == 0u ? e : __umulhi(e, magic);
}

// ---------------------------------------------------------------- number formats
// bf16 is the top half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round an fp32 (finite) to the nearest bf16, ties to even: add just under half
// a bf16 unit plus the kept LSB, then truncate.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// OCP E4M3FN encode (bias 7, max 448, no infinity), nearest with ties to even,
// saturating to +-448.  Finite inputs.
//  - |f| >= 448          -> 0x7E
//  - |f| <  2^-6         -> subnormal code m = rint(|f| * 2^9) in 0..8
//                           (8 is the smallest normal, code 0x08)
//  - otherwise           -> round the fp32 mantissa to 3 bits at bit 20
//                           (ties to even) and rebias the exponent 127 -> 7.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a >= 0x43E00000u) {                 // 448.0
        code = 0x7Eu;
    } else if (a < 0x3C800000u) {           // 2^-6
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    } else {
        const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        code = r - ((127u - 7u) << 3);
    }
    return sign | code;
}

// OCP E4M3FN decode.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t sign = (c & 0x80u) << 24;
    const uint32_t X = (c >> 3) & 15u, M = c & 7u;
    float v;
    if (X == 15u && M == 7u) return __uint_as_float(0x7FC00000u | sign);
    if (X == 0u) v = (float)M * 0.001953125f;                 // M/8 * 2^-6
    else v = __uint_as_float(((X + 120u) << 23) | (M << 20));  // (1 + M/8) 2^(X-7)
    return __uint_as_float(__float_as_uint(v) | sign);
}

// ---------------------------------------------------------------- atomics (vector memory ops)
__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_acquire(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_relaxed(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_release(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_acq_rel(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t ld_relaxed64(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// First error wins; later ones are dropped.
__device__ __forceinline__ void raise_status(uint32_t* status, uint32_t code) {
    uint32_t expected = 0u;
    __hip_atomic_compare_exchange_strong(status, &expected, code, __ATOMIC_RELAXED,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Constant-rate device clock used for bounded waits.
// Block of work of this workgroup.  The first n_static workgroups (about the
// ones that fit on the chip at once, which start together) take their own
// index.  Later workgroups start one by one as slots free up and take the next
// ticket of *ctr: blocks then go out in the order workgroups start, whichever
// XCD runs them, so the rows in flight stay close together in memory even
// when the XCDs drift apart.  The workgroup that draws the last ticket (all
// others have drawn theirs) resets *ctr for the next call.  A ticket past the
// end means a call that never finished left *ctr behind: the workgroup then
// gets no block and reports UBEP_ERR_WORKSPACE.
__device__ __forceinline__ uint32_t claim_block(uint32_t* ctr, uint32_t n_static, uint32_t* status) {
    __shared__ uint32_t s_block;
    if (blockIdx.x < n_static) return blockIdx.x;      // uniform across the workgroup
    if (threadIdx.x == 0) {
        const uint32_t n_dyn = gridDim.x - n_static;
        const uint32_t tk = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tk == n_dyn - 1u) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tk >= n_dyn) raise_status(status, UBEP_ERR_WORKSPACE);
        s_block = tk < n_dyn ? n_static + tk : gridDim.x;
    }
    __syncthreads();
    return s_block;
}

__device__ __forceinline__ uint64_t now_ticks() { return wall_clock64(); }

}  // namespace ubep

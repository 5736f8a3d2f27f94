// Per-expert linear map on the expert-grouped receive rows: the real expert
// computation that sits between dispatch and combine (the opening section of
// "NJU x Huawei UBEP: Reengineering MoE Expert Parallelism": each token is
// processed by the experts it selected and the results are gathered back).
//
//   y[r][n] = bf16( sum over c of x[r][c] * w[e][n][c] )   for r in expert e's run
//
// The weights come packed (expert_pack_kernel): each k step of an output tile
// reads one contiguous 16 KB block, so the weight stream, the bulk of the
// bytes when few rows reach each expert, is sequential per workgroup instead
// of 128 rows read 128 bytes at a time (scattered rows thrash the HBM row
// buffers: half the bandwidth).
//
// A dense contraction per expert, so it runs on the matrix cores:
// v_mfma_f32_16x16x32_bf16 (gfx950) with fp32 accumulation.  A workgroup of
// 8 waves computes a 256 (output channels) x BM (rows, 128 or 192) tile of
// one expert; each wave a 64 x BM/2 part as 4 x BM/32 MFMA tiles.  The wide
// output tile matters: every output tile re-reads the expert's receive rows
// from L2, and at 128 channels that re-read traffic equalled the weight
// stream itself.  The weight rows are the MFMA's A operand and the receive
// rows its B operand, both read as 16-byte runs of 8 channels, so each lane's
// 4 accumulator values are 4 consecutive output channels of one row (one
// 8-byte store).  k steps of 64 channels are staged through two LDS stages
// (16-byte units swizzled per row pair): step s+1 is written while step s is
// multiplied, and the weight loads run two steps ahead.
//
// Rows past a run's end are loaded as zeros and not stored.  Consecutive
// workgroups share a row tile and walk the output channels, so the tile's
// receive rows stay in L2 while the weights stream.
#include <utility>

#include "launch.h"
#include "rows.h"

namespace ubep {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 512;       // 8 waves: 4 along the output channels x 2 along the rows
constexpr int kBN = 256;                 // output channels per tile
constexpr int kPackN = 128;              // output channels per packed weight block
constexpr int kBShort = 128;             // rows per tile of experts with at most this many rows
constexpr int kBTall = 192;              // rows per tile of the others
constexpr int kBK = 64;                  // channels per k step
constexpr int kWDepth = 2;               // weight steps in flight (register sets)
constexpr int kUnroll = kWDepth % 2 == 0 ? kWDepth : 2 * kWDepth;   // a multiple of 2 and kWDepth
constexpr int kLdsStride = kBK;          // bf16 per LDS row: 128 bytes, 16-byte units swizzled
static_assert(kBK == 64, "the LDS swizzle permutes the 8 units of a 64-channel row");

// LDS element offset of 16-byte unit u of tile row r.  Rows are 128 bytes, so
// an even and an odd row together span the 64 banks; unit u of row r sits at
// position u ^ ((r / 2) % 8).  A quarter wave's stores (two rows) and its
// fragment loads (16 rows at one unit) then each touch every bank once.
__device__ __forceinline__ int lds_at(int r, int u) { return r * kLdsStride + ((u ^ ((r >> 1) & 7)) << 3); }
constexpr int kPerThreadE = kExpertMaxE / kGemmThreads;
constexpr int kVecPerRow = kBK / 8;                          // 16-byte vectors per tile row
constexpr int kLoadsW = kBN * kVecPerRow / kGemmThreads;     // weight vectors per thread and step
template <int BM>
constexpr int loads_x() { return BM * kVecPerRow / kGemmThreads; }   // receive-row vectors per thread and step

struct ExpertArgs {
    const int32_t* eoff;     // [E+1]
    const u32x4* x;          // [n_rows][H/8]
    const u32x4* w;          // packed [E][N/128][H/64][128][64 / 8]
    uint2* y;                // [n_rows][N/4]
    uint32_t* status;
    int64_t H, N, n_rows;
    int32_t E;
};

__device__ __forceinline__ uint2 pack_bf16x4(f32x4 v) {
    uint2 o;
    o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
    o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
    return o;
}

// One tile: rows [r_lo, min(r_lo + BM, r_end)) of expert e (a run ending at
// r_end), output channels [256 nt, 256 nt + 256).  Run by the whole workgroup.
// NTW: the expert has this one row tile, so its weights are read once and
// are loaded non-temporally (they then do not push out the receive rows,
// which every output tile of the expert reads again); an expert with several
// row tiles keeps its weights cacheable for the others.
template <int BM, bool NTW>
__device__ __forceinline__ void expert_tile(const ExpertArgs& a, int32_t e, int64_t r_lo, int64_t r_end,
                                            int64_t nt, uint16_t* s_dyn) {
    constexpr int kBM = BM;
    constexpr int kLoadsX = loads_x<BM>();
    constexpr int JT = BM / 32;                          // 16-row MFMA tiles per wave (two waves share the rows)
    // two LDS stages of (weights, receive rows): step kt+1 is written while
    // step kt is multiplied, one barrier per k step
    constexpr int kStage = (kBN + BM) * kLdsStride;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n0 = nt * kBN;

    // ---- k loop
    // Buffer resources over the tile's 128 weight rows and its receive rows
    // (at most 128; loads past the run's end read zeros).  Each lane's row and
    // vector offset stays in one VGPR per load; the k step is a scalar offset.
    const int64_t nvh = a.H / 8;
    const int32_t row_bytes = (int32_t)(a.H * 2);
    const int64_t n_x = r_end - r_lo < kBM ? r_end - r_lo : kBM;
    // packed weights: the (expert, output tile) block holds the tile's k steps
    // back to back, each a row-major 128 x 64 bf16 block of 16 KB
    const int64_t n_ksteps = a.H / kBK;
    // this tile's output channels are two packed blocks, adjacent in memory
    // (one when N is an odd number of blocks and this is the last tile: the
    // second half then loads zeros and stores nothing)
    const int64_t nblk = a.N / kPackN, b0 = 2 * nt;
    const int64_t halves = nblk - b0 < 2 ? nblk - b0 : 2;
    const int64_t blk_bytes = n_ksteps * kPackN * kBK * 2;
    const u32x4* wblk = a.w + ((int64_t)e * nblk + b0) * n_ksteps * (kPackN * kVecPerRow);
    const __amdgpu_buffer_rsrc_t rw = row_rsrc(wblk, halves * blk_bytes);
    const __amdgpu_buffer_rsrc_t rx = row_rsrc(a.x + r_lo * nvh, n_x * row_bytes);
    // The weights come from HBM and get kWDepth register sets: the loads of
    // step s+1+kWDepth are issued while step s is multiplied.  The receive
    // rows are mostly L2 hits (every output tile of the expert reads them)
    // and get one set, loaded a step ahead.
    u32x4 pw[kWDepth][kLoadsW], px[kLoadsX];
    int32_t xoff[kLoadsX];
#pragma unroll
    for (int i = 0; i < kLoadsX; ++i) {
        const int q = tid + kGemmThreads * i;            // kBM rows x kVecPerRow vectors
        xoff[i] = (q / kVecPerRow) * row_bytes + (q % kVecPerRow) * 16;
    }
    constexpr int kVecPerBlock = kPackN * kVecPerRow;   // vectors of one block's k step
    auto load_w = [&](int64_t kt, u32x4 (&dw)[kLoadsW]) {
        const int32_t wso = (int32_t)(kt * (kPackN * kBK * 2));
#pragma unroll
        for (int i = 0; i < kLoadsW; ++i) {  // a contiguous 16 KB run of each block per step
            const int q = tid + kGemmThreads * i;
            const int32_t half = q / kVecPerBlock;       // a constant per i
            dw[i] = __builtin_amdgcn_raw_buffer_load_b128(
                rw, (int32_t)(half * blk_bytes) + (q % kVecPerBlock) * 16, wso, NTW ? kCachePolicyNt : 0);
        }
    };
    auto load_x = [&](int64_t kt, u32x4 (&dx)[kLoadsX]) {
        const int32_t xso = (int32_t)(kt * (kBK * 2));
#pragma unroll
        for (int i = 0; i < kLoadsX; ++i)
            dx[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[i], xso, 0);
    };
    auto write_stage = [&](int b, const u32x4 (&sw)[kLoadsW], const u32x4 (&sx)[kLoadsX]) {
        uint16_t* s_w = s_dyn + b * kStage;
        uint16_t* s_x = s_w + kBN * kLdsStride;
#pragma unroll
        for (int i = 0; i < kLoadsW; ++i) {
            const int q = tid + kGemmThreads * i;
            *reinterpret_cast<u32x4*>(&s_w[lds_at(q / kVecPerRow, q % kVecPerRow)]) = sw[i];
        }
#pragma unroll
        for (int i = 0; i < kLoadsX; ++i) {
            const int q = tid + kGemmThreads * i;
            *reinterpret_cast<u32x4*>(&s_x[lds_at(q / kVecPerRow, q % kVecPerRow)]) = sx[i];
        }
    };
    f32x4 acc[4][JT];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JT; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int wn = (wave & 3) * 64, wm = (wave >> 2) * (BM / 2);
    const int fr = lane & 15, fk = (lane >> 4) * 8;      // fragment row and channel offset
    auto multiply = [&](int b) {
        const uint16_t* s_w = s_dyn + b * kStage;
        const uint16_t* s_x = s_w + kBN * kLdsStride;
#pragma unroll
        for (int ks = 0; ks < kBK; ks += 32) {
            bf16x8 fa[4], fb[JT];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fa[i] = *reinterpret_cast<const bf16x8*>(&s_w[lds_at(wn + 16 * i + fr, (ks + fk) >> 3)]);
#pragma unroll
            for (int j = 0; j < JT; ++j)
                fb[j] = *reinterpret_cast<const bf16x8*>(&s_x[lds_at(wm + 16 * j + fr, (ks + fk) >> 3)]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < JT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    };
    const int64_t nk = n_ksteps;
    // Step s multiplies LDS stage s % 2, writes step s+1 (weight set
    // (s+1) % kWDepth, the receive-row set) into the other stage, whose last
    // reader passed the previous barrier, and refills the two register sets
    // it emptied.  Unrolled by kUnroll so that every set index is a constant.
    // Every load is unconditional, its step clamped to the last one (a repeat
    // of the last step is an L2 hit): with no branch around a load, the
    // compiler's wait counts stay exact, so a step waits only for the loads
    // it consumes and not for the ones just issued for later steps.  The
    // prologue issues in the steady state's order: W(s+1), X(s+1), W(s+2).
    const int64_t last = nk - 1;
    auto clamp = [&](int64_t s_) { return s_ < last ? s_ : last; };
    auto step = [&](int64_t s_, auto jc) {
        constexpr int J = decltype(jc)::value;
        multiply(J % 2);
        write_stage((J + 1) % 2, pw[(J + 1) % kWDepth], px);   // step s+1 (unused after the last)
        load_x(clamp(s_ + 2), px);
        load_w(clamp(s_ + 1 + kWDepth), pw[(J + 1) % kWDepth]);
        __syncthreads();
    };
    auto steps = [&]<int... J>(int64_t kt, std::integer_sequence<int, J...>) {
        (step(kt + J, std::integral_constant<int, J>{}), ...);
    };
    auto first_steps = [&]<int... J>(int64_t kt, std::integer_sequence<int, J...>) {
        (void)((kt + J < nk && (step(kt + J, std::integral_constant<int, J>{}), true)) && ...);
    };
    // (scheduling barriers keep that order: the compiler may not merge the
    // groups and move a load the loop waits for behind one it does not)
    load_w(0, pw[0]);
    load_x(0, px);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 1; d < kWDepth; ++d) load_w(clamp(d), pw[d]);
    __builtin_amdgcn_sched_barrier(0);
    write_stage(0, pw[0], px);
    load_x(clamp(1), px);
    __builtin_amdgcn_sched_barrier(0);
    load_w(clamp(kWDepth), pw[0]);
    __syncthreads();
    // whole groups of kUnroll steps in the loop (no exit between its steps,
    // so the loop head sees one pattern of pending loads), the rest after it
    int64_t kt = 0;
    for (; kt + kUnroll <= nk; kt += kUnroll) steps(kt, std::make_integer_sequence<int, kUnroll>{});
    first_steps(kt, std::make_integer_sequence<int, kUnroll>{});

    // ---- epilogue: lane holds channels n .. n+3 of row r for each (i, j)
    const int64_t nq = a.N / 4;
#pragma unroll
    for (int j = 0; j < JT; ++j) {
        const int64_t r = r_lo + wm + 16 * j + fr;
        if (r >= r_end) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t n = n0 + wn + 16 * i + (lane >> 4) * 4;
            if (n < a.N) a.y[r * nq + n / 4] = pack_bf16x4(acc[i][j]);
        }
    }
}

// The tile-selection words of the prologue sit in LDS stage 1 of both tile
// heights, which a tile first writes after the barrier that ends its own
// prologue (so every read of them has happened).
constexpr int kSelAt = (kBN + kBTall) * kLdsStride;
static_assert(kSelAt >= (kBN + kBShort) * kLdsStride && kSelAt + 64 <= 2 * (kBN + kBShort) * kLdsStride,
              "the selection words lie in stage 1 of both tile heights");

// Tiles: blockIdx.x is the output-channel tile, blockIdx.y a row tile: first
// the 192-row tiles of the experts above 128 rows (the longer tiles start
// first), then one 128-row tile per expert of 1 to 128 rows.  An expert whose
// rows need two tiles streams its weights twice, so experts above 128 rows
// (about half of them in a decode step of 128 rows per expert) take 192-row
// tiles, while the others multiply no more zero rows than they must.  Each
// workgroup finds its expert and tile from expert_offset with one
// workgroup-wide scan, so no host round trip is needed between the layout
// and this kernel.
__global__ __launch_bounds__(kGemmThreads, 2) void expert_linear_kernel(ExpertArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t s_dyn[];
    constexpr int W = kGemmThreads / 64;
    int32_t* s_wsum = reinterpret_cast<int32_t*>(s_dyn + kSelAt);   // [2][W]: tall, short
    int32_t* s_sel = s_wsum + 2 * W;                                   // expert, tile within it
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t m = (int32_t)blockIdx.y;

    // offsets must run non-decreasing from 0 within [0, n_rows]; an expert
    // whose run is reversed gets no tiles, and workgroup (0, 0) reports any
    // violation (the tiles are then no longer sure to cover every run)
    int32_t ct[kPerThreadE], cs[kPerThreadE];
    int32_t mt = 0, ms = 0;
    bool bad_off = false;
#pragma unroll
    for (int i = 0; i < kPerThreadE; ++i) {
        const int32_t e = tid * kPerThreadE + i;
        ct[i] = cs[i] = 0;
        if (e < a.E) {
            const int32_t lo = a.eoff[e], hi = a.eoff[e + 1];
            const int32_t rows = hi - lo;
            if (rows < 0 || lo < 0 || (int64_t)hi > a.n_rows || (e == 0 && lo != 0)) bad_off = true;
            if (rows > kBShort) ct[i] = (rows + kBTall - 1) / kBTall;
            else if (rows > 0) cs[i] = 1;
        }
        mt += ct[i];
        ms += cs[i];
    }
    if (bad_off && blockIdx.x == 0 && blockIdx.y == 0) raise_status(a.status, UBEP_ERR_BAD_POSITION);
    int32_t it = mt, is = ms;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t ut = __shfl_up(it, o, 64), us = __shfl_up(is, o, 64);
        if (lane >= o) {
            it += ut;
            is += us;
        }
    }
    if (lane == 63) {
        s_wsum[wave] = it;
        s_wsum[W + wave] = is;
    }
    if (tid == 0) s_sel[0] = -1;
    __syncthreads();
    int32_t tall_total = 0, run_t = it - mt, run_s = is - ms;
    for (int i = 0; i < W; ++i) {
        tall_total += s_wsum[i];
        if (i < wave) {
            run_t += s_wsum[i];
            run_s += s_wsum[W + i];
        }
    }
    const bool tall = m < tall_total;                    // uniform
    const int32_t mm = tall ? m : m - tall_total;
#pragma unroll
    for (int i = 0; i < kPerThreadE; ++i) {
        const int32_t c = tall ? ct[i] : cs[i], r = tall ? run_t : run_s;
        if (c > 0 && mm >= r && mm < r + c) {
            s_sel[0] = tid * kPerThreadE + i;
            s_sel[1] = mm - r;
        }
        run_t += ct[i];
        run_s += cs[i];
    }
    __syncthreads();
    const int32_t e = s_sel[0];
    if (e < 0) return;                                   // past the last tile (uniform)
    const int64_t run_lo = a.eoff[e], r_end = a.eoff[e + 1];
    if (run_lo < 0 || r_end > a.n_rows) {                // inconsistent offsets
        if (tid == 0) raise_status(a.status, UBEP_ERR_BAD_POSITION);
        return;
    }
    const int64_t tile = s_sel[1];
    if (!tall)
        expert_tile<kBShort, true>(a, e, run_lo + tile * kBShort, r_end, blockIdx.x, s_dyn);
    else if (r_end - run_lo <= kBTall)
        expert_tile<kBTall, true>(a, e, run_lo + tile * kBTall, r_end, blockIdx.x, s_dyn);
    else
        expert_tile<kBTall, false>(a, e, run_lo + tile * kBTall, r_end, blockIdx.x, s_dyn);
}

// packed[e][nt][kt][r][c] = w[e][nt*128 + r][kt*64 + c]: every 128 x 64 block
// that one k step of one output tile reads becomes 16 contiguous KB.  One
// thread moves one 16-byte vector (8 channels).
__global__ __launch_bounds__(256) void expert_pack_kernel(const u32x4* __restrict__ w,
                                                          u32x4* __restrict__ packed, int64_t N,
                                                          int64_t H, int64_t total) {
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // packed vector index
    if (v >= total) return;
    const int64_t vpb = kPackN * kVecPerRow;                // vectors per 128 x 64 block
    const int64_t blk = v / vpb, in = v % vpb;
    const int64_t r = in / kVecPerRow, cv = in % kVecPerRow;
    const int64_t ksteps = H / kBK, ntiles = N / kPackN;
    const int64_t kt = blk % ksteps, nt = (blk / ksteps) % ntiles, e = blk / (ksteps * ntiles);
    const int64_t n = nt * kPackN + r;
    packed[v] = w[(e * N + n) * (H / 8) + kt * kVecPerRow + cv];
}

hipError_t launch_expert_pack(int32_t E, int64_t N, int64_t H, const void* w, void* packed,
                              hipStream_t stream) {
    const int64_t total = (int64_t)E * N * H / 8;
    const int64_t blocks = (total + 255) / 256;
    return launch_kernel(expert_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                         static_cast<const u32x4*>(w), static_cast<u32x4*>(packed), N, H, total);
}

// two stages of the taller tile: more than the default 64 KB of LDS per workgroup
static size_t expert_lds_bytes(int bm) { return (size_t)2 * (kBN + bm) * kLdsStride * sizeof(uint16_t); }


hipError_t launch_expert_linear(int32_t E, int64_t H, int64_t N, int64_t n_rows,
                                const int32_t* expert_offset, const void* x, const void* w, void* y,
                                uint32_t* status, hipStream_t stream) {
    ExpertArgs a;
    a.eoff = expert_offset;
    a.x = static_cast<const u32x4*>(x);
    a.w = static_cast<const u32x4*>(w);
    a.y = static_cast<uint2*>(y);
    a.status = status;
    a.H = H;
    a.N = N;
    a.n_rows = n_rows;
    a.E = E;
    // tall tiles: experts above 128 rows, at most n_rows / 129 of them, each
    // with one partial tile; short tiles: at most one per expert
    const int64_t tall_e = n_rows / (kBShort + 1) < E ? n_rows / (kBShort + 1) : E;
    const int64_t tiles = (n_rows + kBTall - 1) / kBTall + tall_e + E;
    const size_t lds = expert_lds_bytes(kBTall);
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(expert_linear_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    return launch_kernel(expert_linear_kernel, dim3((unsigned)((N + kBN - 1) / kBN), (unsigned)tiles),
                         dim3(kGemmThreads), lds, stream, a);
}

}  // namespace ubep

// Host-side launch entry points of the kernels (one per .hip file); the C ABI
// in api.hip validates arguments and calls these.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

#include "plan.h"

namespace ubep {

// Events set by ubep_time_next_launch on the calling host thread: the next
// kernel launch records them at its start and end, and clears them.
struct LaunchEvents {
    hipEvent_t start;
    hipEvent_t stop;
};
void set_launch_events(hipEvent_t start, hipEvent_t stop);
LaunchEvents take_launch_events();

// Every library kernel launches through here: the arguments are converted to
// the kernel's parameter types, and a pending event pair is recorded by the
// dispatch itself (hipExtLaunchKernel), with no marker packet in the stream.
// launch_kernel with explicit events (each may be null): a call of several
// launches hands its pending pair out across them.
template <typename... P, typename... A>
hipError_t launch_kernel_ev(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                            hipEvent_t start, hipEvent_t stop, A... args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<P...> vals{static_cast<P>(args)...};
    void* ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1];
    std::apply([&ptrs](auto&... v) {
        int i = 0;
        ((ptrs[i++] = static_cast<void*>(&v)), ...);
    }, vals);
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, stream,
                              start, stop, 0);
}

template <typename... P, typename... A>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                         A... args) {
    const LaunchEvents ev = take_launch_events();
    return launch_kernel_ev(kernel, grid, block, lds, stream, ev.start, ev.stop, args...);
}

// expert_offset: [E+1] output of the expert order (p.order == 1), may be null.
// status: the device status word (null: the one in the workspace header).
hipError_t launch_layout(const Plan& p, const int32_t* idx, int32_t* pos, int32_t* expert_count,
                         int32_t* expert_offset, int32_t* rank_count, int32_t* recv_offset,
                         int32_t* send_offset, int32_t* chunk_offset, int32_t* recv_src, void* ws,
                         uint64_t spin_ticks, hipStream_t stream, uint32_t* status = nullptr);

// Device address of the allocation-free layout's per-device scratch array
// (kScratchBytes), found once per device with that device current;
// *first_use is true on the call that found it.
hipError_t layout_scratch(int device, void** out, bool* first_use);

int64_t layout_workers(const Plan& p, int cus);
bool layout_lds_fits(const Plan& p);
void set_layout_worker_cap(int32_t n);   // 0: default

hipError_t launch_layout_dispatch(const Plan& p, const int32_t* idx, const void* x, int32_t* pos,
                                  int32_t* expert_count, int32_t* rank_count, int32_t* recv_offset,
                                  int32_t* send_offset, int32_t* chunk_offset, int32_t* recv_src,
                                  void* recv, void* ws, uint64_t spin_ticks, hipStream_t stream);
bool layout_fits_one_group(const Plan& p);

hipError_t launch_dispatch_bf16(const Plan& p, const void* x, const int32_t* pos, void* recv,
                                uint32_t* status, hipStream_t stream);

hipError_t launch_dispatch_fp8(const Plan& p, const void* x, const int32_t* pos, void* recv8,
                               float* recv_scale, uint32_t* status, hipStream_t stream);

hipError_t launch_combine(const Plan& p, const void* y, const int32_t* pos, const float* topk_w,
                          void* out, uint32_t* status, hipStream_t stream);

// chunk_order: host order (or null); dev_order: a device order (LPT policy) that
// takes its place when not null.
hipError_t launch_chunked(const Plan& p, const void* x, const int32_t* pos, const float* topk_w,
                          void* recv, void* out, const int32_t* chunk_order,
                          const int32_t* dev_order, uint64_t spin_ticks, uint32_t debug_flags,
                          void* ws, int device, hipStream_t stream);

hipError_t launch_chunk_lpt(const Plan& p, const int32_t* chunk_offset, const int32_t* rank_count,
                            int32_t* order, hipStream_t stream);

hipError_t launch_gate(const ubep_gate_shape& g, const float* logits, int32_t* idx, float* w,
                       hipStream_t stream);

// The gate that also counts its selections per layout tile (ubep_gate_layout).
struct GateCountArgs {
    int32_t* rank_cnt;       // [n_tiles][R], zero on entry
    int32_t* expert_cnt;     // [n_tiles][E], zero on entry
    int64_t tile_tokens;
    int32_t R;
    uint32_t epr_magic;
};
bool gate_counts_fit(const ubep_gate_shape& g, const float* logits, int64_t tile_tokens);
hipError_t launch_gate_counting(const ubep_gate_shape& g, const float* logits, int32_t* idx,
                                float* w, const GateCountArgs* counts, hipStream_t stream);

// The layout from per-tile counts that the counting gate left in the workspace.
hipError_t launch_layout_from_counts(const Plan& p, const int32_t* idx, int32_t* pos,
                                     int32_t* expert_count, int32_t* rank_count,
                                     int32_t* recv_offset, int32_t* send_offset,
                                     int32_t* chunk_offset, int32_t* recv_src, void* ws,
                                     hipStream_t stream);
bool layout_from_counts_fits(const Plan& p);

hipError_t launch_sentinel_pipeline(const Plan& p, const void* x, const int32_t* pos,
                                    const float* topk_w, void* recv, void* out, uint64_t spin_ticks,
                                    uint32_t debug_flags, void* ws, int device, hipStream_t stream);
hipError_t launch_sentinel_fill(void* recv, int64_t rows, int64_t H, hipStream_t stream);

hipError_t launch_expert_linear(int32_t E, int64_t H, int64_t N, int64_t n_rows,
                                const int32_t* expert_offset, const void* x, const void* w, void* y,
                                uint32_t* status, hipStream_t stream);

hipError_t launch_expert_pack(int32_t E, int64_t N, int64_t H, const void* w, void* packed,
                              hipStream_t stream);

hipError_t launch_identity_fp8(int64_t rows, int64_t H, const uint8_t* q, const float* scale,
                               void* y, hipStream_t stream);

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

hipError_t launch_stream_probe(const void* src, void* dst, int64_t n, int fan_in, int fan_out,
                               hipStream_t stream);

hipError_t launch_fill_zero(void* ws, size_t bytes, hipStream_t stream);

hipError_t launch_clear_status(uint32_t* status, hipStream_t stream);

// Workgroups of `kernel` (block threads, lds bytes of dynamic LDS) that fit on
// the current device at once: blocks per CU times CUs (cached per kernel).
hipError_t resident_blocks(const void* kernel, int block, size_t lds, int64_t* out);

// Grids of fewer than this many resident waves of workgroups hand out token
// blocks by workgroup index alone (no start-order tickets).
constexpr int64_t kTicketMinWaves = 8;

// Device properties used to size persistent grids and bounded waits.
struct DeviceInfo {
    int cus;
    int64_t wall_clock_khz;
};
hipError_t device_info(int device, DeviceInfo* out);

}  // namespace ubep

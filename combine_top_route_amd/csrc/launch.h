// Host-side launch entry points of the kernels (one per .hip file); the C ABI
// in api.hip validates arguments and calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace ubep {

hipError_t launch_layout(const Plan& p, const int32_t* idx, int32_t* pos, int32_t* expert_count,
                         int32_t* rank_count, int32_t* recv_offset, int32_t* send_offset,
                         int32_t* chunk_offset, int32_t* recv_src, void* ws, uint64_t spin_ticks,
                         hipStream_t stream);

int64_t layout_workers(const Plan& p, int cus);
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

hipError_t launch_chunked(const Plan& p, const void* x, const int32_t* pos, const float* topk_w,
                          void* recv, void* out, const int32_t* chunk_order, uint64_t spin_ticks,
                          uint32_t debug_flags, void* ws, int device, hipStream_t stream);

hipError_t launch_identity_fp8(int64_t rows, int64_t H, const uint8_t* q, const float* scale,
                               void* y, hipStream_t stream);

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

hipError_t launch_fill_zero(void* ws, size_t bytes, hipStream_t stream);

hipError_t launch_clear_status(uint32_t* status, hipStream_t stream);

// Device properties used to size persistent grids and bounded waits.
struct DeviceInfo {
    int cus;
    int64_t wall_clock_khz;
};
hipError_t device_info(int device, DeviceInfo* out);

}  // namespace ubep

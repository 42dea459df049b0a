// hstu_launch.h - host-side launchers of the HSTU forward kernels (hstu_fwd_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "hstu_params.h"

namespace hstu {

// Query rows per work-group and key-tile width per head dim (the kernels' tiling).
constexpr int kBlockM = 128;
constexpr int key_tile_for(int D) { return D == 64 ? 128 : (D == 128 ? 64 : 32); }

hipError_t launch_forward(const KernelParams &p, int dtype, int D, bool softmax, bool split,
                          hipStream_t stream);
hipError_t launch_combine(const KernelParams &p, int dtype, int D, bool softmax, hipStream_t stream);
hipError_t launch_count(const KernelParams &p, int D, unsigned long long *count, hipStream_t stream);

}  // namespace hstu

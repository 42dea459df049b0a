// hstu_launch.h - host-side launchers of the HSTU forward kernels (hstu_fwd_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "hstu_params.h"

namespace hstu {

// The kernels' tiling per head dim: key-tile width, waves per work-group (32
// query rows each) and so query rows per work-group.  hdim 256 runs one
// work-group per CU (its registers), so its 64-key stages (64 KB each) cost no
// occupancy, and the tile's fixed costs (barrier, wait) are halved against 32 keys.
constexpr int key_tile_for(int D) { return D <= 64 ? 128 : 64; }
// Four waves (128 rows): two work-groups then share a CU; eight-wave work-groups
// (one per CU) halve the key/value traffic into LDS per row but measured slower,
// since the CU-wide barrier keeps the two waves of each SIMD in the same phase.
constexpr int waves_for(int) { return 4; }
constexpr int block_m_for(int D) { return 32 * waves_for(D); }
// Work-groups of the forward kernel resident per CU (its occupancy bound: two
// waves per SIMD, one for hdim 256) and the CUs of an MI355X: a per-item grid of
// fewer work-groups than their product leaves CUs idle.
constexpr int groups_per_cu_for(int D) { return D >= 256 ? 1 : 2; }
constexpr int kChipCUs = 256;

hipError_t launch_forward(const KernelParams &p, int dtype, int D, int DV, bool softmax, bool split,
                          hipStream_t stream);
hipError_t launch_combine(const KernelParams &p, int dtype, int D, bool softmax, hipStream_t stream);
// combine pass of the cut (heavy) q-tiles of an unsplit call on the per-item grid
hipError_t launch_heavy_combine(const KernelParams &p, int dtype, int D, int DV, bool softmax, hipStream_t stream);
hipError_t launch_count(const KernelParams &p, int D, unsigned long long *count, hipStream_t stream);

// The allocation-free entry point's static scratch (HSTU_NOALLOC_SCRATCH_BYTES,
// 256-byte aligned): its device address on the current device, looked up on the
// first call per device.  Calls on one device share it.
constexpr size_t kScratchBytes = HSTU_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
hipError_t scratch_region(void **ptr);

}  // namespace hstu

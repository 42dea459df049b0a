// hstu_layer_launch.h - kernel parameters and launchers of the HSTU layer kernels
// (hstu_layer_kernels.hip), filled by hstu_layer_api.cpp after validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hstu.h"

namespace hstu {
namespace layer {

// y[m, n] = act(sum_k x[m, k] w[n, k] + bias[n]) (+ res[m, n]); strides in elements
struct LinearParams {
    const uint16_t *x;
    int64_t x_stride;
    const uint16_t *w;  // [N][K] contiguous
    const float *bias;  // [N] or nullptr (16-byte aligned)
    const uint16_t *res;
    int64_t r_stride;
    uint16_t *y;
    int64_t y_stride;
    int64_t M;
    int32_t N, K;  // K % 64 == 0, N % 8 == 0
    int32_t act;   // 0 identity, 1 SiLU
    int64_t m_tiles;
    int32_t n_tiles;
};

// z[m, :] = (LayerNorm(a[m, :]) * gamma + beta) * u[m, :], W features per row
struct NormGateParams {
    const uint16_t *a;
    int64_t a_stride;
    const uint16_t *u;
    int64_t u_stride;
    const float *gamma, *beta;  // [W] or nullptr
    float eps;
    uint16_t *z;  // may equal a
    int64_t z_stride;
    int64_t M;
    int32_t W;  // % 8 == 0, <= 4096
};

hipError_t launch_linear(const LinearParams &p, int dtype, hipStream_t stream);
hipError_t launch_norm_gate(const NormGateParams &p, int dtype, hipStream_t stream);

}  // namespace layer
}  // namespace hstu

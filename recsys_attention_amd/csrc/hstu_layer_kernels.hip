// hstu_layer_kernels.hip - gfx950 kernels of the HSTU layer around the attention
// (HSTU explainer, "The layer, line by line"): the two pointwise linear maps
// with their fused epilogues, and the normalisation gated by U.
//
//   linear:    y[m, n] = act(sum_k x[m, k] w[n, k] + bias[n]) (+ res[m, n])
//              act = SiLU for f1 (sub-layer (a)), identity + residual for f2 (c)
//   norm_gate: z[m, :] = LayerNorm(a[m, :]) * gamma + beta, times u[m, :]
//
// linear: a work-group of 4 waves owns a BM x BN tile of y (128 x 128, two
// work-groups per CU); wave (wm, wn) owns a quarter as (BM/64) x (BN/64)
// blocks of v_mfma_f32_32x32x16.  The MFMA computes the
// transposed block y^T = W . x^T (A = 32 rows of w, B = 32 rows of x, both read
// along k), so the accumulator gives each lane one row m of y and four
// consecutive columns per register group: the epilogue stores 8 bytes per lane
// and group.  x and w tiles (64 k wide) move global -> LDS directly
// (buffer_load_dwordx4 ... lds) into a two-stage ring; the 16-byte k-chunks of
// each 128-byte row are XOR-swizzled by (row & 7) so the operand reads of eight
// consecutive rows touch all 32 banks.  The epilogue goes through LDS so that
// every store instruction writes whole 128-byte row segments.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "hstu_layer_launch.h"

namespace hstu {
namespace layer {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr float kLog2e = 1.4426950408889634f;

template <int DT>
struct Elem;
template <>
struct Elem<HSTU_BF16> {
    static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ u32x2_t pack4(f32x4_t v) {
        bf16x4_t h = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
        return __builtin_bit_cast(u32x2_t, h);
    }
    static __device__ __forceinline__ f32x4_t unpack4(u32x2_t b) {
        const bf16x4_t h = __builtin_bit_cast(bf16x4_t, b);
        return f32x4_t{(float)h.x, (float)h.y, (float)h.z, (float)h.w};
    }
};
template <>
struct Elem<HSTU_FP16> {
    static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ u32x2_t pack4(f32x4_t v) {
        f16x4_t h = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
        return __builtin_bit_cast(u32x2_t, h);
    }
    static __device__ __forceinline__ f32x4_t unpack4(u32x2_t b) {
        const f16x4_t h = __builtin_bit_cast(f16x4_t, b);
        return f32x4_t{(float)h.x, (float)h.y, (float)h.z, (float)h.w};
    }
};

__device__ __forceinline__ i32x4_t make_rsrc_words(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    return i32x4_t{__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a),
                   __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(a >> 32) & 0xffffu)),
                   __builtin_amdgcn_readfirstlane((int32_t)bytes), 0x00020000};
}

// 16 bytes per lane from global memory straight into LDS (lane i lands at
// lds_wave + 16 i); rows past the descriptor's range read as zeros.  M0 is not
// otherwise used by these kernels (gfx9+ LDS instructions do not read it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_to_lds(const i32x4_t &rsrc, uint32_t lds_wave, uint32_t off) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(lds_wave), "v"(off), "s"(rsrc)
        : "m0");
}
// vmcnt(0) at this point of the instruction stream (the compiler does not see the
// loads above, so a builtin wait could be merged into an earlier one)
__device__ __forceinline__ void wait_all_loads_here() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
#pragma clang diagnostic pop

constexpr int kBK = 64, kNT = 256;

// Tile of one work-group: BM rows x BN columns of y; the four waves split it 2 x 2,
// each wave (BM/2) x (BN/2) as (BM/64) x (BN/64) blocks of 32 x 32.  One k-tile
// stage holds the x tile (BM rows) and the w tile (BN rows), 128 bytes a row.
template <int BM, int BN>
struct LinTile {
    static constexpr int MB = BM / 64, NB = BN / 64;         // 32-row blocks per wave
    static constexpr int XBYTES = BM * kBK * 2, WBYTES = BN * kBK * 2;
    static constexpr int STAGE = XBYTES + WBYTES;
    static constexpr int XLOADS = BM / 32, WLOADS = BN / 32;  // wave-loads per tile and thread
};

template <int DT, int BM, int BN, bool SILU, bool RES>
__global__ __launch_bounds__(kNT, BM == 256 ? 1 : 2) void linear_kernel(LinearParams p) {
    using E = Elem<DT>;
    using T = LinTile<BM, BN>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][T::STAGE];  // [stage][x tile | w tile]

    // tile of this work-group: consecutive ids go to consecutive XCDs; on one XCD
    // the column tiles of a row tile follow each other, so its x rows are fetched
    // from HBM once into that XCD's L2 (w is small enough to stay in every L2)
    const int64_t bid = blockIdx.x;
    const int64_t xcd = bid % 8, loc = bid / 8;
    const int64_t mt = (loc / p.n_tiles) * 8 + xcd;
    const int nt = (int)(loc % p.n_tiles);
    if (mt >= p.m_tiles) return;
    const int64_t m0 = mt * BM;
    const int n0 = nt * BN;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave & 1, wn = wave >> 1;

    const uint32_t xs2 = (uint32_t)p.x_stride * 2, ks2 = (uint32_t)p.K * 2;
    const int64_t mrows = p.M - m0 < BM ? p.M - m0 : BM;
    const int nrows = p.N - n0 < BN ? p.N - n0 : BN;
    const i32x4_t xr = make_rsrc_words(p.x + m0 * p.x_stride, (uint32_t)mrows * xs2);
    const i32x4_t wr = make_rsrc_words(p.w + (int64_t)n0 * p.K, (uint32_t)nrows * ks2);

    // DMA: wave-load c of wave w fills physical chunks c*256 + tid of a tile:
    // row 32c + tid/8, position tid%8, which holds logical k-chunk (tid%8) ^ (row & 7)
    const int row_in = tid >> 3, pc = tid & 7;
    const uint32_t chunk = (uint32_t)((pc ^ (row_in & 7)) * 16);
    const uint32_t x_lane = (uint32_t)row_in * xs2 + chunk, w_lane = (uint32_t)row_in * ks2 + chunk;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t *)&lds[0][0] + (uint32_t)wave_u * 1024;
    auto issue = [&](int kt, int st) {
        const uint32_t kb = (uint32_t)kt * (kBK * 2);
        const uint32_t dst = lds0 + (uint32_t)(st * T::STAGE);
#pragma unroll
        for (int c = 0; c < T::XLOADS; ++c)
            load_to_lds(xr, dst + c * 4096, x_lane + (uint32_t)(32 * c) * xs2 + kb);
#pragma unroll
        for (int c = 0; c < T::WLOADS; ++c)
            load_to_lds(wr, dst + T::XBYTES + c * 4096, w_lane + (uint32_t)(32 * c) * ks2 + kb);
    };

    // operand reads: row (block base) + r32, logical chunk 2kk + g, swizzled by r32 & 7
    uint32_t off[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) off[kk] = (uint32_t)(r32 * 128 + (((2 * kk + g) ^ (r32 & 7)) * 16));

    f32x16_t acc[T::NB][T::MB];
#pragma unroll
    for (int a = 0; a < T::NB; ++a)
#pragma unroll
        for (int b = 0; b < T::MB; ++b) acc[a][b] = f32x16_t{};

    const int KT = p.K / kBK;
    issue(0, 0);
    wait_all_loads_here();
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < KT) issue(kt + 1, st ^ 1);
        const uint8_t *xs = &lds[st][0] + wm * (BM / 2) * 128;
        const uint8_t *ws = &lds[st][0] + T::XBYTES + wn * (BN / 2) * 128;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4_t xo[T::MB], wo[T::NB];
#pragma unroll
            for (int b = 0; b < T::MB; ++b) xo[b] = *(const u32x4_t *)(xs + b * 32 * 128 + off[kk]);
#pragma unroll
            for (int b = 0; b < T::NB; ++b) wo[b] = *(const u32x4_t *)(ws + b * 32 * 128 + off[kk]);
#pragma unroll
            for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
                for (int mb = 0; mb < T::MB; ++mb) acc[nb][mb] = E::mfma(wo[nb], xo[mb], acc[nb][mb]);
        }
        wait_all_loads_here();
        __syncthreads();
    }

    // epilogue, in two phases through LDS (the ring is free after the last barrier):
    // 1. block (nb, mb), register group i4 is row (BM/2) wm + 32mb + r32, columns
    //    (BN/2) wn + 32nb + 8 i4 + 4g .. +3 of the tile: bias, activation and residual
    //    in fp32, rounded to the dtype, written to the wave's own LDS region (rows of
    //    the wave's BN/2 columns, padded by 8 bytes against bank conflicts);
    // 2. read back 16 bytes per lane along rows (eight lanes cover 128 bytes of one
    //    row), so every store instruction writes whole row segments.
    constexpr int WR = BM / 2, WC = BN / 2;        // wave tile
    constexpr int RSTRIDE = WC * 2 + 8;            // bytes per LDS row
    static_assert(4 * WR * RSTRIDE <= 2 * T::STAGE, "the staged tile fits in the ring");
    uint8_t *stage_out = &lds[0][0] + wave * (WR * RSTRIDE);
#pragma unroll
    for (int mb = 0; mb < T::MB; ++mb) {
        const int64_t m = m0 + wm * WR + mb * 32 + r32;
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int c = nb * 32 + 8 * i4 + 4 * g;  // column inside the wave tile
                const int n = n0 + wn * WC + c;
                f32x4_t v = {acc[nb][mb][4 * i4], acc[nb][mb][4 * i4 + 1], acc[nb][mb][4 * i4 + 2],
                             acc[nb][mb][4 * i4 + 3]};
                if (p.bias != nullptr && n < p.N) v += *(const f32x4_t *)(p.bias + n);
                if constexpr (SILU) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = v[e] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * v[e]));
                }
                if constexpr (RES) {
                    if (m < p.M && n < p.N) v += E::unpack4(*(const u32x2_t *)(p.res + m * p.r_stride + n));
                }
                *(u32x2_t *)(stage_out + (mb * 32 + r32) * RSTRIDE + c * 2) = E::pack4(v);
            }
        }
    }
    __syncthreads();
    constexpr int CH = WC / 8;                     // 16-byte chunks per wave-tile row
    constexpr int RPI = 64 / CH;                   // rows per store instruction
#pragma unroll
    for (int pass = 0; pass < WR / RPI; ++pass) {
        const int r = pass * RPI + lane / CH, ch = lane % CH;
        const uint8_t *src = stage_out + r * RSTRIDE + ch * 16;
        const u32x2_t lo = *(const u32x2_t *)src, hi = *(const u32x2_t *)(src + 8);
        const int64_t m = m0 + wm * WR + r;
        const int n = n0 + wn * WC + ch * 8;
        if (m < p.M && n < p.N) *(u32x4_t *)(p.y + m * p.y_stride + n) = u32x4_t{lo.x, lo.y, hi.x, hi.y};
    }
}

// ---------------------------------------------------------------- norm * gate

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// One wave per row: the row's W features (W = 8 * 64 * c for c chunks per lane
// at most kMaxChunks) are held in registers, mean and variance in two passes.
constexpr int kMaxChunks = 8;  // W <= 4096

template <int DT>
__global__ __launch_bounds__(256) void norm_gate_kernel(NormGateParams p) {
    using E = Elem<DT>;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.M) return;
    const int nch = p.W / 8;  // 8-element chunks of the row
    const uint16_t *a = p.a + row * p.a_stride;
    const uint16_t *u = p.u + row * p.u_stride;
    f32x4_t v[kMaxChunks][2];
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < kMaxChunks; ++t) {
        const int c = lane + 64 * t;
        if (c < nch) {
            const u32x4_t b = *(const u32x4_t *)(a + 8 * c);
            v[t][0] = E::unpack4(u32x2_t{b.x, b.y});
            v[t][1] = E::unpack4(u32x2_t{b.z, b.w});
            s += (v[t][0].x + v[t][0].y + v[t][0].z + v[t][0].w) + (v[t][1].x + v[t][1].y + v[t][1].z + v[t][1].w);
        }
    }
    const float mean = wave_sum(s) / (float)p.W;
    float q = 0.0f;
#pragma unroll
    for (int t = 0; t < kMaxChunks; ++t) {
        const int c = lane + 64 * t;
        if (c < nch) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                v[t][h] -= mean;
                q += v[t][h].x * v[t][h].x + v[t][h].y * v[t][h].y + v[t][h].z * v[t][h].z + v[t][h].w * v[t][h].w;
            }
        }
    }
    const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)p.W + p.eps);
    uint16_t *z = p.z + row * p.z_stride;
#pragma unroll
    for (int t = 0; t < kMaxChunks; ++t) {
        const int c = lane + 64 * t;
        if (c < nch) {
            const u32x4_t ub = *(const u32x4_t *)(u + 8 * c);
            u32x2_t o[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4_t y = v[t][h] * rstd;
                const int f = 8 * c + 4 * h;
                if (p.gamma != nullptr) y *= *(const f32x4_t *)(p.gamma + f);
                if (p.beta != nullptr) y += *(const f32x4_t *)(p.beta + f);
                y *= E::unpack4(h ? u32x2_t{ub.z, ub.w} : u32x2_t{ub.x, ub.y});
                o[h] = E::pack4(y);
            }
            *(u32x4_t *)(z + 8 * c) = u32x4_t{o[0].x, o[0].y, o[1].x, o[1].y};
        }
    }
}

// ------------------------------------------------------------------ launchers

template <int DT, int BM, int BN>
static hipError_t launch_linear_tile(LinearParams p, hipStream_t stream) {
    p.m_tiles = (p.M + BM - 1) / BM;
    p.n_tiles = (p.N + BN - 1) / BN;
    const int64_t grid = (int64_t)((p.m_tiles + 7) / 8) * 8 * p.n_tiles;
    if (grid <= 0) return hipSuccess;
    const dim3 g((unsigned)grid), b(kNT);
    if (p.act == 1) {
        if (p.res != nullptr) hipLaunchKernelGGL((linear_kernel<DT, BM, BN, true, true>), g, b, 0, stream, p);
        else hipLaunchKernelGGL((linear_kernel<DT, BM, BN, true, false>), g, b, 0, stream, p);
    } else {
        if (p.res != nullptr) hipLaunchKernelGGL((linear_kernel<DT, BM, BN, false, true>), g, b, 0, stream, p);
        else hipLaunchKernelGGL((linear_kernel<DT, BM, BN, false, false>), g, b, 0, stream, p);
    }
    return hipGetLastError();
}

// 128 x 128 tiles, two work-groups per CU (256 x 256 tiles, one work-group per CU
// with 256 accumulators per lane, measured slower: nothing overlaps a work-group's
// first load and its epilogue)
template <int DT>
static hipError_t launch_linear_dt(const LinearParams &p, hipStream_t stream) {
    return launch_linear_tile<DT, 128, 128>(p, stream);
}

hipError_t launch_linear(const LinearParams &p, int dtype, hipStream_t stream) {
    return dtype == HSTU_BF16 ? launch_linear_dt<HSTU_BF16>(p, stream) : launch_linear_dt<HSTU_FP16>(p, stream);
}

hipError_t launch_norm_gate(const NormGateParams &p, int dtype, hipStream_t stream) {
    if (p.M <= 0) return hipSuccess;
    const dim3 g((unsigned)((p.M + 3) / 4)), b(256);
    if (dtype == HSTU_BF16) hipLaunchKernelGGL((norm_gate_kernel<HSTU_BF16>), g, b, 0, stream, p);
    else hipLaunchKernelGGL((norm_gate_kernel<HSTU_FP16>), g, b, 0, stream, p);
    return hipGetLastError();
}

}  // namespace layer
}  // namespace hstu

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
// each 128-byte row are XOR-swizzled by (row >> 1) & 7 so the operand reads of
// sixteen consecutive rows (one 16-lane group) touch all 64 banks.  The epilogue goes through LDS so that
// every store instruction writes whole 128-byte row segments.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

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
    // row 32c + tid/8, position tid%8, which holds logical k-chunk
    // (tid%8) ^ ((row >> 1) & 7): the 16 rows of a 16-lane read group then cover
    // all 64 banks (two rows per 256 bytes, eight distinct chunk positions)
    const int row_in = tid >> 3, pc = tid & 7;
    const uint32_t chunk = (uint32_t)((pc ^ ((row_in >> 1) & 7)) * 16);
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

    // operand reads: row (block base) + r32, logical chunk 2kk + g, swizzled by (r32 >> 1) & 7
    uint32_t off[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) off[kk] = (uint32_t)(r32 * 128 + (((2 * kk + g) ^ ((r32 >> 1) & 7)) * 16));

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
        // non-temporal: y is not read again by this kernel, and allocating it in L2
        // evicts the x rows the other column tiles of the XCD still need
        if (m < p.M && n < p.N)
            __builtin_nontemporal_store(u32x4_t{lo.x, lo.y, hi.x, hi.y}, (u32x4_t *)(p.y + m * p.y_stride + n));
    }
}

// ------------------------------------------------ persistent 256 x 256 linear
//
// For shapes with many output tiles (f1 of a layer): one work-group of 8 waves
// per CU walks its share of 256 x 256 tiles.  Wave (wm, wn) of the 2 x 4 wave
// grid owns 128 rows x 64 columns (4 x 2 MFMA blocks, 128 accumulators).  k-tiles
// are 32 wide (64-byte rows, chunks XOR-swizzled by (row >> 2) & 3) and run
// through a 4-stage LDS ring that continues across the work-group's tiles: the
// loads of step s + 3 are issued at step s, so three steps (96 KB per CU) are in
// flight and a tile's first loads overlap the previous tile's last steps and
// epilogue.  Twice the output per loaded byte of the 128 x 128 tiles.  The tile
// bookkeeping is incremental (no divisions per step).
constexpr int kPBM = 256, kPBN = 256, kPBK = 32, kPNT = 512, kPStages = 4;
constexpr int kPStage = (kPBM + kPBN) * kPBK * 2;  // 32 KB: x tile | w tile
constexpr int kPStageOut = 32 * 128;              // per-wave epilogue staging (32 rows x 64 cols)
constexpr int kPBiasSlots = 4;                    // bias of four consecutive tiles (1 KB each)
static_assert(8 * kPStageOut == kPStage, "the epilogue stages through one ring stage");

// LDS writes of a wave made visible to the wave's other lanes (one wave's LDS
// instructions execute in order; this keeps the compiler from reordering them)
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int DT, bool SILU, bool RES>
__global__ __launch_bounds__(kPNT) __attribute__((amdgpu_waves_per_eu(2, 2))) void linear_persistent_kernel(
    LinearParams p) {
    using E = Elem<DT>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kPStages * kPStage + kPBiasSlots * 1024];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave & 1, wn = wave >> 1;  // 2 x 4 waves: 128 rows x 64 columns each

    // this work-group's tiles: T = blockIdx.x + i * gridDim.x (gridDim a multiple of
    // 8, so every T of a work-group maps to its own XCD); the valid ones form a prefix
    const int32_t G = gridDim.x, b0 = blockIdx.x;
    const int32_t total = ((p.m_tiles + 7) / 8) * 8 * p.n_tiles;
    auto tile_of = [&](int32_t i, int64_t &m0, int32_t &n0) {  // i-th tile of this work-group
        const int32_t T = b0 + i * G, loc = T >> 3;
        m0 = (int64_t)((loc / p.n_tiles) * 8 + (T & 7)) * kPBM;
        n0 = (loc % p.n_tiles) * kPBN;
    };
    int32_t ntiles = 0;
    for (int32_t T = b0; T < total && ((T >> 3) / p.n_tiles) * 8 + (T & 7) < p.m_tiles; T += G) ++ntiles;
    if (ntiles == 0) return;
    const int32_t KT = p.K / kPBK;
    const int32_t steps = ntiles * KT;

    const uint32_t xs2 = (uint32_t)p.x_stride * 2, ks2 = (uint32_t)p.K * 2;
    // DMA: wave w loads x rows [32w, 32w + 32) and w rows [32w, 32w + 32) of a stage,
    // two wave-loads of 16 rows each; lane -> row lane/4, position lane%4, which holds
    // logical chunk (lane%4) ^ ((row >> 2) & 3): the 16 rows of a 16-lane read group
    // then cover all 64 banks (four rows per 256 bytes, four distinct positions)
    const int lrow = lane >> 2;
    const uint32_t lchunk = (uint32_t)(((lane & 3) ^ ((lrow >> 2) & 3)) * 16);
    const uint32_t ldsb = (uint32_t)(uintptr_t)(lds_void_t *)&lds[0];
    // the step being loaded: tile iss_i, k-tile iss_kt, with that tile's descriptors
    int32_t iss_i = 0, iss_kt = 0;
    i32x4_t xr, wr, br;
    auto set_tile = [&]() {
        int64_t m0;
        int32_t n0;
        tile_of(iss_i, m0, n0);
        const int64_t mrows = p.M - m0 < kPBM ? p.M - m0 : kPBM;
        const int32_t nrows = p.N - n0 < kPBN ? p.N - n0 : kPBN;
        xr = make_rsrc_words(p.x + m0 * p.x_stride, (uint32_t)mrows * xs2);
        wr = make_rsrc_words(p.w + (int64_t)n0 * p.K, (uint32_t)nrows * ks2);
        br = make_rsrc_words((const void *)((uintptr_t)p.bias + 4u * (uint32_t)n0), (uint32_t)nrows * 4u);
    };
    set_tile();
    auto issue = [&](int32_t s) {  // the loads of step s (= iss_i * KT + iss_kt) into stage s % 4
        const uint32_t dst = ldsb + (uint32_t)((s & (kPStages - 1)) * kPStage) + (uint32_t)wave_u * 2048;
        const uint32_t kb = (uint32_t)iss_kt * (kPBK * 2);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t row = (uint32_t)(32 * wave_u + 16 * h + lrow);
            load_to_lds(xr, dst + h * 1024, row * xs2 + lchunk + kb);
            load_to_lds(wr, dst + kPBM * kPBK * 2 + h * 1024, row * ks2 + lchunk + kb);
        }
        // the tile's 256 bias values, with its first k-tile, into bias slot i % 4 (the
        // slot's previous tile finished its epilogue before this tile's loads began,
        // three steps ahead of it, since a tile has at least one step)
        if (iss_kt == 0 && wave_u == 0 && p.bias != nullptr)
            load_to_lds(br, ldsb + kPStages * kPStage + (uint32_t)(iss_i & (kPBiasSlots - 1)) * 1024,
                        (uint32_t)lane * 16u);
        if (++iss_kt == KT) {
            iss_kt = 0;
            if (++iss_i < ntiles) set_tile();
        }
    };
    // wait until the loads of step s + 1 have landed (those of s + 2, s + 3 may be in flight)
    auto wait_next = [&](int32_t s) {
        __builtin_amdgcn_sched_barrier(0);
        const int after = (s + 2 < steps) + (s + 3 < steps);
        if (after == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else if (after == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    // operand reads: row (block base) + r32, logical chunk 2kk + g, swizzled by (r32 >> 2) & 3
    uint32_t off[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) off[kk] = (uint32_t)(r32 * 64 + (((2 * kk + g) ^ ((r32 >> 2) & 3)) * 16));

    f32x16_t acc[2][4];
    for (int32_t s = 0; s < 3 && s < steps; ++s) issue(s);
    wait_next(-1);
    __syncthreads();
    int32_t kt = 0, cur_i = 0;  // the step computed: tile cur_i, k-tile kt
    for (int32_t s = 0; s < steps; ++s) {
        if (kt == 0) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = f32x16_t{};
        }
        if (s + 3 < steps) issue(s + 3);
        const uint8_t *st = &lds[(s & (kPStages - 1)) * kPStage];
        const uint8_t *xs = st + wm * 128 * 64;
        const uint8_t *ws = st + kPBM * kPBK * 2 + wn * 64 * 64;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            u32x4_t xo[4], wo[2];
#pragma unroll
            for (int b = 0; b < 4; ++b) xo[b] = *(const u32x4_t *)(xs + b * 32 * 64 + off[kk]);
#pragma unroll
            for (int b = 0; b < 2; ++b) wo[b] = *(const u32x4_t *)(ws + b * 32 * 64 + off[kk]);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = E::mfma(wo[nb], xo[mb], acc[nb][mb]);
        }
        wait_next(s);
        __syncthreads();
        if (++kt != KT) continue;
        kt = 0;

        // epilogue of this tile, 32 rows (one m-block) at a time through the wave's
        // 4 KB of the stage just consumed (refilled only after the barrier below):
        // rows of 128 bytes, 16-byte chunks XOR-swizzled by row & 7.  The bias comes
        // from LDS, so the epilogue issues no global load that would wait behind the
        // in-flight tile loads and its own stores.
        const float *bias = (const float *)&lds[kPStages * kPStage + (cur_i & (kPBiasSlots - 1)) * 1024] + wn * 64;
        int64_t m0;
        int32_t n0;
        tile_of(cur_i++, m0, n0);
        m0 += wm * 128;
        n0 += wn * 64;
        uint8_t *so = &lds[(s & (kPStages - 1)) * kPStage + wave * kPStageOut];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int64_t m = m0 + mb * 32 + r32;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int c = nb * 32 + 8 * i4 + 4 * g;  // column inside the wave's 64
                    const int n = n0 + c;
                    f32x4_t v = {acc[nb][mb][4 * i4], acc[nb][mb][4 * i4 + 1], acc[nb][mb][4 * i4 + 2],
                                 acc[nb][mb][4 * i4 + 3]};
                    if (p.bias != nullptr) v += *(const f32x4_t *)(bias + c);
                    if constexpr (SILU) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[e] = v[e] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * v[e]));
                    }
                    if constexpr (RES) {
                        if (m < p.M && n < p.N) v += E::unpack4(*(const u32x2_t *)(p.res + m * p.r_stride + n));
                    }
                    const int chunk = (c >> 3) ^ (r32 & 7);
                    *(u32x2_t *)(so + r32 * 128 + chunk * 16 + (c & 7) * 2) = E::pack4(v);
                }
            }
            wave_lds_sync();
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int r = it * 8 + (lane >> 3), ch = lane & 7;
                const u32x4_t val = *(const u32x4_t *)(so + r * 128 + ((ch ^ (r & 7)) * 16));
                const int64_t mm = m0 + mb * 32 + r;
                const int n = n0 + ch * 8;
                // non-temporal (as in linear_kernel): measured HBM reads of f1 on the
                // layer workload 270 MB -> 104 MB (x and w are 87 MB)
                if (mm < p.M && n < p.N) __builtin_nontemporal_store(val, (u32x4_t *)(p.y + mm * p.y_stride + n));
            }
            wave_lds_sync();
        }
        __syncthreads();  // the stage is refilled from the next step on
    }
}

// ---------------------------------------------------------------- norm * gate

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// One wave per row: the row's W features (up to CH 16-byte chunks per lane, W <=
// 512 CH) are held in registers with the gate row, mean and variance in two passes.
template <int DT, int CH>
__global__ __launch_bounds__(256) void norm_gate_kernel(NormGateParams p) {
    constexpr int kMaxChunks = CH;
    using E = Elem<DT>;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.M) return;
    const int nch = p.W / 8;  // 8-element chunks of the row
    const uint16_t *a = p.a + row * p.a_stride;
    const uint16_t *u = p.u + row * p.u_stride;
    f32x4_t v[kMaxChunks][2];
    u32x4_t ub[kMaxChunks];  // the gate, loaded together with the row (one memory latency per row)
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < kMaxChunks; ++t) {
        const int c = lane + 64 * t;
        if (c < nch) {
            const u32x4_t b = *(const u32x4_t *)(a + 8 * c);
            ub[t] = *(const u32x4_t *)(u + 8 * c);
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
            u32x2_t o[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4_t y = v[t][h] * rstd;
                const int f = 8 * c + 4 * h;
                if (p.gamma != nullptr) y *= *(const f32x4_t *)(p.gamma + f);
                if (p.beta != nullptr) y += *(const f32x4_t *)(p.beta + f);
                y *= E::unpack4(h ? u32x2_t{ub[t].z, ub[t].w} : u32x2_t{ub[t].x, ub[t].y});
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

template <int DT>
static hipError_t launch_linear_persistent(LinearParams p, int cus, hipStream_t stream) {
    p.m_tiles = (p.M + kPBM - 1) / kPBM;
    p.n_tiles = (p.N + kPBN - 1) / kPBN;
    const dim3 g((unsigned)((cus / 8) * 8)), b(kPNT);
    if (p.act == 1) {
        if (p.res != nullptr) hipLaunchKernelGGL((linear_persistent_kernel<DT, true, true>), g, b, 0, stream, p);
        else hipLaunchKernelGGL((linear_persistent_kernel<DT, true, false>), g, b, 0, stream, p);
    } else {
        if (p.res != nullptr) hipLaunchKernelGGL((linear_persistent_kernel<DT, false, true>), g, b, 0, stream, p);
        else hipLaunchKernelGGL((linear_persistent_kernel<DT, false, false>), g, b, 0, stream, p);
    }
    return hipGetLastError();
}

// compute units of the current device (cached per device; safe to call from
// several host threads, which at worst query the attribute more than once)
static int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Persistent 256 x 256 tiles when there are at least two per CU (and K is a
// multiple of their 32-wide k-tiles), else 128 x 128 tiles, two work-groups per CU.
// (The layer's f2, 83302 x 512 x 512 with the residual: 82 us persistent against
// 91 us with 128 x 128 tiles; 64 x 256 tiles: 96 us.)
template <int DT>
static hipError_t launch_linear_dt(const LinearParams &p, hipStream_t stream) {
    const int cus = device_cus();
    const int64_t big = ((p.M + kPBM - 1) / kPBM) * ((p.N + kPBN - 1) / kPBN);
    if (cus >= 8 && big >= 2 * (int64_t)cus && p.K % kPBK == 0) return launch_linear_persistent<DT>(p, cus, stream);
    return launch_linear_tile<DT, 128, 128>(p, stream);
}

hipError_t launch_linear(const LinearParams &p, int dtype, hipStream_t stream) {
    return dtype == HSTU_BF16 ? launch_linear_dt<HSTU_BF16>(p, stream) : launch_linear_dt<HSTU_FP16>(p, stream);
}

template <int DT>
static void launch_norm_gate_dt(const NormGateParams &p, dim3 g, dim3 b, hipStream_t stream) {
    // registers sized to the row: chunks of 8 features per lane, 64 lanes
    if (p.W <= 512) hipLaunchKernelGGL((norm_gate_kernel<DT, 1>), g, b, 0, stream, p);
    else if (p.W <= 1024) hipLaunchKernelGGL((norm_gate_kernel<DT, 2>), g, b, 0, stream, p);
    else if (p.W <= 2048) hipLaunchKernelGGL((norm_gate_kernel<DT, 4>), g, b, 0, stream, p);
    else hipLaunchKernelGGL((norm_gate_kernel<DT, 8>), g, b, 0, stream, p);
}

hipError_t launch_norm_gate(const NormGateParams &p, int dtype, hipStream_t stream) {
    if (p.M <= 0) return hipSuccess;
    const dim3 g((unsigned)((p.M + 3) / 4)), b(256);
    if (dtype == HSTU_BF16) launch_norm_gate_dt<HSTU_BF16>(p, g, b, stream);
    else launch_norm_gate_dt<HSTU_FP16>(p, g, b, stream);
    return hipGetLastError();
}

}  // namespace layer
}  // namespace hstu

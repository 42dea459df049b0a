// hstu_fwd_kernels.hip - gfx950 kernels of the HSTU attention forward.
//
// Operator: CK example README "18_hstu_attention", "Forward computation"
// (s = alpha * q.k, functional mask, SiLU * attn_scale or attn_scale * softmax,
// o = p @ v) and "Split-KV" (key axis cut across work-groups + combine pass).
//
// Work-group = 4 waves (waves_for); it owns 32 query rows per wave of one
// (sequence, head), 32 rows per wave.  Within a wave, lane l owns query row
// l % 32 and half of each key block (lane group g = l / 32):
//   S^T = K . Q^T   v_mfma_f32_32x32x16_{bf16,f16}: A = K tile from LDS
//                   (row = key, 8 consecutive d per lane), B = Q^T kept in
//                   VGPRs for the whole work-group lifetime.
//   The accumulator gives lane l the scores of its own query against 16 keys
//   of each 32-key block, so the mask is a per-lane interval test against the
//   row's visible key set [0, ctx) U [lo, hi].
//   O^T += V^T . P^T   A = V^T read from the row-major V tile with the gfx950
//                   LDS transpose read (ds_read_b64_tr_b16), B = P^T straight
//                   from the score registers: the key order inside each
//                   16-key MFMA step is permuted identically on both operands,
//                   so no cross-lane shuffle is needed.
// K and V tiles go global -> LDS directly (buffer_load_dwordx4 ... lds, no
// staging registers) into a two-stage ring; the next tile's loads are issued
// before the current tile's MFMAs, one barrier per tile.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "hstu_launch.h"
#include "hstu_plan.h"

namespace hstu {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
// an object in global memory (address space 1): accesses through it are global
// loads and stores
template <class T> using gmem_t = __attribute__((address_space(1))) T;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int DT>
struct Elem;

template <>
struct Elem<HSTU_BF16> {
    static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float x, float y) {
        bf16x2_t v = {(__bf16)x, (__bf16)y};
        return __builtin_bit_cast(uint32_t, v);
    }
};

template <>
struct Elem<HSTU_FP16> {
    static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float x, float y) {
        f16x2_t v = {(_Float16)x, (_Float16)y};
        return __builtin_bit_cast(uint32_t, v);
    }
};

// Tile geometry for head dim D (= hdim_qk = hdim_v) and key-tile width BN.
// K and V tiles sit in LDS row-major (BN rows of D elements, no padding); the
// 16-byte chunks of each row are XOR-swizzled against LDS bank conflicts of the
// MFMA operand reads (tables chosen by timing the exact read patterns on the
// device): K chunk c of row r is stored at chunk c ^ (r & 15) (the 32 lanes of
// a half-wave read one chunk of 32 consecutive rows), V chunk c at c ^ 4(r & 3)
// (the transposed reads touch four consecutive rows, 64 bytes each).
template <int D, int BN, int NW = 4, int DV = D>
struct Tile {
    static constexpr int BM = 32 * NW;       // query rows per work-group (32 per wave)
    static constexpr int NT = 64 * NW;       // threads
    static constexpr int RB = D * 2;         // bytes per K row (hdim_qk = D)
    static constexpr int CPR = D / 8;        // 16-byte chunks per K row
    static constexpr int TILE_BYTES = BN * RB;   // K tile
    static constexpr int RBV = DV * 2;       // bytes per V row (hdim_v = DV)
    static constexpr int CPRV = DV / 8;
    static constexpr int TILE_V = BN * RBV;
    static constexpr int STAGE = TILE_BYTES + TILE_V;  // one ring stage: [K tile | V tile]
    static constexpr int KSTEPS = D / 16;    // MFMA k-steps of Q.K^T
    static constexpr int NKB = BN / 32;      // 32-key blocks per tile
    static constexpr int NDB = DV / 32;      // 32-column blocks of the output
    static constexpr int LOADS = BN * CPR / NT;     // 16-byte chunks each thread loads of K
    static constexpr int LOADS_V = BN * CPRV / NT;  // and of V
    static_assert(LOADS * NT == BN * CPR && LOADS_V * NT == BN * CPRV, "the loads cover the tiles exactly");
};

// Per-work-group set-up shared by the attention and the pair-count kernels:
// the work item, its sequence, the lane's row interval and the key-tile list.
struct BlockPlan {
    WorkItem it;
    SeqGeom s;
    RowSpan span;
    TileList tiles;
    int32_t row;  // row inside the sequence owned by this lane
    BlockBand band;  // the work-group's rows together (union and intersection of their bands)
    // key tile [j0, j0 + BN) is visible to every valid row of the work-group
    __device__ __forceinline__ bool tile_full(int32_t j0, int32_t BN) const {
        return block_tile_full(band, s.Ck, j0, BN);
    }
};

template <int BN, int NW>
__device__ __forceinline__ bool plan_block(const KernelParams &p, bool split, BlockPlan &bp,
                                           const WorkItem &item) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    bp.it = item;
    if (!bp.it.valid) return false;
    bp.s = seq_geom(p, bp.it.b);
    if (p.levels && p.queue == nullptr) {
        // level l counted from the sequence's last q-tile: q-tile nq - 1 - l, and
        // the levels past the sequence onto the q-tiles past it (one to one)
        bp.it.qt = level_qtile(bp.it.qt, (bp.s.S_q + 32 * NW - 1) / (32 * NW));
    }
    const int32_t r0 = bp.it.qt * (32 * NW);
    if (r0 >= bp.s.S_q) return false;
    bp.row = r0 + wave * 32 + (lane & 31);
    bp.span = row_span(bp.s, p.causal, bp.row);
    // the work-group's BlockBand in closed form from a few of its rows (uniform
    // across the work-group: no reduction over the lanes, no barrier)
    const BlockBand band = qtile_band(bp.s, p.causal, r0, r0 + 32 * NW - 1);
    bp.band = band;
    int32_t tb = 0, te = (bp.s.S_kv + BN - 1) / BN;
    if (split) split_range(bp.s.S_kv, BN, p.num_splits, bp.it.sp, &tb, &te);
    // rows r0.. exist (r0 < S_q), so the context tiles are needed
    bp.tiles = make_tile_list(bp.s.Ck, true, band.lo, band.hi, BN, tb, te);
    return true;
}

// Raw buffer descriptor over [base, base + bytes): loads past the end return 0,
// which zero-fills the ragged tail of a sequence without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// SiLU on one 32-key block of raw scores x = q.k, in place, without the factor
// alpha: p = x / (1 + 2^(-alpha log2e x)) = SiLU(alpha x) / alpha; zeroed
// outside the row's visible keys when MASK.
//
// With MASK, the row's visibility of the block's 16 keys comes as one bit mask
// (lane_key_mask: bit i for key key0 + 8 (i / 4) + i % 4), and each score is
// ANDed with its bit spread over the word (v_bfe_i32: 0 or all ones): two VALU
// instructions per score instead of evaluating the interval test per key.
template <bool MASK>
__device__ __forceinline__ void silu_block(f32x16_t &x, float neg_alpha_log2e, const RowSpan &span,
                                           int key0) {
    const uint32_t vis = MASK ? lane_key_mask(span, key0) : 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float v = x[i];
        float pv = v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * neg_alpha_log2e));
        if constexpr (MASK) {
            // written out so the compiler keeps the two instructions (it otherwise
            // turns the select into a compare and a select)
            int32_t keep;
            asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(keep) : "v"(vis), "n"(i));
            pv = __builtin_bit_cast(float, __builtin_bit_cast(int32_t, pv) & keep);
        }
        x[i] = pv;
    }
}

// Online softmax: the reference maximum of a row moves only when a tile's maximum
// exceeds it by more than this (log2 units); exponents stay below 2^8, far from
// fp32's and bf16's ranges.
constexpr float kLazyRescale = 8.0f;

// Softmax scores of one block in the log2 domain, -inf outside the visible keys.
template <bool MASK>
__device__ __forceinline__ float scale_block(f32x16_t &x, float sc, const RowSpan &span, int key0) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float v = x[i] * sc;
        if constexpr (MASK) v = span_visible(span, key0 + 8 * (i >> 2) + (i & 3)) ? v : -INFINITY;
        x[i] = v;
        mx = fmaxf(mx, v);
    }
    return mx;
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land at
// LDS byte address lds_wave + 16 i (lds_wave must be the same for the whole wave).
// Issued through inline assembly so the compiler does not order later LDS reads
// of the other stage behind it; completion is awaited explicitly (vmcnt(0) and a
// barrier) before the stage is read.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc_words(const void *base, uint32_t bytes) {
    // the words are work-group uniform; readfirstlane keeps them in SGPRs, where
    // the buffer instruction needs its descriptor
    const uint64_t a = (uint64_t)base;
    return i32x4_t{__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a),
                   __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(a >> 32) & 0xffffu)),
                   __builtin_amdgcn_readfirstlane((int32_t)bytes), 0x00020000};
}
// M0 is a reserved register: the compiler neither preserves it across this
// statement nor relies on it elsewhere in these kernels (gfx9+ LDS instructions
// do not read M0; no other LDS-direct, message or indexed-register instruction
// is used), so setting it here is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_to_lds(const i32x4_t &rsrc, uint32_t lds_wave, uint32_t off) {
    lds_wave = __builtin_amdgcn_readfirstlane(lds_wave);  // wave-uniform by contract
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(lds_wave), "v"(off), "s"(rsrc)
        : "m0");
}
// 4 bytes per lane, landing at lds_wave + 4 i (same rules as load_to_lds).
__device__ __forceinline__ void load_to_lds4(const i32x4_t &rsrc, uint32_t lds_wave, uint32_t off) {
    lds_wave = __builtin_amdgcn_readfirstlane(lds_wave);  // wave-uniform by contract
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %1, %2, 0 offen lds"
        :
        : "s"(lds_wave), "v"(off), "s"(rsrc)
        : "m0");
}
#pragma clang diagnostic pop

// Transposed LDS read of 4 16-bit elements (gfx950): within each group of 16
// lanes, lane i receives element i%4 of the 8-byte chunks addressed by lanes
// 4r + i/4, r = 0..3.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint8_t *addr) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)addr));
#else
    return u32x2_t{0, 0};
#endif
}

__device__ __forceinline__ void wait_all_loads() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every global->LDS load of this wave landed
}
// The same wait at a fixed place in the instruction stream.  The compiler does
// not see the global->LDS loads, so it treats a vmcnt wait written with the
// builtin as free to merge into an earlier wait (it has moved the one closing a
// tile to before the tile's last eight MFMAs, serialising the next tile's load
// latency into the tile); as a fenced inline-assembly statement it stays where
// it is written.  (The prologue keeps the builtin: that one also tells the
// compiler that its own Q loads have completed.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void wait_all_loads_here() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

#pragma clang diagnostic pop

// Relative attention bias (HSTU explainer, "The relative attention bias").
// |a - b| of two int32 values: exact in 32-bit unsigned arithmetic.
__device__ __forceinline__ uint32_t abs_gap(int32_t a, int32_t b) {
    return a >= b ? (uint32_t)a - (uint32_t)b : (uint32_t)b - (uint32_t)a;
}
// Time-gap buckets: the bucket of a gap d (seconds) is how many of the edges
// 1, 5, 30, 60, 300, 1800, 3600, 86400, 604800, 2600000 are <= d.  No two edges
// share a binade [2^L, 2^(L+1)), so per binade the bucket is lo or lo + 1
// (lo: edges <= 2^L) with one threshold between them.  The per-head lookup
// table has one 16-byte entry per binade: entry 0 is d = 0, entry L + 1 covers
// [2^L, 2^(L+1)); fields {threshold, value below it, value from it on,
// bucket below | bucket from it on << 8}.
constexpr int kRabBinades = 33;
__device__ __forceinline__ int rab_binade(uint32_t d) { return 32 - __clz(d); }
__device__ __forceinline__ void rab_binade_entry(int idx, const float *tab, u32x4_t *out) {
    constexpr uint32_t kEdges[HSTU_RAB_TIME_BUCKETS - 1] = {1u,    5u,    30u,    60u,     300u,
                                                            1800u, 3600u, 86400u, 604800u, 2600000u};
    const uint32_t dmin = idx == 0 ? 0u : (1u << (idx - 1));
    int lo = 0;
#pragma unroll
    for (int k = 0; k < HSTU_RAB_TIME_BUCKETS - 1; ++k) lo += dmin >= kEdges[k] ? 1 : 0;
    uint32_t thr = 0xffffffffu;
#pragma unroll
    for (int k = 0; k < HSTU_RAB_TIME_BUCKETS - 1; ++k) thr = k == lo ? kEdges[k] : thr;
    const int hi = imin(lo + 1, HSTU_RAB_TIME_BUCKETS - 1);
    *out = u32x4_t{thr, __float_as_uint(tab[lo]), __float_as_uint(tab[hi]),
                   (uint32_t)lo | ((uint32_t)hi << 8)};
}
// bucket of d and its table value from the binade table (LDS)
__device__ __forceinline__ float rab_time_value(uint32_t d, const u32x4_t *oct) {
    const u32x4_t e = oct[rab_binade(d)];
    return __uint_as_float(d >= e.x ? e.z : e.y);
}
__device__ __forceinline__ int rab_bucket_of(uint32_t d, const u32x4_t *oct) {
    const u32x4_t e = oct[rab_binade(d)];
    return (int)(d >= e.x ? e.w >> 8 : e.w & 0xffu);
}

// Wave-wide minimum / maximum through DPP (quad permutes and row rotations give
// every lane its 16-lane row's result; four lane reads combine the rows).
__device__ __forceinline__ int32_t wave_min_dpp(int32_t x) {
    x = imin(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    x = imin(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    x = imin(x, __builtin_amdgcn_update_dpp(x, x, 0x124, 0xF, 0xF, false));  // row_ror 4
    x = imin(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));  // row_ror 8
    return imin(imin(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
                imin(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
__device__ __forceinline__ int32_t wave_max_dpp(int32_t x) {
    x = imax(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));
    x = imax(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));
    x = imax(x, __builtin_amdgcn_update_dpp(x, x, 0x124, 0xF, 0xF, false));
    x = imax(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));
    return imax(imax(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
                imax(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// Bias of one 32-key block of this lane's row, divided by alpha, as the initial
// accumulator of the block's score MFMAs:
//   x <- (pos[min(|row - j|, pmax)] + time[bucket(|t_row - t_j|)]) / alpha,
// so the MFMAs leave q.k + b / alpha and alpha times that is the biased score
// alpha q.k + b; from there the path is the one without bias.
// Element i is key key0 + 8(i/4) + i%4; ts4 points at that key0's timestamp in
// the LDS copy of the tile's key timestamps (16-byte aligned).
__device__ __forceinline__ void rab_block(f32x16_t &x, float inv_a, int row, int key0, const float *pos,
                                          int pmax, const int32_t *ts4, int32_t t_row, const u32x4_t *oct,
                                          bool has_pos, bool has_time) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        i32x4_t tk = {};
        if (has_time) tk = *(const i32x4_t *)(ts4 + 8 * q4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * q4 + e;
            float b = 0.0f;
            if (has_pos) {
                const int j = key0 + 8 * q4 + e;
                b = pos[imin(row > j ? row - j : j - row, pmax)];
            }
            if (has_time) b += rab_time_value(abs_gap(t_row, tk[e]), oct);
            x[i] = b * inv_a;
        }
    }
}

// The bias of one key tile (keys j0 .. j0 + BN - 1) for this lane's row, divided
// by alpha, as the initial accumulator of the tile's score MFMAs (see
// rab_block), with the two terms taken per tile where the tile allows it:
//  * time: the tile's smallest and largest key timestamps bound every gap of the
//    row; when both bounds fall into one bucket (for every row of the wave), the
//    time term is one value per row for the whole tile;
//  * position: in a tile wholly below the wave's rows (every key <= every row)
//    or wholly above them, |row - j| runs linearly over the tile's keys, so the
//    table is read at one per-lane base plus compile-time offsets.  The table in
//    LDS is padded with copies of its last entry up to P + BN - 1 entries, which
//    takes the clamp to P - 1 off those reads.
// Other tiles (the diagonal, gaps across a bucket edge) go element by element.
// Element (kb, i) is key j0 + 32 kb + 4 g + c with c = 8(i/4) + i%4.
template <int NKB, int BN>
__device__ __forceinline__ void rab_tile(f32x16_t *x, float inv_a, int row, int j0, int g, int wrow0,
                                         const float *pos, int P, const int32_t *ts, int32_t t_row,
                                         bool row_valid, int32_t S_kv, const u32x4_t *oct, bool has_pos,
                                         bool has_time, int lane) {
    float tv = 0.0f;
    bool time_tile = true;
    if (has_time) {
        int32_t lo = INT32_MAX, hi = INT32_MIN;
#pragma unroll
        for (int c = 0; c < (BN + 63) / 64; ++c) {
            const int k = c * 64 + lane;
            if (k < BN && j0 + k < S_kv) {
                const int32_t t = ts[k];
                lo = imin(lo, t);
                hi = imax(hi, t);
            }
        }
        lo = wave_min_dpp(lo);
        hi = wave_max_dpp(hi);
        uint32_t dlo, dhi;
        if (t_row >= hi) {
            dlo = abs_gap(t_row, hi);
            dhi = abs_gap(t_row, lo);
        } else if (t_row <= lo) {
            dlo = abs_gap(lo, t_row);
            dhi = abs_gap(hi, t_row);
        } else {
            dlo = 0u;
            dhi = max(abs_gap(t_row, lo), abs_gap(hi, t_row));
        }
        const bool one = !row_valid || rab_bucket_of(dlo, oct) == rab_bucket_of(dhi, oct);
        time_tile = __ballot(!one) == 0;
        tv = rab_time_value(dlo, oct);
    }
    if (!time_tile) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            rab_block(x[kb], inv_a, row, j0 + kb * 32 + 4 * g, pos, P - 1, ts + kb * 32 + 4 * g, t_row, oct,
                      has_pos, has_time);
        return;
    }
    const float tva = tv * inv_a;
    if (has_pos && wrow0 - j0 >= BN - 1) {
        // below: index row - j = (row - j0) - 4g - c, read at base + (BN - 5 - c) >= 0
        const int base = imin(row - j0, P + BN - 2) - 4 * g - (BN - 5);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int c = 32 * kb + 8 * (i >> 2) + (i & 3);
                x[kb][i] = fmaf(pos[base + (BN - 5 - c)], inv_a, tva);
            }
    } else if (has_pos && wrow0 + 31 < j0) {
        // above: index j - row = (j0 - row) + 4g + c
        const int base = imin(j0 - row, P - 1) + 4 * g;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int c = 32 * kb + 8 * (i >> 2) + (i & 3);
                x[kb][i] = fmaf(pos[base + c], inv_a, tva);
            }
    } else if (has_pos) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int j = j0 + 32 * kb + 4 * g + 8 * (i >> 2) + (i & 3);
                x[kb][i] = fmaf(pos[imin(row > j ? row - j : j - row, P - 1)], inv_a, tva);
            }
    } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) x[kb][i] = tva;
    }
}

// SiLU of one score without the factor alpha (see silu_block), unmasked.
__device__ __forceinline__ float silu_raw(float v, float neg_alpha_log2e) {
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * neg_alpha_log2e));
}

// One SiLU key tile of 64 keys (two 32-key blocks) for one wave at hdim 128 or
// 256 (k_addr: NKA lane offsets, the k-steps past them one swizzle period
// further on; v_addr: NVA, the 32-column blocks past them 64 NVA bytes further),
// software-pipelined so that the wave keeps the matrix pipe and the VALU busy
// together.  Written in issue order, one step per MFMA, with scheduling fences
// (sched_barrier) between steps so the compiler keeps the interleave (KS = D/16
// k-steps; 2 DV/32 = KS P.V steps per block):
//   A: block 0 scores (KS MFMAs)           + block 1 K operand reads
//   B: block 1 scores (KS MFMAs)           + block 0 SiLU (16/KS scores/step) + block 0 V^T reads
//   C: block 0 P.V    (KS MFMAs)           + block 1 SiLU (16/KS scores/step) + block 1 V^T reads
//   D: block 1 P.V    (KS MFMAs)
// The next tile's global->LDS loads (issue_load(0..KS-1)) are spread over phase A.
// Inside each step sched_group_barrier puts the MFMA first (mask 0x008), then
// the step's LDS reads (0x100), then its VALU work (0x002), so the matrix pipe
// is fed before the SiLU arithmetic of the same step.
// The fences change the instruction order only, never the arithmetic.
template <class E, int D, int NKA, int NVA, class IssueLoad>
__device__ __forceinline__ void silu_tile_pipelined(const uint8_t *stage, const uint32_t *k_addr,
                                                    const uint32_t *v_addr, const u32x4_t *qreg,
                                                    f32x16_t *oacc, float neg_alpha_log2e,
                                                    const f32x16_t &init0, const f32x16_t &init1,
                                                    IssueLoad &&issue_load) {
    using C = Tile<D, 64>;
    constexpr int KS = C::KSTEPS, NDB = C::NDB, SPS = 16 / KS;  // SiLU scores per step
    static_assert(C::NKB == 2 && (D == 128 || D == 256) && 2 * NDB == KS, "64-key tiles, hdim 128 or 256");
    auto kread = [&](int kb, int kk) {
        return *(const u32x4_t *)(stage + k_addr[kk % NKA] + kb * 32 * C::RB + (kk / NKA) * (NKA * 32));
    };
    // P.V step i of block kb: t2 = i / NDB (16-key half), nb = i % NDB (32-column block)
    auto vread = [&](int kb, int i) {
        const int t2 = i / NDB, nb = i % NDB;
        const uint8_t *va = stage + v_addr[nb % NVA] + (kb * 32 + 16 * t2) * C::RBV + (nb / NVA) * (NVA * 64);
        const u32x2_t a0 = lds_read_tr16(va);
        const u32x2_t a1 = lds_read_tr16(va + 8 * C::RBV);
        return u32x4_t{a0.x, a0.y, a1.x, a1.y};
    };
    auto pack8 = [&](const f32x16_t &x, int i0) {
        return u32x4_t{E::pack2(x[i0 + 0], x[i0 + 1]), E::pack2(x[i0 + 2], x[i0 + 3]),
                       E::pack2(x[i0 + 4], x[i0 + 5]), E::pack2(x[i0 + 6], x[i0 + 7])};
    };

    f32x16_t s0 = init0, s1 = init1;
    u32x4_t op0[KS], op1[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) op0[kk] = kread(0, kk);
    // Phases A-C run at wave priority 1 and the MFMA-only phase D at 0, so the
    // SIMD's other wave (another work-group, usually in a different phase) is
    // issued ahead of a wave that only feeds the matrix pipe (measured: about
    // 2 % on the long causal workload).
    __builtin_amdgcn_s_setprio(1);
    // A (also issues the next tile's global->LDS loads, one per step)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        s0 = E::mfma(op0[kk], qreg[kk], s0);
        op1[kk] = kread(1, kk);
        issue_load(kk);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    // B
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        s1 = E::mfma(op1[kk], qreg[kk], s1);
        op0[kk] = vread(0, kk);
#pragma unroll
        for (int e = 0; e < SPS; ++e) s0[SPS * kk + e] = silu_raw(s0[SPS * kk + e], neg_alpha_log2e);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8 * SPS, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    const u32x4_t p0[2] = {pack8(s0, 0), pack8(s0, 8)};
    // C
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        oacc[i % NDB] = E::mfma(op0[i], p0[i / NDB], oacc[i % NDB]);
        op1[i] = vread(1, i);
#pragma unroll
        for (int e = 0; e < SPS; ++e) s1[SPS * i + e] = silu_raw(s1[SPS * i + e], neg_alpha_log2e);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8 * SPS, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    const u32x4_t p1[2] = {pack8(s1, 0), pack8(s1, 8)};
    // D
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < KS; ++i) oacc[i % NDB] = E::mfma(op1[i], p1[i / NDB], oacc[i % NDB]);
}

// One softmax key tile of 64 keys (two 32-key blocks) for one wave at hdim 128 or
// 256, software-pipelined like silu_tile_pipelined, with the online softmax of
// the generic body (log2 domain, lazy reference maximum m_run, sum l_run):
//   A: block 0 scores (KS MFMAs)           + block 1 K operand reads + the next tile's loads
//      then block 0 scaled, its row maximum, the reference raised if needed
//   B: block 1 scores (KS MFMAs)           + block 0 exponentials + block 0 V^T reads
//   C: block 0 P.V    (KS MFMAs)           + block 1 scaled and its maximum + block 1 V^T reads
//      then the reference raised if needed (O, l and block 0's sum rescaled, after
//      block 0's P.V), block 1 exponentials
//   D: block 1 P.V    (KS MFMAs)
// Hidden scores come in through the initial accumulators as in the SiLU body
// (about -1e30 |alpha log2e| once scaled): their exponentials are exact zeros.
template <class E, int D, int NKA, int NVA, class IssueLoad>
__device__ __forceinline__ void softmax_tile_pipelined(const uint8_t *stage, const uint32_t *k_addr,
                                                       const uint32_t *v_addr, const u32x4_t *qreg,
                                                       f32x16_t *oacc, float sc, float &m_run, float &l_run,
                                                       const f32x16_t &init0, const f32x16_t &init1,
                                                       IssueLoad &&issue_load) {
    using C = Tile<D, 64>;
    constexpr int KS = C::KSTEPS, NDB = C::NDB, SPS = 16 / KS;
    static_assert(C::NKB == 2 && (D == 128 || D == 256) && 2 * NDB == KS, "64-key tiles, hdim 128 or 256");
    auto kread = [&](int kb, int kk) {
        return *(const u32x4_t *)(stage + k_addr[kk % NKA] + kb * 32 * C::RB + (kk / NKA) * (NKA * 32));
    };
    auto vread = [&](int kb, int i) {
        const int t2 = i / NDB, nb = i % NDB;
        const uint8_t *va = stage + v_addr[nb % NVA] + (kb * 32 + 16 * t2) * C::RBV + (nb / NVA) * (NVA * 64);
        const u32x2_t a0 = lds_read_tr16(va);
        const u32x2_t a1 = lds_read_tr16(va + 8 * C::RBV);
        return u32x4_t{a0.x, a0.y, a1.x, a1.y};
    };
    auto pack8 = [&](const f32x16_t &x, int i0) {
        return u32x4_t{E::pack2(x[i0 + 0], x[i0 + 1]), E::pack2(x[i0 + 2], x[i0 + 3]),
                       E::pack2(x[i0 + 4], x[i0 + 5]), E::pack2(x[i0 + 6], x[i0 + 7])};
    };
    // the row's maximum over both lane groups; a block without a visible key (all
    // its scores the masking value, -1e30 |sc| once scaled) gives -inf, so that it
    // never becomes the row's reference
    const float no_key = -5e29f * fabsf(sc);
    auto row_max = [&](float mx) {
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        return mx < no_key ? -INFINITY : mx;
    };
    // raise the reference to mx where it exceeds it by more than kLazyRescale:
    // O, l (and the sum so far of this tile) rescaled to the new reference
    auto raise_to = [&](float mx, float &lsum) {
        const bool raise = mx > m_run + kLazyRescale;
        if (__ballot(raise) != 0) {
            const float corr = raise ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;
            l_run *= corr;
            lsum *= corr;
#pragma unroll
            for (int nb = 0; nb < NDB; ++nb) oacc[nb] *= corr;
            m_run = raise ? mx : m_run;
        }
    };

    f32x16_t s0 = init0, s1 = init1;
    u32x4_t op0[KS], op1[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) op0[kk] = kread(0, kk);
    __builtin_amdgcn_s_setprio(1);
    // A
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        s0 = E::mfma(op0[kk], qreg[kk], s0);
        op1[kk] = kread(1, kk);
        issue_load(kk);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    float lsum = 0.0f;
    {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s0[i] *= sc;
            mx = fmaxf(mx, s0[i]);
        }
        raise_to(row_max(mx), lsum);
    }
    float m_use = m_run == -INFINITY ? 0.0f : m_run;
    // B
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        s1 = E::mfma(op1[kk], qreg[kk], s1);
        op0[kk] = vread(0, kk);
#pragma unroll
        for (int e = 0; e < SPS; ++e) {
            const float x = __builtin_amdgcn_exp2f(s0[SPS * kk + e] - m_use);
            lsum += x;
            s0[SPS * kk + e] = x;
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4 * SPS, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    const u32x4_t p0[2] = {pack8(s0, 0), pack8(s0, 8)};
    // C
    float mx1 = -INFINITY;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
        oacc[i % NDB] = E::mfma(op0[i], p0[i / NDB], oacc[i % NDB]);
        op1[i] = vread(1, i);
#pragma unroll
        for (int e = 0; e < SPS; ++e) {
            s1[SPS * i + e] *= sc;
            mx1 = fmaxf(mx1, s1[SPS * i + e]);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2 * SPS, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    raise_to(row_max(mx1), lsum);
    m_use = m_run == -INFINITY ? 0.0f : m_run;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float x = __builtin_amdgcn_exp2f(s1[i] - m_use);
        lsum += x;
        s1[i] = x;
    }
    const u32x4_t p1[2] = {pack8(s1, 0), pack8(s1, 8)};
    // D
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < KS; ++i) oacc[i % NDB] = E::mfma(op1[i], p1[i / NDB], oacc[i % NDB]);
    l_run += lsum;
}

// RAB: relative attention bias.  The bias is added to alpha q.k before the mask
// and the non-linearity; it enters as the score MFMAs' initial accumulator,
// divided by alpha (rab_tile), so the scores, the non-linearity and the epilogue
// are those of the variant without bias.
template <int DT, int D, bool SOFTMAX, bool SPLIT, int DV = D, bool RAB = false>
__global__ __launch_bounds__(64 * waves_for(D)) __attribute__((amdgpu_waves_per_eu(D == 256 ? 1 : 2, 2))) void hstu_fwd_kernel(KernelParams p) {
    constexpr int BN = key_tile_for(D);
    constexpr int NW = waves_for(D);
    using C = Tile<D, BN, NW, DV>;
    // K swizzle over the low 4 chunk bits (3 when a row has only 8 chunks);
    // V swizzle 4(r & 3) needs 16 chunks per row, 2(r & 3) with 8.  Rows of 12
    // chunks (hdim 96) are not swizzled (an XOR would leave the row).
    constexpr int kKSwz = C::CPR >= 16 ? 15 : (C::CPR == 8 ? 7 : 0);
    constexpr int kVSwz = C::CPRV >= 16 ? 4 : (C::CPRV == 8 ? 2 : 0);
    using E = Elem<DT>;
    // two stages of [K tile | V tile]
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][C::STAGE];
    // bias only: the head's positional table and each stage's key timestamps
    // (at least 64 entries: one wave-load)
    constexpr int TSN = RAB ? (BN < 64 ? 64 : BN) : 1;
    __shared__ float pos_lds[RAB ? HSTU_RAB_MAX_POS + BN - 1 : 1];
    __shared__ __attribute__((aligned(16))) int32_t ts_lds[2][TSN];
    __shared__ u32x4_t oct_lds[RAB ? kRabBinades : 1];  // time-bucket lookup per binade
    __shared__ int32_t next_item[2][2];

    // The kernel arguments are re-read for every item through a pointer the
    // compiler cannot see through; otherwise it hoists their loads out of the
    // item loop and keeps the values live across it, in registers the tile loop
    // needs.
    auto args = [&]() -> const KernelParams & {
        auto *a = (const __attribute__((address_space(4))) KernelParams *)
            __builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(a));
        return *(const KernelParams *)a;
    };
    // Persistent schedule (queues written by hstu_plan_kernel): the work-group's
    // own queue is that of its XCD (work-group ids go to the 8 XCDs in turn).
    // Thread 0 reserves the next item (an atomic on the queue's counter) when
    // the current item starts its next-to-last key tile and loads the item's
    // entry when it starts the last, so both latencies hide behind those tiles.
    // (Reserving at the start of an item instead doubled the items in flight and
    // with them the keys competing for the XCD's L2: 6 % slower.)  The queue's
    // addresses are derived from the re-read arguments at each use, so that
    // nothing of them stays live in scalar registers across the item loop.
    constexpr uint32_t kNone = 0xffffffffu;
    constexpr uint64_t kNoItem = 0xffffffffu;  // bh = -1
    const int xq = (int)(blockIdx.x % 8);
    uint32_t reserved = kNone;
    uint64_t entry = kNoItem;
    bool have_entry = false;
    // (the planning kernel fills each queue's unused tail with "no item", so
    // one load tells both whether and which)
    auto queue_item = [&](const KernelParams &a, int y, uint32_t i) -> uint64_t {
        const gmem_t<uint64_t> *list = (const gmem_t<uint64_t> *)((const uint8_t *)a.queue + kQueueHeader);
        const uint32_t per_queue = (uint32_t)(grid_size(a) / 8);
        return i < per_queue ? list[(size_t)y * per_queue + i] : kNoItem;
    };
    auto reserve_next = [&]() {
        const KernelParams &a = args();
        if (a.queue != nullptr && threadIdx.x == 0 && reserved == kNone)
            reserved = atomicAdd(&a.queue[xq], 1u);
    };
    auto fetch_next = [&]() {
        const KernelParams &a = args();
        if (a.queue != nullptr && threadIdx.x == 0 && !have_entry) {
            if (reserved == kNone) reserved = atomicAdd(&a.queue[xq], 1u);
            entry = queue_item(a, xq, reserved);
            have_entry = true;
        }
    };

    // One work item (sequence, head, q-tile, split) from plan to output.
    auto run_item = [&](const KernelParams &p, const WorkItem &item) __attribute__((always_inline)) {
        BlockPlan bp;
        const bool planned = plan_block<BN, NW>(p, SPLIT, bp, item);
        // heavy q-tiles: the chunk of this item (hslot >= 0 when the q-tile is cut);
        // the first chunk's work-group records the q-tile for the combine pass.
        // Only the first p.heavy levels (item.qt before plan_block turned it into
        // the q-tile) are cut.
        int32_t hslot = -1;
        if (!SPLIT && item.qt < p.heavy) {
            const int64_t hq = ((int64_t)item.b * p.H + item.h) * p.heavy + item.qt;
            int32_t nsp = 0;
            if (planned) nsp = heavy_splits(bp.tiles.count(), p.heavy_tiles, p.num_splits);
            if (item.valid && item.sp == 0 && threadIdx.x == 0) {
                const int32_t r0 = bp.it.qt * C::BM;
                const int32_t rows = planned ? imin(C::BM, bp.s.S_q - r0) : 0;
                p.hmeta[2 * hq] = nsp | (rows << 8);
                p.hmeta[2 * hq + 1] = planned ? (int32_t)(bp.s.q0 + r0) : 0;
            }
            if (!planned || item.sp >= nsp) return;
            if (nsp > 1) {
                int32_t nb, ne;
                heavy_chunk(bp.tiles.count(), nsp, item.sp, &nb, &ne);
                bp.tiles = bp.tiles.sub(nb, ne);
                hslot = (int32_t)(hq * p.num_splits + item.sp);
            }
        }
        if (!planned) return;
        const SeqGeom &s = bp.s;
        const RowSpan &span = bp.span;
        // the lane's constants are derived per item (an opaque copy of the thread
        // id keeps the compiler from hoisting them out of the item loop)
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
        const int h = bp.it.h;
        const int ntiles = bp.tiles.count();

        // Buffer descriptors over this (sequence, head): rows past the sequence read as 0.
        const uint32_t qs2 = (uint32_t)p.q_stride * 2, ks2 = (uint32_t)p.k_stride * 2,
                       vs2 = (uint32_t)p.v_stride * 2;
        const __amdgpu_buffer_rsrc_t qr =
            make_rsrc((const uint16_t *)p.q + s.q0 * p.q_stride + h * D, (uint32_t)s.S_q * qs2);
        const i32x4_t kr =
            make_rsrc_words((const uint16_t *)p.k + s.kv0 * p.k_stride + h * D, (uint32_t)s.S_kv * ks2);
        const i32x4_t vr =
            make_rsrc_words((const uint16_t *)p.v + s.kv0 * p.v_stride + h * DV, (uint32_t)s.S_kv * vs2);

        // ---- Q^T operand: lane holds d = 16*kk + 8*g .. +7 of its row
        u32x4_t qreg[C::KSTEPS];
#pragma unroll
        for (int kk = 0; kk < C::KSTEPS; ++kk)
            qreg[kk] = buf_load16(qr, (uint32_t)bp.row * qs2 + (kk * 16 + g * 8) * 2);

        // ---- global -> LDS loads of key tile t into stage b.  Wave-load c of wave w
        //      fills physical chunks [(4c + w) 64, +64); the chunk a lane lands on
        //      decides which logical chunk (swizzle undone) it fetches.
        //      Physical chunk (c NT + tid) is row (c NT + tid) / CPR, chunk (c NT + tid) %
        //      CPR; the lane's byte offset is its row's offset plus the swizzled chunk.
        //      With whole rows per wave-load (CPR divides NT) the part that grows with c
        //      is uniform (it goes with the tile into the scalar part of the address),
        //      and when RPC is a multiple of the swizzle period the per-lane parts of all
        //      c coincide (one register each).
        constexpr bool kRowsK = C::NT % C::CPR == 0, kRowsV = C::NT % C::CPRV == 0;
        constexpr int RPC = kRowsK ? C::NT / C::CPR : 0, RPCV = kRowsV ? C::NT / C::CPRV : 0;
        uint32_t k_lane[C::LOADS], v_lane[C::LOADS_V];
#pragma unroll
        for (int c = 0; c < C::LOADS; ++c) {
            const int phys = kRowsK ? tid : c * C::NT + tid;
            const int row = phys / C::CPR, pc = phys % C::CPR;
            const int rsw = (RPC & kKSwz) == 0 ? row : c * RPC + row;
            k_lane[c] = (uint32_t)row * ks2 + (uint32_t)(pc ^ (rsw & kKSwz)) * 16;
        }
#pragma unroll
        for (int c = 0; c < C::LOADS_V; ++c) {
            const int phys = kRowsV ? tid : c * C::NT + tid;
            const int row = phys / C::CPRV, pc = phys % C::CPRV;
            v_lane[c] = (uint32_t)row * vs2 + (uint32_t)(pc ^ (kVSwz * (row & 3))) * 16;
        }
        // LDS byte address of this wave's first landing slot (wave-uniform)
        const int wave_u = __builtin_amdgcn_readfirstlane(wave);
        const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void_t *)&lds[0][0] + (uint32_t)wave_u * 1024;

        // ---- relative attention bias set-up
        const bool has_pos = RAB && p.rab_pos != nullptr, has_time = RAB && p.rab_ts != nullptr;
        int32_t t_row = 0;
        i32x4_t tsr = {};
        const int wrow0 = bp.it.qt * C::BM + wave_u * 32;  // first row of this wave
        if constexpr (RAB) {
            if (has_pos) {
                // The head's table, padded with its last entry up to P + BN - 1 entries
                // (see rab_tile): whole 64-entry chunks go global -> LDS directly (they
                // land with the first key tile, before the prologue's barrier), the
                // rest (< 64 + BN - 1 <= NT entries) through registers, one per thread.
                const int P = p.rab_pos_len, full = P / 64;
                const float *ph = p.rab_pos + (int64_t)h * P;
                const i32x4_t pr = make_rsrc_words(ph, (uint32_t)P * 4u);
                const uint32_t pos_base = (uint32_t)(uintptr_t)(lds_void_t *)&pos_lds[0];
                for (int c = wave_u; c < full; c += NW)
                    load_to_lds4(pr, pos_base + (uint32_t)c * 256u, (uint32_t)(c * 64 + lane) * 4u);
                const int i = full * 64 + tid;
                if (i < P + BN - 1) pos_lds[i] = ph[imin(i, P - 1)];
            }
            if (has_time) {
                if (tid < kRabBinades)
                    rab_binade_entry(tid, p.rab_time + h * HSTU_RAB_TIME_BUCKETS, &oct_lds[tid]);
                t_row = bp.row < s.S_q ? p.rab_ts[s.q0 + bp.row] : 0;
                tsr = make_rsrc_words(p.rab_ts + s.kv0, (uint32_t)s.S_kv * 4u);
            }
        }
        const uint32_t ts_base = (uint32_t)(uintptr_t)(lds_void_t *)&ts_lds[0][0];
        // the key timestamps of tile t into stage b: wave w < TSN / 64 loads 64 of them
        auto issue_ts = [&](int t, int b) {
            if constexpr (RAB) {
                if (has_time && wave_u < TSN / 64)
                    load_to_lds4(tsr, ts_base + (uint32_t)(b * TSN + wave_u * 64) * 4u,
                                 (uint32_t)(t * BN + wave_u * 64 + lane) * 4u);
            }
        };
        // load idx of key tile t into stage b: idx < LOADS are K chunks, the rest V
        constexpr int LPT = C::LOADS + C::LOADS_V;  // loads per tile and wave
        auto issue_one = [&](int t, int b, int idx) {
            if (idx < C::LOADS) {
                const int c = idx;
                const uint32_t r = (uint32_t)(t * BN + c * RPC);  // uniform
                load_to_lds(kr, lds_base + b * C::STAGE + c * NW * 1024, k_lane[c] + r * ks2);
            } else {
                const int c = idx - C::LOADS;
                const uint32_t r = (uint32_t)(t * BN + c * RPCV);
                load_to_lds(vr, lds_base + b * C::STAGE + C::TILE_BYTES + c * NW * 1024, v_lane[c] + r * vs2);
            }
        };
        auto issue_loads = [&](int t, int b) {
#pragma unroll
            for (int idx = 0; idx < LPT; ++idx) issue_one(t, b, idx);
            issue_ts(t, b);
        };

        // ---- per-lane LDS read addresses (stage 0; stage 1 adds 2 * TILE_BYTES)
        // K operand of S^T = K Q^T: row 32kb + r32, logical chunk 2kk + g
        // (the swizzle mixes the low log2(NKA)+1 chunk bits, so NKA k-steps get their own
        //  lane offsets and later k-steps repeat them one swizzle period further on)
        constexpr int NKA = kKSwz ? (kKSwz + 1) / 2 : 1, NVA = kVSwz == 4 ? 4 : (kVSwz == 2 ? 2 : 1);
        uint32_t k_addr[NKA];
#pragma unroll
        for (int m = 0; m < NKA; ++m)
            k_addr[m] = (uint32_t)(r32 * C::RB + (((2 * m + g) ^ (r32 & kKSwz)) * 16));
        // V^T operand (transposed read): row K0 + 4g + (i/4), columns 32nb + 16hb + 4(i%4)
        const int i16 = lane & 15, hb = (lane >> 4) & 1;
        const int vy = kVSwz * ((i16 >> 2) & 3);
        uint32_t v_addr[NVA];
#pragma unroll
        for (int b2 = 0; b2 < NVA; ++b2)
            v_addr[b2] = (uint32_t)(C::TILE_BYTES + (4 * g + (i16 >> 2)) * C::RBV +
                                    (((4 * b2 + 2 * hb + ((i16 & 3) >> 1)) ^ vy) * 16) + (i16 & 1) * 8);

        f32x16_t oacc[C::NDB];
#pragma unroll
        for (int nb = 0; nb < C::NDB; ++nb) oacc[nb] = f32x16_t{};
        float m_run = -INFINITY, l_run = 0.f;
        const float neg_alpha_log2e = -p.alpha * kLog2e;
        const float sc_soft = p.alpha * kLog2e;
        // the bias's scalars, held in registers: re-read from the (re-read per
        // item) arguments inside the tile loop, their loads each waited for the
        // outstanding LDS reads too (a scalar-memory wait)
        float rab_inv_alpha = p.inv_alpha;
        int32_t rab_pos_len = p.rab_pos_len;
        if constexpr (RAB) asm volatile("" : "+s"(rab_inv_alpha), "+s"(rab_pos_len));
        const uint8_t *lds0 = &lds[0][0];

        if (ntiles > 0) issue_loads(bp.tiles.at(0), 0);
        wait_all_loads();
        __syncthreads();
        // key tile of step n's loads: tile n + 1, or, after the last tile, a tile
        // past the sequence's end (the buffer range turns those loads into zeros
        // without memory traffic, so no load needs a branch)
        auto tile_ahead = [&](int n) { return n + 1 < ntiles ? bp.tiles.at(n + 1) : (s.S_kv + 2 * BN - 1) / BN; };

        // Runs step(n, stage) on tiles n, n + 1, ... while more(n) holds.  Tile n
        // uses ring stage n & 1, passed as a template constant: each step body
        // exists once per stage, so the stage sits in the immediate offsets of the
        // LDS reads instead of costing address instructions on every tile.
        auto run_tiles = [&](int &n, auto &&more, auto &&step) {
            while (more(n)) {
                if ((n & 1) == 0) {
                    step(n, std::integral_constant<int, 0>{});
                    if (!more(++n)) break;
                }
                step(n, std::integral_constant<int, 1>{});
                ++n;
            }
        };
        // the end of a step: the next tile's loads have landed and every wave is
        // done with this tile's stage
        auto end_step = [&]() {
            wait_all_loads_here();
            __syncthreads();
        };

        // one key tile through the generic body (any mask, any variant)
        auto generic_step = [&](int n, auto stage_const) {
            constexpr int buf = decltype(stage_const)::value;
            constexpr int nbuf = buf ^ 1;
            if (n == ntiles - 2) reserve_next();
            if (n == ntiles - 1) fetch_next();
            const int t_next = tile_ahead(n);
            const int j0 = bp.tiles.at(n) * BN;
            const int32_t st = tile_state(span, j0, j0 + BN);
            const bool wave_any = __ballot(st != kTileEmpty) != 0;
            const bool wave_mask = __ballot(span.valid && st != kTileFull) != 0;

            issue_loads(t_next, nbuf);
            if (wave_any) {
                const uint8_t *stage = lds0 + buf * C::STAGE;
                // scores and non-linearity at wave priority 1, P.V at 0 (as in the
                // pipelined tile)
                __builtin_amdgcn_s_setprio(1);
                // ---- S^T = K Q^T, the key blocks' MFMA chains interleaved
                f32x16_t sacc[C::NKB];
                if constexpr (RAB) {
                    rab_tile<C::NKB, BN>(sacc, rab_inv_alpha, bp.row, j0, g, wrow0, pos_lds, rab_pos_len,
                                         ts_lds[buf], t_row, bp.row < s.S_q, s.S_kv, oct_lds, has_pos,
                                         has_time, lane);
                } else {
#pragma unroll
                    for (int kb = 0; kb < C::NKB; ++kb) sacc[kb] = f32x16_t{};
                }
#pragma unroll
                for (int kk = 0; kk < C::KSTEPS; ++kk) {
#pragma unroll
                    for (int kb = 0; kb < C::NKB; ++kb) {
                        const uint8_t *ka = stage + k_addr[kk % NKA] + kb * 32 * C::RB + (kk / NKA) * (NKA * 32);
                        sacc[kb] = E::mfma(*(const u32x4_t *)ka, qreg[kk], sacc[kb]);
                    }
                }

                // ---- mask + non-linearity; element i of block kb is key
                //      j0 + 32*kb + 8*(i/4) + 4*g + i%4 of this lane's row
                if constexpr (!SOFTMAX) {
                    // p = x sigmoid(alpha x); the factor alpha of SiLU(alpha x) goes into the epilogue
                    if (wave_mask) {
#pragma unroll
                        for (int kb = 0; kb < C::NKB; ++kb)
                            silu_block<true>(sacc[kb], neg_alpha_log2e, span, j0 + kb * 32 + 4 * g);
                    } else {
#pragma unroll
                        for (int kb = 0; kb < C::NKB; ++kb)
                            silu_block<false>(sacc[kb], neg_alpha_log2e, span, 0);
                    }
                } else {
                    float mx = -INFINITY;
                    if (wave_mask) {
#pragma unroll
                        for (int kb = 0; kb < C::NKB; ++kb)
                            mx = fmaxf(mx, scale_block<true>(sacc[kb], sc_soft, span, j0 + kb * 32 + 4 * g));
                    } else {
#pragma unroll
                        for (int kb = 0; kb < C::NKB; ++kb)
                            mx = fmaxf(mx, scale_block<false>(sacc[kb], sc_soft, span, 0));
                    }
                    mx = fmaxf(mx, __shfl_xor(mx, 32));
                    // lazy rescale: the row's reference maximum m_run moves (and O and
                    // l are rescaled to it) only when the tile's maximum exceeds it by
                    // more than kLazyRescale (log2 units), so every exponent stays at
                    // most 2^kLazyRescale; the result is the same up to rounding, and
                    // the rescale runs a few times per row instead of on most tiles
                    const bool raise = mx > m_run + kLazyRescale;  // m_run = -inf: any finite max
                    if (__ballot(raise) != 0) {
                        const float corr = raise ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;
                        l_run *= corr;
#pragma unroll
                        for (int nb = 0; nb < C::NDB; ++nb) oacc[nb] *= corr;
                        m_run = raise ? mx : m_run;
                    }
                    const float m_use = m_run == -INFINITY ? 0.0f : m_run;
                    float lsum = 0.f;
#pragma unroll
                    for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const float e = __builtin_amdgcn_exp2f(sacc[kb][i] - m_use);
                            lsum += e;
                            sacc[kb][i] = e;
                        }
                    }
                    l_run += lsum;
                }

                __builtin_amdgcn_s_setprio(0);
                // ---- O^T += V^T P^T; MFMA step (kb, t2) covers keys
                //      32kb + 16t2 + {4g..4g+3, 8+4g..8+4g+3} in both operands
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
                    for (int t2 = 0; t2 < 2; ++t2) {
                        const int i0 = 8 * t2;
                        const u32x4_t pb = {E::pack2(sacc[kb][i0 + 0], sacc[kb][i0 + 1]),
                                            E::pack2(sacc[kb][i0 + 2], sacc[kb][i0 + 3]),
                                            E::pack2(sacc[kb][i0 + 4], sacc[kb][i0 + 5]),
                                            E::pack2(sacc[kb][i0 + 6], sacc[kb][i0 + 7])};
                        const int key0 = kb * 32 + 16 * t2;
#pragma unroll
                        for (int nb = 0; nb < C::NDB; ++nb) {
                            const uint8_t *va = stage + v_addr[nb % NVA] + key0 * C::RBV + (nb / NVA) * (NVA * 64);
                            const u32x2_t a0 = lds_read_tr16(va);
                            const u32x2_t a1 = lds_read_tr16(va + 8 * C::RBV);
                            oacc[nb] = E::mfma(u32x4_t{a0.x, a0.y, a1.x, a1.y}, pb, oacc[nb]);
                        }
                    }
                }
            }

            end_step();
        };
        // (the softmax body at hdim 256 would spill: it keeps the generic body there)
        if constexpr (BN == 64 && (D == 128 || (D == 256 && !SOFTMAX)) && DV == D) {
            // Every key tile runs through the software-pipelined body.  In a tile
            // that some valid row of the work-group sees only in part, the mask
            // enters the score MFMAs' initial accumulator: a hidden score starts at
            // mask_val = 1e30 with the sign of -alpha, so that -alpha log2e times it
            // is huge and positive, exp2 of it +inf, and SiLU of it exactly zero
            // (softmax: alpha log2e times it is huge and negative, its exponential
            // exactly zero; with the bias, a visible score keeps its bias and a
            // hidden one is replaced).  Building the accumulators costs two VALU instructions per
            // score (v_bfe_i32 of the lane's key bit, then a bitfield select), only
            // in those tiles; one body, one call site, so the loop keeps one
            // register set.  A wave none of whose rows sees such a tile only issues
            // its share of the next tile's loads.
            const float mask_val = copysignf(1e30f, neg_alpha_log2e);
            static_assert(LPT <= C::KSTEPS, "phase A issues every load of the next tile");
            auto step = [&](int n, auto stage_const) {
                constexpr int buf = decltype(stage_const)::value;
                constexpr int nbuf = buf ^ 1;
                if (n == ntiles - 2) reserve_next();
                if (n == ntiles - 1) fetch_next();
                const int t_next = tile_ahead(n);
                const int j0 = bp.tiles.at(n) * BN;
                f32x16_t init[2] = {};
                if constexpr (RAB) {
                    rab_tile<2, BN>(init, rab_inv_alpha, bp.row, j0, g, wrow0, pos_lds, rab_pos_len, ts_lds[buf],
                                    t_row, bp.row < s.S_q, s.S_kv, oct_lds, has_pos, has_time, lane);
                    issue_ts(t_next, nbuf);
                }
                bool wave_any = true;
                if (!bp.tile_full(j0, BN)) {
                    wave_any = __ballot(tile_state(span, j0, j0 + BN) != kTileEmpty) != 0;
                    const uint32_t vis = lane_key_mask(span, j0 + 4 * g);
                    const uint32_t mv = __builtin_bit_cast(uint32_t, mask_val);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            int32_t keep;  // bit 16 kb + i of vis spread over the word
                            asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(keep) : "v"(vis), "n"(16 * kb + i));
                            // (through a scalar copy: __builtin_bit_cast of a vector element
                            // read the vector's first element here)
                            const float cur = init[kb][i];
                            const uint32_t ib = __float_as_uint(cur);
                            init[kb][i] = __uint_as_float((ib & (uint32_t)keep) | (mv & ~(uint32_t)keep));
                        }
                }
                if (wave_any) {
                    auto issue = [&](int idx) {
                        if (idx < LPT) issue_one(t_next, nbuf, idx);
                    };
                    if constexpr (SOFTMAX)
                        softmax_tile_pipelined<E, D, NKA, NVA>(lds0 + buf * C::STAGE, k_addr, v_addr, qreg, oacc,
                                                               sc_soft, m_run, l_run, init[0], init[1], issue);
                    else
                        silu_tile_pipelined<E, D, NKA, NVA>(lds0 + buf * C::STAGE, k_addr, v_addr, qreg, oacc,
                                                            neg_alpha_log2e, init[0], init[1], issue);
                } else {
#pragma unroll
                    for (int idx = 0; idx < LPT; ++idx) issue_one(t_next, nbuf, idx);
                }
                end_step();
            };
            int n = 0;
            run_tiles(n, [&](int n) { return n < ntiles; }, step);
        } else {
            int n = 0;
            run_tiles(n, [&](int n) { return n < ntiles; }, generic_step);
        }

        // ---- epilogue: lane holds columns 32nb + 8(i/4) + 4g + i%4 of its row
        float scale = s.attn_scale * p.alpha;
        float lse_val = 0.f;
        if constexpr (SOFTMAX) {
            const float l = l_run + __shfl_xor(l_run, 32);
            scale = l > 0.f ? s.attn_scale / l : 0.f;
            lse_val = l > 0.f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
        }
        // (a lane whose row lies past the sequence still takes part in the
        // staged store below; only its row is not written)
        if (SPLIT && !span.valid) return;
        const int64_t grow = s.q0 + bp.row;  // token row of o
        if (!SPLIT && hslot >= 0) {
            // a chunk of a cut q-tile: fp32 partial rows, scaled like the split-KV
            // partials; the combine pass adds the chunks up (softmax: by their LSEs)
            if (!span.valid) return;
            const int64_t prow = (int64_t)hslot * C::BM + (bp.row - bp.it.qt * C::BM);
            float *pp = p.hpart_o + prow * DV + 4 * g;
#pragma unroll
            for (int nb = 0; nb < C::NDB; ++nb) {
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const f32x16_t &a = oacc[nb];
                    *(f32x4_t *)(pp + nb * 32 + 8 * i4) =
                        f32x4_t{a[4 * i4] * scale, a[4 * i4 + 1] * scale, a[4 * i4 + 2] * scale,
                                a[4 * i4 + 3] * scale};
                }
            }
            if constexpr (SOFTMAX) {
                if (g == 0) p.hpart_lse[prow] = lse_val;
            }
            return;
        }
        if constexpr (!SPLIT) {
            // The wave's 32 output rows go through LDS (both ring stages are free
            // once the last tile's barrier has passed; each wave uses a region of
            // its own, so no barrier is needed here) and leave as whole rows: a
            // lane holds 8-byte pieces of its row, scattered over 16-byte chunks;
            // read back, each lane stores one 16-byte chunk and the wave writes
            // LPR-lane runs of complete rows (8 stores for hdim 128 instead of 16
            // stores of 32 scattered 16-byte pieces).  Rows of CH 16-byte chunks
            // sit at a pitch of LPR chunks (a power of two), chunk c of row r at
            // c ^ (r & SWZ) against bank conflicts.
            constexpr int CH = DV / 8;
            constexpr int LPR = CH <= 8 ? 8 : (CH <= 16 ? 16 : 32);
            constexpr int SWZ = (LPR < 16 ? LPR : 16) - 1;
            constexpr int PITCH = LPR * 16;
            static_assert(NW * 32 * PITCH <= 2 * C::STAGE, "the output staging fits in the ring");
            uint8_t *stg = &lds[0][0] + wave * 32 * PITCH;
#pragma unroll
            for (int nb = 0; nb < C::NDB; ++nb) {
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const f32x16_t &a = oacc[nb];
                    const int c = 4 * nb + i4;
                    *(u32x2_t *)(stg + r32 * PITCH + ((c ^ (r32 & SWZ)) * 16) + 8 * g) =
                        u32x2_t{E::pack2(a[4 * i4] * scale, a[4 * i4 + 1] * scale),
                                E::pack2(a[4 * i4 + 2] * scale, a[4 * i4 + 3] * scale)};
                }
            }
            constexpr int RPI = 64 / LPR;  // rows per store instruction
            const int c = lane % LPR;
            const int64_t wtok = s.q0 + (int64_t)wrow0;  // token of the wave's first row
            // every read back first, then the stores; the output's base and stride
            // in registers (read from the arguments after a store, they would be
            // reloaded, and waited for, before each store)
            u32x4_t v[32 / RPI];
#pragma unroll
            for (int k = 0; k < 32 / RPI; ++k) {
                const int r = k * RPI + lane / LPR;
                v[k] = *(const u32x4_t *)(stg + r * PITCH + ((c ^ (r & SWZ)) * 16));
            }
            uint16_t *const o_row = (uint16_t *)p.o + wtok * p.o_stride + h * DV + c * 8;
            const int64_t o_stride = p.o_stride;
#pragma unroll
            for (int k = 0; k < 32 / RPI; ++k) {
                const int r = k * RPI + lane / LPR;
                if (c < CH && wrow0 + r < s.S_q) *(u32x4_t *)(o_row + r * o_stride) = v[k];
            }
            if constexpr (SOFTMAX) {
                if (p.lse != nullptr && g == 0 && span.valid) {
                    const int64_t li = p.jagged ? (int64_t)h * p.total_rows + grow
                                                : ((int64_t)bp.it.b * p.H + h) * p.seqlen_q + bp.row;
                    p.lse[li] = lse_val;
                }
            }
        } else {
            // fp32 partials, already multiplied by attn_scale (softmax: normalised
            // by this split's own sum; the combine pass reweights by the LSEs)
            const int64_t prow = ((int64_t)bp.it.sp * p.total_rows + grow) * p.H + h;
            float *pp = p.part_o + prow * DV + 4 * g;
#pragma unroll
            for (int nb = 0; nb < C::NDB; ++nb) {
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const f32x16_t &a = oacc[nb];
                    *(f32x4_t *)(pp + nb * 32 + 8 * i4) =
                        f32x4_t{a[4 * i4] * scale, a[4 * i4 + 1] * scale, a[4 * i4 + 2] * scale,
                                a[4 * i4 + 3] * scale};
                }
            }
            if constexpr (SOFTMAX) {
                if (g == 0) p.part_lse[prow] = lse_val;
            }
        }
    };

    // Persistent schedule: the grid holds about as many work-groups as fit on the
    // chip at once, and each takes items until none are left.  take() turns the
    // prefetched entry (fetched now if the item had no tiles) into the next item
    // or, once the own queue is empty, tries the other XCDs' queues in turn;
    // counters only grow, so every work-group ends after at most all items plus
    // 8 failed takes.  The entry reaches all waves through LDS.
    auto take = [&](int k) -> int2 {
        if (threadIdx.x == 0) {
            fetch_next();
            const KernelParams &a = args();
            uint64_t e = entry;
            for (int t = 1; t < 8 && e == kNoItem; ++t) {
                const int y = (xq + t) & 7;
                e = queue_item(a, y, atomicAdd(&a.queue[y], 1u));
            }
            reserved = kNone;
            have_entry = false;
            next_item[k & 1][0] = (int32_t)(uint32_t)e;
            next_item[k & 1][1] = (int32_t)(e >> 32);
        }
        // two slots: a wave still reading slot k & 1 cannot see it overwritten
        // before it has passed the barrier of take k + 1
        __syncthreads();
        // work-group uniform: keeps the loop and everything derived from the
        // item in scalar registers
        return int2{__builtin_amdgcn_readfirstlane(next_item[k & 1][0]),
                    __builtin_amdgcn_readfirstlane(next_item[k & 1][1])};
    };
    // (one call site, so the item body is inlined once)
    for (int k = 0;; ++k) {
        WorkItem it;
        const KernelParams &a = args();
        if (a.queue == nullptr) {
            // one item per work-group, the work-group id
            if (k > 0) break;
            it = decode_work(a, blockIdx.x);
        } else {
            const int2 e = take(k);
            if (e.x < 0) break;
            it.b = e.x / a.H;
            it.h = e.x % a.H;
            it.qt = e.y >> 8;
            it.sp = e.y & 255;
            it.valid = true;
        }
        run_item(args(), it);
    }
}

// Split-KV combine: one thread per (row, head, 4 columns); the 32 threads of a
// (row, head) read one contiguous 512-byte slice of every split's partial row.
//   SiLU:    o = sum_c o_c
//   softmax: lse = ln sum_c exp(lse_c); o = sum_c exp(lse_c - lse) o_c
//            (a row no split sees: o = 0, lse = -inf)
// HBM-bound: the splits are read in unrolled chunks of CH, every load of a
// chunk (LSEs and partial rows) issued before any is used, and the softmax
// weights are folded in with a running maximum, so the whole reduction is one
// pass with CH loads per thread in flight.
template <int DT, bool SOFTMAX>
__global__ __launch_bounds__(256) void hstu_combine_kernel(KernelParams p, int D) {
    using E = Elem<DT>;
    constexpr int CH = 16;
    const int nchunk = D / 4;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)p.total_rows * p.H * nchunk;
    if (idx >= total) return;
    const int chunk = (int)(idx % nchunk);
    const int64_t rh = idx / nchunk;  // row * H + h
    const int64_t split_stride = (int64_t)p.total_rows * p.H;
    const float *po = p.part_o + rh * D + chunk * 4;
    const int64_t po_stride = split_stride * D;
    const float *pl = p.part_lse + rh;
    const int ns = p.num_splits;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, sum = 0.f;  // softmax: running max of the LSEs, sum of exp(lse_c - m)
    for (int c0 = 0; c0 < ns; c0 += CH) {
        f32x4_t v[CH];
        float l[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bool in = c0 + c < ns;
            v[c] = in ? *(const f32x4_t *)(po + (c0 + c) * po_stride) : f32x4_t{0.f, 0.f, 0.f, 0.f};
            if constexpr (SOFTMAX) l[c] = in ? pl[(c0 + c) * split_stride] : -INFINITY;
        }
        if constexpr (!SOFTMAX) {
#pragma unroll
            for (int c = 0; c < CH; ++c) acc += v[c];
        } else {
            float cm = m;
#pragma unroll
            for (int c = 0; c < CH; ++c) cm = fmaxf(cm, l[c]);
            if (cm == -INFINITY) continue;  // no split of this chunk (or before) saw a key
            // rescale what was accumulated against the new maximum (m = -inf: factor 0)
            const float r = __builtin_amdgcn_exp2f((m - cm) * kLog2e);
            sum *= r;
            acc *= r;
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                // a split that saw nothing has lse_c = -inf and an all-zero partial row
                const float wc = __builtin_amdgcn_exp2f((l[c] - cm) * kLog2e);
                sum += wc;
                acc += wc * v[c];
            }
            m = cm;
        }
    }
    float lse = 0.f;
    if constexpr (SOFTMAX) {
        if (m == -INFINITY) {
            lse = -INFINITY;  // acc stayed 0
        } else {
            acc *= __builtin_amdgcn_rcpf(sum);
            lse = m + __builtin_amdgcn_logf(sum) * kLn2;  // v_log_f32 is log2
        }
    }
    const int64_t grow = rh / p.H;
    const int h = (int)(rh % p.H);
    uint16_t *op = (uint16_t *)p.o + grow * p.o_stride + h * D + chunk * 4;
    *(u32x2_t *)op = u32x2_t{E::pack2(acc[0], acc[1]), E::pack2(acc[2], acc[3])};
    if constexpr (SOFTMAX) {
        if (p.lse != nullptr && chunk == 0) {
            int64_t li;
            if (p.jagged) {
                li = (int64_t)h * p.total_rows + grow;
            } else {
                const int64_t b = grow / p.seqlen_q, i = grow % p.seqlen_q;
                li = (b * p.H + h) * p.seqlen_q + i;
            }
            p.lse[li] = lse;
        }
    }
}

// Combine pass of the cut (heavy) q-tiles: kHeavyCombineBlocks work-groups per
// q-tile, each over a run of its rows; a q-tile that was not cut (chunk count < 2)
// or lies past its sequence is skipped.  A thread takes 4 columns of a row, loads
// every chunk's partial (and LSE) before using any, and adds them in chunk order
// (SiLU: a sum; softmax: weights exp(lse_c - lse) as in the split-KV combine),
// then writes o (and the LSE).
constexpr int kHeavyCombineBlocks = 8;
template <int DT, bool SOFTMAX, int BM>
__global__ __launch_bounds__(256) void hstu_heavy_combine_kernel(KernelParams p, int D) {
    using E = Elem<DT>;
    const int64_t hq = blockIdx.x / kHeavyCombineBlocks;  // (b, h) and level
    const int part = blockIdx.x % kHeavyCombineBlocks;
    const int64_t bh = hq / p.heavy;
    if (bh >= (int64_t)p.B * p.H) return;
    const int32_t meta = p.hmeta[2 * hq], tok0 = p.hmeta[2 * hq + 1];
    const int nsp = meta & 255, rows = meta >> 8;
    if (nsp < 2) return;
    const int h = (int)(bh % p.H);
    const int nchunk = D / 4;
    constexpr int RPB = BM / kHeavyCombineBlocks;  // rows of this work-group
    const int64_t slot0 = hq * p.num_splits;
    for (int idx = threadIdx.x; idx < RPB * nchunk; idx += 256) {
        const int row = part * RPB + idx / nchunk, c4 = idx % nchunk;
        if (row >= rows) break;
        f32x4_t v[kHeavyMaxSplits];
        float l[kHeavyMaxSplits];
#pragma unroll
        for (int c = 0; c < kHeavyMaxSplits; ++c) {
            const bool in = c < nsp;
            const int64_t prow = (slot0 + c) * BM + row;
            v[c] = in ? *(const f32x4_t *)(p.hpart_o + prow * D + c4 * 4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
            if constexpr (SOFTMAX) l[c] = in ? p.hpart_lse[prow] : -INFINITY;
        }
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        float lse = 0.f;
        if constexpr (!SOFTMAX) {
#pragma unroll
            for (int c = 0; c < kHeavyMaxSplits; ++c) acc += v[c];
        } else {
            float m = -INFINITY;
#pragma unroll
            for (int c = 0; c < kHeavyMaxSplits; ++c) m = fmaxf(m, l[c]);
            if (m == -INFINITY) {
                lse = -INFINITY;  // no chunk saw a key: o = 0
            } else {
                float sum = 0.f;
#pragma unroll
                for (int c = 0; c < kHeavyMaxSplits; ++c) {
                    const float wc = __builtin_amdgcn_exp2f((l[c] - m) * kLog2e);  // 0 for absent chunks
                    sum += wc;
                    acc += wc * v[c];
                }
                acc *= __builtin_amdgcn_rcpf(sum);
                lse = m + __builtin_amdgcn_logf(sum) * kLn2;
            }
        }
        const int64_t grow = (int64_t)tok0 + row;
        uint16_t *op = (uint16_t *)p.o + grow * p.o_stride + h * D + c4 * 4;
        *(u32x2_t *)op = u32x2_t{E::pack2(acc[0], acc[1]), E::pack2(acc[2], acc[3])};
        if constexpr (SOFTMAX) {
            if (p.lse != nullptr && c4 == 0) {
                int64_t li;
                if (p.jagged) {
                    li = (int64_t)h * p.total_rows + grow;
                } else {
                    const int64_t b = grow / p.seqlen_q, i = grow % p.seqlen_q;
                    li = (b * p.H + h) * p.seqlen_q + i;
                }
                p.lse[li] = lse;
            }
        }
    }
}

// Visible pairs inside the scheduled key tiles, counted with the forward
// kernel's own plan, lane -> (row, key) assignment and tile classes: a tile the
// work-group-level test (BlockPlan::tile_full, which sends a tile through the
// unmasked pipelined body) calls full counts BN keys for every valid row; a tile
// a wave's rows classify as FULL (tile_state, the generic body's unmasked path)
// counts BN keys per row; otherwise the predicate decides per key.  A tile the
// work-group test calls full although one of its valid rows does not see all of
// it adds 2^40, so that a wrong classification can never go unnoticed by an exact
// comparison with an independently computed count of the mask's visible pairs.
template <int BN, int NW>
__global__ __launch_bounds__(64 * NW) void hstu_count_kernel(KernelParams p, unsigned long long *count) {
    BlockPlan bp;
    if (!plan_block<BN, NW>(p, false, bp, decode_work(p, blockIdx.x))) return;
    const int lane = threadIdx.x & 63, g = lane >> 5;
    unsigned long long mine = 0;
    const int ntiles = bp.tiles.count();
    for (int n = 0; n < ntiles; ++n) {
        const int j0 = bp.tiles.at(n) * BN;
        const int32_t st = tile_state(bp.span, j0, j0 + BN);
        if (bp.tile_full(j0, BN)) {
            if (bp.span.valid) mine += st == kTileFull ? BN / 2 : (1ull << 40);
            continue;
        }
        const bool wave_any = __ballot(st != kTileEmpty) != 0;
        const bool wave_mask = __ballot(bp.span.valid && st != kTileFull) != 0;
        if (!wave_any || !bp.span.valid) continue;
        if (!wave_mask) {
            mine += BN / 2;
            continue;
        }
        for (int kb = 0; kb < BN / 32; ++kb)
            for (int i = 0; i < 16; ++i)
                mine += span_visible(bp.span, j0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3)) ? 1 : 0;
    }
    for (int o = 32; o >= 1; o >>= 1) mine += __shfl_xor(mine, o);
    if (lane == 0 && mine) atomicAdd(count, mine);
}

__global__ void hstu_zero_u64(unsigned long long *x) { *x = 0; }

// Planning kernel of the persistent schedule: work-group x writes XCD x's queue.
// The queue holds the existing q-tiles of the XCD's (b, h) pairs (bh = x + 8k),
// the pairs ordered from the most expensive sequence to the cheapest (cost:
// q-tiles x keys; ties by k; at most kPlanSortPairs pairs are sorted, beyond
// that they keep their order), each pair's q-tiles heaviest first and, per
// q-tile, its splits.  Running the longest pairs first keeps their long q-tiles
// out of the kernel's tail; listing only existing q-tiles spares the item loop
// the empty ones.  It also clears the take counter.  (A kernel, not a memset,
// so that the launch sequence can be captured into a graph and replayed.)
constexpr int kPlanThreads = 64;  // one wave: the barriers cost next to nothing
constexpr int kPlanSortPairs = 2048;
template <int BM>
__global__ __launch_bounds__(kPlanThreads) void hstu_plan_kernel(KernelParams p) {
    __shared__ float key[kPlanSortPairs];
    __shared__ int32_t order[kPlanSortPairs];
    __shared__ int32_t nq_of[kPlanSortPairs];  // q-tiles of pair k (sorted queues)
    __shared__ int32_t scan[kPlanThreads];
    const int x = blockIdx.x, t = threadIdx.x;
    const int K = p.bh_pad / 8;
    const uint32_t per_queue = (uint32_t)(grid_size(p) / 8);
    gmem_t<uint64_t> *list = (gmem_t<uint64_t> *)((uint8_t *)p.queue + kQueueHeader) + (size_t)x * per_queue;
    // q-tiles and cost of pair k of this queue
    auto pair = [&](int k, int &nq, float &cost) {
        const int bh = x + 8 * k;
        nq = 0;
        cost = -0.5f;
        if (bh >= p.B * p.H) return;
        const int b = bh / p.H;
        int S_q = p.seqlen_q, S_kv = p.seqlen_kv;
        if (p.jagged) {
            S_q = p.off_q[b + 1] - p.off_q[b];
            S_kv = p.cross ? p.off_kv[b + 1] - p.off_kv[b] : S_q;
        }
        nq = imin((S_q + BM - 1) / BM, p.num_qt);
        cost = (float)nq * (float)S_kv;
    };
    if (K <= kPlanThreads) {
        // one pair per lane: its position in the order is the number of pairs
        // before it, and its first entry the items of those pairs
        int nq = 0;
        float c = -1.0f;
        if (t < K) pair(t, nq, c);
        const int items = nq * p.num_splits;
        int e = 0, total = 0;
        for (int j = 0; j < K; ++j) {
            const float cj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c), j));
            const int ij = __builtin_amdgcn_readlane(items, j);
            e += (cj > c || (cj == c && j < t)) ? ij : 0;
            total += ij;
        }
        const int bh = x + 8 * t;
        for (int qt = nq - 1; qt >= 0; --qt)
            for (int sp = 0; sp < p.num_splits; ++sp)
                list[e++] = (uint64_t)(uint32_t)bh | (uint64_t)(uint32_t)(qt << 8 | sp) << 32;
        for (uint32_t i = (uint32_t)total + t; i < per_queue; i += kPlanThreads) list[i] = 0xffffffffu;
        if (t == 0) {
            p.queue[x] = 0;
            p.queue[kQueueCount + x] = (uint32_t)total;
        }
        return;
    }
    const bool sorted = K <= kPlanSortPairs;
    if (sorted) {
        int n = 1;
        while (n < K) n <<= 1;
        for (int i = t; i < n; i += kPlanThreads) {
            int nq = 0;
            float c = -1.0f;  // padding entries sort last
            if (i < K) pair(i, nq, c);
            key[i] = c;
            order[i] = i;
            nq_of[i] = nq;
        }
        __syncthreads();
        // bitonic sort into "a before b": larger cost first, then smaller k
        for (int size = 2; size <= n; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = t; i < n; i += kPlanThreads) {
                    const int j = i ^ stride;
                    if (j > i) {
                        const bool i_first = key[i] > key[j] || (key[i] == key[j] && order[i] < order[j]);
                        if (((i & size) == 0) != i_first) {
                            const float kt = key[i];
                            key[i] = key[j];
                            key[j] = kt;
                            const int ot = order[i];
                            order[i] = order[j];
                            order[j] = ot;
                        }
                    }
                }
                __syncthreads();
            }
        }
    }
    // in order, kPlanThreads pairs at a time: inclusive scan of their item
    // counts, then each thread writes its pair's items
    int carry = 0;
    for (int r0 = 0; r0 < K; r0 += kPlanThreads) {
        const int r = r0 + t;
        int k = 0, nq = 0;
        if (r < K) {
            k = sorted ? order[r] : r;
            float c;
            if (sorted)
                nq = nq_of[k];
            else
                pair(k, nq, c);
        }
        const int bh = x + 8 * k;
        const int items = nq * p.num_splits;
        scan[t] = items;
        __syncthreads();
        for (int o = 1; o < kPlanThreads; o <<= 1) {
            const int v = t >= o ? scan[t - o] : 0;
            __syncthreads();
            scan[t] += v;
            __syncthreads();
        }
        int e = carry + scan[t] - items;
        for (int qt = nq - 1; qt >= 0; --qt)
            for (int sp = 0; sp < p.num_splits; ++sp)
                list[e++] = (uint64_t)(uint32_t)bh | (uint64_t)(uint32_t)(qt << 8 | sp) << 32;
        carry += scan[kPlanThreads - 1];
        __syncthreads();
    }
    // the rest of the queue: "no item" (bh = -1)
    for (uint32_t i = (uint32_t)carry + t; i < per_queue; i += kPlanThreads) list[i] = 0xffffffffu;
    if (t == 0) {
        p.queue[x] = 0;
        p.queue[kQueueCount + x] = (uint32_t)carry;
    }
}

// ------------------------------------------------------------------ launchers

// Static scratch of the allocation-free entry point: split-KV partials and the
// persistent schedule's work queues of one call, in a file-scope device array
// that every GPU the library runs on holds (at its own address) until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in): the address comes from hipGetSymbolAddress, once
// per device with that device current, and is kept per device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_region(void **ptr) {
    static std::mutex mu;
    static void *addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}


// compute units of the current device (cached per device)
static int current_device_cus() {
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

// Work-groups of kernel K resident per CU (cached per kernel; the kernels'
// resources do not depend on the device among gfx950 parts).
template <void (*K)(KernelParams)>
static int resident_per_cu(int threads) {
    static std::atomic<int> cache{0};
    int n = cache.load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, K, threads, 0) != hipSuccess || n < 1) n = 1;
        cache.store(n, std::memory_order_relaxed);
    }
    return n;
}

template <void (*K)(KernelParams), int D>
static hipError_t launch_items(const KernelParams &p, int threads, hipStream_t stream) {
    const int64_t items = grid_size(p);
    if (items <= 0) return hipSuccess;
    int64_t grid = items;
    if (p.queue != nullptr) {
        // persistent: as many work-groups as are resident at once (a multiple of
        // the 8 XCDs), never more than there are items
        const int64_t slots = (int64_t)current_device_cus() * resident_per_cu<K>(threads);
        grid = slots >= 8 ? (slots / 8) * 8 : 8;
        if (grid > items) grid = items;
        hipLaunchKernelGGL((hstu_plan_kernel<block_m_for(D)>), dim3(8), dim3(kPlanThreads), 0, stream, p);
    }
    hipLaunchKernelGGL(K, dim3((unsigned)grid), dim3(threads), 0, stream, p);
    return hipGetLastError();
}

template <int DT, int D, int DV, bool SOFTMAX, bool SPLIT>
static hipError_t launch_one(const KernelParams &p, hipStream_t stream) {
    constexpr int threads = 64 * waves_for(D);
    if (p.rab_pos != nullptr || p.rab_ts != nullptr)
        return launch_items<hstu_fwd_kernel<DT, D, SOFTMAX, SPLIT, DV, true>, D>(p, threads, stream);
    return launch_items<hstu_fwd_kernel<DT, D, SOFTMAX, SPLIT, DV, false>, D>(p, threads, stream);
}

template <int DT, int D, int DV>
static hipError_t launch_d(const KernelParams &p, bool softmax, bool split, hipStream_t stream) {
    if (softmax)
        return split ? launch_one<DT, D, DV, true, true>(p, stream) : launch_one<DT, D, DV, true, false>(p, stream);
    return split ? launch_one<DT, D, DV, false, true>(p, stream) : launch_one<DT, D, DV, false, false>(p, stream);
}

template <int DT>
static hipError_t launch_dt(const KernelParams &p, int D, int DV, bool softmax, bool split, hipStream_t stream) {
    if (D == 64 && DV == 64) return launch_d<DT, 64, 64>(p, softmax, split, stream);
    if (D == 96 && DV == 96) return launch_d<DT, 96, 96>(p, softmax, split, stream);
    if (D == 96 && DV == 64) return launch_d<DT, 96, 64>(p, softmax, split, stream);
    if (D == 128 && DV == 128) return launch_d<DT, 128, 128>(p, softmax, split, stream);
    if (D == 256 && DV == 256) return launch_d<DT, 256, 256>(p, softmax, split, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_forward(const KernelParams &p, int dtype, int D, int DV, bool softmax, bool split,
                          hipStream_t stream) {
    return dtype == HSTU_BF16 ? launch_dt<HSTU_BF16>(p, D, DV, softmax, split, stream)
                              : launch_dt<HSTU_FP16>(p, D, DV, softmax, split, stream);
}

hipError_t launch_combine(const KernelParams &p, int dtype, int D, bool softmax, hipStream_t stream) {
    const int64_t total = (int64_t)p.total_rows * p.H * (D / 4);
    if (total <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (dtype == HSTU_BF16) {
        if (softmax)
            hipLaunchKernelGGL((hstu_combine_kernel<HSTU_BF16, true>), dim3(blocks), dim3(256), 0, stream, p, D);
        else
            hipLaunchKernelGGL((hstu_combine_kernel<HSTU_BF16, false>), dim3(blocks), dim3(256), 0, stream, p, D);
    } else {
        if (softmax)
            hipLaunchKernelGGL((hstu_combine_kernel<HSTU_FP16, true>), dim3(blocks), dim3(256), 0, stream, p, D);
        else
            hipLaunchKernelGGL((hstu_combine_kernel<HSTU_FP16, false>), dim3(blocks), dim3(256), 0, stream, p, D);
    }
    return hipGetLastError();
}

hipError_t launch_heavy_combine(const KernelParams &p, int dtype, int D, int DV, bool softmax, hipStream_t stream) {
    const int64_t blocks = (int64_t)p.bh_pad * p.heavy * kHeavyCombineBlocks;
    if (blocks <= 0) return hipSuccess;
    const int bm = block_m_for(D);
    if (bm != 128) return hipErrorInvalidValue;
    if (dtype == HSTU_BF16) {
        if (softmax)
            hipLaunchKernelGGL((hstu_heavy_combine_kernel<HSTU_BF16, true, 128>), dim3((unsigned)blocks), dim3(256), 0, stream, p, DV);
        else
            hipLaunchKernelGGL((hstu_heavy_combine_kernel<HSTU_BF16, false, 128>), dim3((unsigned)blocks), dim3(256), 0, stream, p, DV);
    } else {
        if (softmax)
            hipLaunchKernelGGL((hstu_heavy_combine_kernel<HSTU_FP16, true, 128>), dim3((unsigned)blocks), dim3(256), 0, stream, p, DV);
        else
            hipLaunchKernelGGL((hstu_heavy_combine_kernel<HSTU_FP16, false, 128>), dim3((unsigned)blocks), dim3(256), 0, stream, p, DV);
    }
    return hipGetLastError();
}

hipError_t launch_count(const KernelParams &p, int D, unsigned long long *count, hipStream_t stream) {
    hipLaunchKernelGGL(hstu_zero_u64, dim3(1), dim3(1), 0, stream, count);
    const int64_t grid = grid_size(p);
    if (grid > 0) {
        switch (D) {
            case 64: hipLaunchKernelGGL((hstu_count_kernel<key_tile_for(64), waves_for(64)>), dim3((unsigned)grid), dim3(64 * waves_for(64)), 0, stream, p, count); break;
            case 96: hipLaunchKernelGGL((hstu_count_kernel<key_tile_for(96), waves_for(96)>), dim3((unsigned)grid), dim3(64 * waves_for(96)), 0, stream, p, count); break;
            case 128: hipLaunchKernelGGL((hstu_count_kernel<key_tile_for(128), waves_for(128)>), dim3((unsigned)grid), dim3(64 * waves_for(128)), 0, stream, p, count); break;
            case 256: hipLaunchKernelGGL((hstu_count_kernel<key_tile_for(256), waves_for(256)>), dim3((unsigned)grid), dim3(64 * waves_for(256)), 0, stream, p, count); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

}  // namespace hstu

// hstu_plan.h - per-sequence geometry, per-row visible key intervals, key-tile
// classification and work decoding of the HSTU forward kernels.
//
// The functional mask (CK example README "18_hstu_attention", "Masking" table) is
// evaluated here in interval form: every query row i of a sequence sees the keys
//     [0, ctx)  U  [lo, hi]          (physical key indices; lo > hi: empty)
// where [0, ctx) is the context prefix (visible to all queries) and [lo, hi] the
// band of UIH keys its causal / local-window / min-full components leave visible.
// Target keys lie beyond every hi, so they are never attended.  Nothing here
// depends on HIP; host and device code include it.
#pragma once

#include <stdint.h>

#include "hstu_params.h"

#if defined(__HIPCC__)
#define HSTU_HD __host__ __device__ __forceinline__
#else
#define HSTU_HD inline
#endif

namespace hstu {

constexpr int32_t kEmptyLo = 0x3fffffff;
constexpr int32_t kEmptyHi = -0x3fffffff;

HSTU_HD int32_t imin(int32_t a, int32_t b) { return a < b ? a : b; }
HSTU_HD int32_t imax(int32_t a, int32_t b) { return a > b ? a : b; }

// Class boundaries of one sequence (README "Masking": physical lengths are
// context + UIH + targets; cross-attention keys carry no targets).
struct SeqGeom {
    int64_t q0, kv0;   // first token in q/o and in k/v
    int32_t S_q, S_kv; // physical lengths
    int32_t Cq, Uq;    // query-side context and UIH counts (targets follow)
    int32_t Ck, Ukv;   // key-side context and UIH counts
    int32_t L, M;      // local_len, minfull_len
    int32_t group;
    float attn_scale;
};

HSTU_HD SeqGeom seq_geom(const KernelParams &p, int32_t b) {
    SeqGeom s;
    s.group = b / p.per_group;
    const GroupDev &g = p.groups[s.group];
    // every load of the sequence's metadata is issued before any of the values
    // is used, so that on the device they cost one memory round trip, not three
    int32_t q_lo = 0, q_hi = 0, kv_lo = 0, kv_hi = 0, T = 0;
    if (p.jagged) {
        // (without targets the count is read from the offsets and discarded)
        const int32_t *ko = p.cross ? p.off_kv : p.off_q;
        const int32_t *tp = p.num_targets ? p.num_targets : p.off_q;
        q_lo = p.off_q[b];
        q_hi = p.off_q[b + 1];
        kv_lo = ko[b];
        kv_hi = ko[b + 1];
        const int32_t t_raw = tp[b];
        T = p.num_targets ? t_raw : 0;
    } else if (p.num_targets) {
        T = p.num_targets[b];
    }
    if (p.jagged) {
        s.q0 = q_lo;
        s.S_q = q_hi - q_lo;
        s.kv0 = kv_lo;
        s.S_kv = kv_hi - kv_lo;
    } else {
        s.q0 = (int64_t)b * p.seqlen_q;
        s.kv0 = (int64_t)b * p.seqlen_kv;
        s.S_q = p.seqlen_q;
        s.S_kv = p.seqlen_kv;
    }
    T = imax(T, 0);
    s.Cq = imin(g.context_len, s.S_q);
    const int32_t Tq = imin(T, s.S_q - s.Cq);
    s.Uq = s.S_q - s.Cq - Tq;
    s.Ck = imin(g.context_len, s.S_kv);
    const int32_t Tk = p.cross ? 0 : imin(T, s.S_kv - s.Ck);
    s.Ukv = s.S_kv - s.Ck - Tk;
    s.L = g.local_len;
    s.M = g.minfull_len;
    s.attn_scale = g.attn_scale;
    return s;
}

// Visible keys of query row i: [0, ctx) U [lo, hi].  Rows outside the
// sequence see nothing (ctx = 0, empty band).
struct RowSpan {
    int32_t ctx, lo, hi;
    bool valid;
};

HSTU_HD RowSpan row_span(const SeqGeom &s, int32_t causal, int32_t i) {
    RowSpan r;
    r.lo = kEmptyLo;
    r.hi = kEmptyHi;
    r.valid = (i >= 0 && i < s.S_q);
    if (!r.valid) {
        r.ctx = 0;
        return r;
    }
    r.ctx = s.Ck;
    int32_t x;
    bool full;
    if (i < s.Cq) {                   // context query: before every UIH key
        if (causal) return r;
        x = -1;
        full = (s.L == 0);
    } else if (i < s.Cq + s.Uq) {     // UIH query at UIH position u
        const int32_t u = i - s.Cq;
        x = u + (s.Ukv - s.Uq);       // aligned to the tail of the key history
        full = (s.L == 0) || (s.M > 0 && u >= s.Uq - s.M);
    } else {                          // target query: after the whole history
        x = s.Ukv;
        full = (s.L == 0) || (s.M > 0);
    }
    const int32_t last = s.Ukv - 1;
    const int32_t hi = causal ? imin(x, last) : (full ? last : imin(x + s.L, last));
    const int32_t lo = full ? 0 : imax(0, x - s.L);
    if (lo <= hi) {
        r.lo = s.Ck + lo;
        r.hi = s.Ck + hi;
    }
    return r;
}

HSTU_HD bool span_visible(const RowSpan &r, int32_t j) {
    return j < r.ctx || (j >= r.lo && j <= r.hi);
}

// Relation of a row to the key tile [j0, j1): nothing visible, everything
// visible, or a mix (the predicate must then be applied per key).  A row
// outside the sequence is EMPTY.
enum TileState : int32_t { kTileEmpty = 0, kTilePartial = 1, kTileFull = 2 };

HSTU_HD int32_t tile_state(const RowSpan &r, int32_t j0, int32_t j1) {
    if (!r.valid) return kTileEmpty;
    const bool any = (j0 < r.ctx) || (r.lo <= r.hi && r.lo < j1 && r.hi >= j0);
    if (!any) return kTileEmpty;
    if (j1 <= r.ctx) return kTileFull;
    const bool all = r.lo <= imax(j0, r.ctx) && j1 - 1 <= r.hi;
    return all ? kTileFull : kTilePartial;
}

// A work-group's rows taken together (reduced over its rows in any order):
//   lo, hi          the union of their bands (min lo, max hi; a row past the
//                   sequence has an empty band and widens nothing);
//   full_lo, full_hi the intersection of the bands of its valid rows (max lo,
//                   min hi; rows past the sequence do not constrain it), empty
//                   (full_lo > full_hi) when some valid row's band is empty.
struct BlockBand {
    int32_t lo, hi, full_lo, full_hi;
};

HSTU_HD BlockBand block_band_init() { return BlockBand{kEmptyLo, kEmptyHi, kEmptyHi, kEmptyLo}; }

// The four terms one row contributes (combined with min, max, max, min).
HSTU_HD BlockBand row_band(const RowSpan &r) {
    return BlockBand{r.lo, r.hi, r.valid ? r.lo : kEmptyHi, r.valid ? r.hi : kEmptyLo};
}

HSTU_HD BlockBand block_band_join(const BlockBand &a, const BlockBand &b) {
    return BlockBand{imin(a.lo, b.lo), imax(a.hi, b.hi), imax(a.full_lo, b.full_lo), imin(a.full_hi, b.full_hi)};
}

// The BlockBand of rows [r0, r1] of a sequence (rows past the sequence count as
// rows without a band that constrain nothing) without visiting every row.  The
// rows fall into four regions: context, UIH rows before the min-full tail, the
// min-full tail, targets.  Inside a region the row's x (its position against the
// key history) is constant or grows with the row, and lo and hi are
// non-decreasing in x; the rows whose band is empty are those with x below a
// threshold (causal: x < 0; otherwise, outside full rows: x < -local_len), so a
// prefix of the region.  Hence a region's rows contribute exactly what its first
// row, its first row with a band and its last row contribute: the union is the
// first non-empty row's lo and the last row's hi, and the intersection is empty
// when the first row's band is, else [last row's lo, first row's hi].  Equal to
// joining row_band over every row of the range.
HSTU_HD BlockBand qtile_band(const SeqGeom &s, int32_t causal, int32_t r0, int32_t r1) {
    BlockBand u = block_band_init();
    r0 = imax(r0, 0);
    r1 = imin(r1, s.S_q - 1);
    if (r0 > r1) return u;
    const int32_t uih0 = s.Cq, tgt0 = s.Cq + s.Uq;
    const int32_t tail0 = s.M > 0 ? imax(uih0, tgt0 - s.M) : tgt0;  // first min-full row
    const int32_t start[5] = {0, uih0, tail0, tgt0, s.S_q};
    for (int k = 0; k < 4; ++k) {
        const int32_t a = imax(r0, start[k]), b = imin(r1, start[k + 1] - 1);
        if (a > b) continue;
        u = block_band_join(u, row_band(row_span(s, causal, a)));
        u = block_band_join(u, row_band(row_span(s, causal, b)));
        if (k == 1 || k == 2) {
            // UIH rows: x = row - Cq + Ukv - Uq; the first row with a band has
            // x >= 0 (causal) or x >= -L (non-causal rows that are not full)
            const bool full = s.L == 0 || k == 2;
            if (causal || !full) {
                const int32_t x_min = causal ? 0 : -s.L;
                const int32_t first = imax(a, x_min + s.Cq + s.Uq - s.Ukv);
                if (first > a && first <= b) u = block_band_join(u, row_band(row_span(s, causal, first)));
            }
        }
    }
    return u;
}

// Key tile [j0, j0 + BN) is visible to every valid row of the work-group: it lies
// in the context prefix [0, ctx), or its part past the prefix lies inside every
// valid row's band.  (A work-group with no valid row has full_lo > full_hi.)
HSTU_HD bool block_tile_full(const BlockBand &bb, int32_t ctx, int32_t j0, int32_t BN) {
    const int32_t j1 = j0 + BN;
    return j1 <= ctx || (bb.full_lo <= imax(j0, ctx) && j1 - 1 <= bb.full_hi);
}

// The 32 keys one lane scores in a 64-key tile: element e (0..31) is key
// jb + 8 (e / 4) + e % 4 (four consecutive keys of every eight).  Bit e of
// lane_key_mask is set when the row sees that key.  The element offsets grow
// with e, so the keys below u are the first cnt(u) = 4 (u / 8) + min(u % 8, 4)
// elements (u clamped to 0..64): each of the row's two intervals is a run of
// consecutive bits.
HSTU_HD uint32_t lane_prefix_bits(int32_t u) {
    u = imin(imax(u, 0), 64);
    const int32_t n = 4 * (u >> 3) + imin(u & 7, 4);  // 0..32
    return n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
}
HSTU_HD uint32_t lane_key_mask(const RowSpan &r, int32_t jb) {
    const uint32_t ctx = lane_prefix_bits(r.ctx - jb);
    if (r.lo > r.hi) return ctx;
    return ctx | (lane_prefix_bits(r.hi + 1 - jb) & ~lane_prefix_bits(r.lo - jb));
}

// Key tiles a q-tile needs: the context tiles [0, ceil(ctx/BN)) and the band
// tiles covering [band_lo, band_hi] (the union of its rows' bands), merged when
// they touch, then intersected with the split's tile range [t_begin, t_end).
struct TileList {
    int32_t a0, a1; // first range [a0, a1)
    int32_t b0, b1; // second range [b0, b1)
    HSTU_HD int32_t count() const { return (a1 - a0) + (b1 - b0); }
    HSTU_HD int32_t at(int32_t n) const { return n < a1 - a0 ? a0 + n : b0 + (n - (a1 - a0)); }
    // the tiles at positions [nb, ne) (0 <= nb <= ne <= count()), as a list
    HSTU_HD TileList sub(int32_t nb, int32_t ne) const {
        const int32_t na = a1 - a0;
        TileList t;
        t.a0 = a0 + imin(nb, na);
        t.a1 = a0 + imin(ne, na);
        t.b0 = b0 + imax(nb - na, 0);
        t.b1 = b0 + imax(ne - na, 0);
        return t;
    }
};

HSTU_HD TileList make_tile_list(int32_t ctx, bool any_valid_row, int32_t band_lo, int32_t band_hi,
                                int32_t BN, int32_t t_begin, int32_t t_end) {
    TileList t;
    int32_t ca = 0, cb = any_valid_row ? (ctx + BN - 1) / BN : 0;   // context tiles
    int32_t ba = 0, bb = 0;                                            // band tiles
    if (band_lo <= band_hi) {
        ba = band_lo / BN;
        bb = band_hi / BN + 1;
    }
    if (bb > ba && cb > ca && ba <= cb) {  // touching or overlapping: one range
        cb = imax(cb, bb);
        ba = bb = 0;
    }
    t.a0 = imax(ca, t_begin);
    t.a1 = imin(cb, t_end);
    if (t.a1 < t.a0) t.a1 = t.a0;
    t.b0 = imax(ba, t_begin);
    t.b1 = imin(bb, t_end);
    if (t.b1 < t.b0) t.b1 = t.b0;
    return t;
}

// Heavy q-tiles (per-item grid): the last kHeavyLevels q-tiles of a sequence,
// whose key-tile lists are long (they hold the min-full and target rows, which
// see the whole history, also when those rows straddle a q-tile boundary), are
// cut into up to kHeavyMaxSplits contiguous chunks of their lists, each processed
// by a work-group of its own, so that no single work-group walks the whole
// history.  A chunk holds at least chunk_tiles tiles (by default 256 keys'
// worth); a list of at most that many is not cut.
constexpr int32_t kHeavyMaxSplits = 4;
constexpr int32_t kHeavyLevels = 2;
HSTU_HD int32_t heavy_chunk_tiles(int32_t BN) { return BN >= 256 ? 1 : 256 / BN; }
HSTU_HD int32_t heavy_splits(int32_t ntiles, int32_t chunk_tiles, int32_t max_splits) {
    if (ntiles <= chunk_tiles) return 1;
    return imin(max_splits, (ntiles + chunk_tiles - 1) / chunk_tiles);
}
// Positions [n_begin, n_end) of chunk sp of a list of ntiles tiles cut into nsp
// chunks whose sizes differ by at most one (earlier chunks the larger).
HSTU_HD void heavy_chunk(int32_t ntiles, int32_t nsp, int32_t sp, int32_t *n_begin, int32_t *n_end) {
    const int32_t q = ntiles / nsp, r = ntiles % nsp;
    *n_begin = sp * q + imin(sp, r);
    *n_end = *n_begin + q + (sp < r ? 1 : 0);
}

// Tiles [t_begin, t_end) of split sp: the sequence's key tiles cut into
// num_splits contiguous chunks of ceil(ntiles / num_splits) tiles.
HSTU_HD void split_range(int32_t S_kv, int32_t BN, int32_t num_splits, int32_t sp, int32_t *t_begin,
                         int32_t *t_end) {
    const int32_t nt = (S_kv + BN - 1) / BN;
    const int32_t per = (nt + num_splits - 1) / num_splits;
    *t_begin = imin(sp * per, nt);
    *t_end = imin((sp + 1) * per, nt);
}

// Work item of a work-group: (sequence b, head h, q-tile qt, split sp).
struct WorkItem {
    int32_t b, h, qt, sp;
    bool valid;
};

// Schedules (the hardware hands consecutive work-group ids to the 8 XCDs in
// turn, so id % 8 is the XCD; both orders keep every (b, h) on one XCD):
//  1: q-tile levels, heaviest (last) q-tile of every (b, h) first;
//  2: per XCD, the (b, h) pairs one after another, each with all its q-tiles
//     heaviest first, so the q-tiles reading the same keys run together;
//  3: per XCD, the (b, h) pairs from the most expensive sequence to the
//     cheapest, each with its existing q-tiles heaviest first, taken from
//     per-XCD queues by a persistent grid (the planning kernel writes the
//     queues; decode_work is not used).
HSTU_HD WorkItem decode_work(const KernelParams &p, int64_t w) {
    WorkItem it;
    int64_t bh, rest;
    if (p.levels) {
        // q-tile levels (qt holds the level; plan_block turns it into the q-tile
        // counted from the end of the sequence), then (b, h): the last q-tiles of
        // every sequence, the heaviest under a causal mask (the min-full and
        // target rows see the whole history), first.  heavy: the first p.heavy
        // levels come with num_splits chunk slots each (level, chunk, (b, h)),
        // the other levels with one; bh % 8 = w % 8 keeps each (b, h) on one XCD
        const int64_t per_hl = (int64_t)p.bh_pad * p.num_splits, hl = (int64_t)p.heavy * per_hl;
        if (w < hl) {
            it.qt = (int32_t)(w / per_hl);
            it.sp = (int32_t)((w % per_hl) / p.bh_pad);
        } else {
            it.qt = p.heavy + (int32_t)((w - hl) / p.bh_pad);
            it.sp = 0;
        }
        bh = w % p.bh_pad;
        it.b = (int32_t)(bh / p.H);
        it.h = (int32_t)(bh % p.H);
        it.valid = bh < (int64_t)p.B * p.H;
        return it;
    }
    if (p.schedule >= 2) {
        const int64_t xcd = w % 8, loc = w / 8;
        const int64_t per_bh = (int64_t)p.num_qt * p.num_splits;
        bh = (loc / per_bh) * 8 + xcd;
        rest = loc % per_bh;
    } else {
        bh = w % p.bh_pad;
        rest = w / p.bh_pad;
    }
    it.sp = (int32_t)(rest % p.num_splits);
    it.qt = p.num_qt - 1 - (int32_t)(rest / p.num_splits);
    it.b = (int32_t)(bh / p.H);
    it.h = (int32_t)(bh % p.H);
    it.valid = bh < (int64_t)p.B * p.H && it.qt >= 0;
    return it;
}

// Level l of a sequence with nq q-tiles (levels order): its q-tile counted from
// the end, nq - 1 - l; the levels past the sequence map one to one onto the
// q-tiles past its end (which hold no rows).  A bijection of [0, num_qt).
HSTU_HD int32_t level_qtile(int32_t l, int32_t nq) { return l < nq ? nq - 1 - l : l; }

HSTU_HD int64_t grid_size(const KernelParams &p) {
    // heavy: num_splits chunk slots for each of the first p.heavy levels
    if (p.heavy) return (int64_t)p.bh_pad * (p.num_qt + (int64_t)p.heavy * (p.num_splits - 1));
    return (int64_t)p.bh_pad * p.num_qt * p.num_splits;
}

// Workspace bytes of the persistent schedule's queues (header + one 8-byte entry
// per possible item).
HSTU_HD size_t queue_bytes(const KernelParams &p) {
    return kQueueHeader + 8 * (size_t)grid_size(p);
}

}  // namespace hstu

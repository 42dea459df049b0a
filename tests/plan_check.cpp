// plan_check.cpp - host build of the forward kernels' planner (hstu_plan.h),
// checked against dense masks read from stdin.  Test infrastructure: built by
// tests/test_plan_cpu.py with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer; the masks come from an independent evaluation of
// the mask rule (the rule form, row by row), never from this planner.
//
// Input, one case per two lines:
//   S_q S_kv C T cross L M causal
//   <S_q * S_kv characters '0' / '1': the dense mask, row-major>
// For every case and every (BM, BN) of kTiles it checks:
//   interval form   span_visible(row_span(i), j) == mask[i][j] for every (i, j);
//   tile list       the key tiles make_tile_list keeps for a q-tile cover every
//                   visible pair of its rows; a tile outside the list holds none;
//                   the list is increasing and inside [0, ceil(S_kv / BN));
//   row classes     tile_state EMPTY: no visible key of the row in the tile; FULL:
//                   every key of the tile exists and is visible; rows past the
//                   sequence are EMPTY;
//   closed form     qtile_band gives the q-tile's joined row bands (union and
//                   intersection) exactly;
//   work-group test block_tile_full (the pipelined body's unmasked tiles): every
//                   valid row of the q-tile sees every key of the tile;
//   lane masks      lane_key_mask (the pipelined body's masked tiles): bit e is
//                   set exactly when the row sees key jb + 8 (e / 4) + e % 4, for
//                   64-key tiles and both lane groups' first keys;
//   heavy chunks    heavy_splits / heavy_chunk / TileList::sub cut a q-tile's list
//                   into at most kHeavyMaxSplits non-empty runs of consecutive
//                   positions that concatenate to the list;
//   splits          split_range cuts [0, nt) into contiguous, disjoint ranges
//                   that cover it (1 .. 6 splits and 16), and the per-split tile
//                   lists concatenate to the unsplit list;
//   work order      decode_work gives each item of the grid exactly once, each
//                   (b, h) on one XCD, for schedules 1 and 2, level order and
//                   level order with chunk slots; levels map onto q-tiles one to
//                   one (once, before the cases);
//   pair count      counting as the device count kernel does (work-group test,
//                   then row classes, then the predicate) gives the mask's
//                   number of visible pairs.
// Prints "checked <cases> cases, <tiles> tiles" and exits 0, or prints the first
// failure and exits 1.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "hstu_plan.h"

using namespace hstu;

namespace {

struct TileCfg {
    int BM, BN;
};
// tiny tiles to exercise the tiling logic at sizes the sweep can enumerate, and
// the kernels' own (128 query rows; 128 keys at head dim 64, 64 above) and 32 keys
constexpr TileCfg kTiles[] = {{1, 1}, {2, 2}, {3, 2}, {4, 3}, {5, 8}, {8, 4}, {128, 128}, {128, 64}, {128, 32}};
constexpr int kSplits[] = {1, 2, 3, 4, 5, 6, 16};

long g_case = 0;
long g_tiles = 0;

[[noreturn]] void fail(const char *what, int a = -1, int b = -1, int c = -1) {
    std::printf("FAIL case %ld: %s (%d, %d, %d)\n", g_case, what, a, b, c);
    std::exit(1);
}

struct Case {
    int S_q, S_kv, C, T, cross, L, M, causal;
    std::vector<unsigned char> mask;  // [S_q][S_kv]
    bool vis(int i, int j) const { return mask[(size_t)i * S_kv + j] != 0; }
};

SeqGeom geom(const Case &c, int32_t *off_q, int32_t *off_kv, int32_t *targets, KernelParams &p) {
    std::memset(&p, 0, sizeof(p));
    off_q[0] = 0;
    off_q[1] = c.S_q;
    off_kv[0] = 0;
    off_kv[1] = c.S_kv;
    targets[0] = c.T;
    p.off_q = off_q;
    p.off_kv = off_kv;
    p.num_targets = targets;
    p.B = 1;
    p.H = 1;
    p.jagged = 1;
    p.cross = c.cross;
    p.causal = c.causal;
    p.G = 1;
    p.per_group = 1;
    p.groups[0].local_len = c.L;
    p.groups[0].context_len = c.C;
    p.groups[0].minfull_len = c.M;
    p.groups[0].attn_scale = 1.0f;
    return seq_geom(p, 0);
}

void check_case(const Case &c) {
    int32_t off_q[2], off_kv[2], targets[1];
    KernelParams p;
    const SeqGeom s = geom(c, off_q, off_kv, targets, p);
    if (s.S_q != c.S_q || s.S_kv != c.S_kv) fail("sequence lengths", s.S_q, s.S_kv);

    // interval form against the rule form
    long visible = 0;
    for (int i = -2; i < c.S_q + 2; ++i) {
        const RowSpan r = row_span(s, c.causal, i);
        if ((i >= 0 && i < c.S_q) != r.valid) fail("row validity", i);
        if (!r.valid) continue;
        for (int j = 0; j < c.S_kv; ++j) {
            if (span_visible(r, j) != c.vis(i, j)) fail("interval form differs from the mask", i, j);
            visible += c.vis(i, j);
        }
    }

    for (const TileCfg &tc : kTiles) {
        const int BM = tc.BM, BN = tc.BN;
        const int nt = (c.S_kv + BN - 1) / BN;
        long counted = 0;
        for (int r0 = 0; r0 < c.S_q; r0 += BM) {
            BlockBand band = block_band_init();
            std::vector<RowSpan> rows(BM);
            for (int k = 0; k < BM; ++k) {
                rows[k] = row_span(s, c.causal, r0 + k);
                band = block_band_join(band, row_band(rows[k]));
            }
            // closed form: the same four terms from at most twelve rows
            const BlockBand qb = qtile_band(s, c.causal, r0, r0 + BM - 1);
            if (qb.lo != band.lo || qb.hi != band.hi || qb.full_lo != band.full_lo || qb.full_hi != band.full_hi)
                fail("qtile_band differs from the rows' joined band", r0, BM, qb.lo - band.lo);
            const TileList tl = make_tile_list(s.Ck, true, band.lo, band.hi, BN, 0, nt);
            std::vector<char> in_list(nt > 0 ? nt : 1, 0);
            int prev = -1;
            for (int n = 0; n < tl.count(); ++n) {
                const int t = tl.at(n);
                if (t <= prev || t < 0 || t >= nt) fail("tile list not increasing or out of range", r0, t, n);
                prev = t;
                in_list[t] = 1;
            }
            for (int t = 0; t < nt; ++t) {
                const int j0 = t * BN, j1 = j0 + BN;
                ++g_tiles;
                const bool wg_full = block_tile_full(band, s.Ck, j0, BN);
                if (wg_full && !in_list[t]) fail("work-group-full tile not in the list", r0, t);
                for (int k = 0; k < BM; ++k) {
                    const int i = r0 + k;
                    const RowSpan &r = rows[k];
                    int nvis = 0;
                    if (r.valid)
                        for (int j = j0; j < j1 && j < c.S_kv; ++j) nvis += c.vis(i, j);
                    if (!in_list[t]) {
                        if (nvis) fail("a skipped tile holds visible pairs", i, t);
                        continue;
                    }
                    const int32_t st = tile_state(r, j0, j1);
                    if (!r.valid && st != kTileEmpty) fail("row past the sequence not EMPTY", i, t);
                    if (st == kTileEmpty && nvis) fail("EMPTY tile holds visible pairs", i, t);
                    if (st == kTileFull && (j1 > c.S_kv || nvis != BN)) fail("FULL tile not all visible", i, t, nvis);
                    if (wg_full && r.valid && (j1 > c.S_kv || nvis != BN))
                        fail("work-group-full tile not all visible to a valid row", i, t, nvis);
                    // the pipelined body's per-lane key masks (64-key tiles: lanes start
                    // at j0 and j0 + 4)
                    if (BN == 64)
                        for (int jb = j0; jb <= j0 + 4; jb += 4) {
                            const uint32_t m = lane_key_mask(r, jb);
                            for (int e = 0; e < 32; ++e) {
                                const int j = jb + 8 * (e / 4) + e % 4;
                                const bool v = r.valid && j < c.S_kv && c.vis(i, j);
                                if (((m >> e) & 1u) != (v ? 1u : 0u)) fail("lane key mask differs from the mask", i, j, jb);
                            }
                        }
                    // the device count kernel's rule
                    if (!r.valid) continue;
                    if (wg_full || st == kTileFull) {
                        counted += BN;
                    } else if (st == kTilePartial) {
                        for (int j = j0; j < j1; ++j) counted += span_visible(r, j) ? 1 : 0;
                    }
                }
            }
            // heavy q-tile chunks: sub-lists of consecutive positions that
            // concatenate to the list, at most kHeavyMaxSplits of them, none
            // empty, none cut from a list of at most chunk_tiles tiles
            for (int chunk_tiles : {1, 2, 3, 4, 8})
            for (int max_splits = 2; max_splits <= kHeavyMaxSplits; ++max_splits) {
                const int cnt = tl.count();
                const int nsp = heavy_splits(cnt, chunk_tiles, max_splits);
                if (nsp < 1 || nsp > max_splits || (nsp > 1 && cnt <= chunk_tiles))
                    fail("heavy split count", cnt, nsp, chunk_tiles);
                int expect = 0;
                for (int sp = 0; sp < nsp; ++sp) {
                    int32_t nb = -1, ne = -1;
                    heavy_chunk(cnt, nsp, sp, &nb, &ne);
                    if (nb != expect || ne < nb || ne > cnt || (cnt > 0 && ne == nb))
                        fail("heavy chunks do not partition the list", cnt, sp, nb);
                    const TileList sl = tl.sub(nb, ne);
                    if (sl.count() != ne - nb) fail("sub-list size", cnt, nb, ne);
                    for (int k = 0; k < sl.count(); ++k)
                        if (sl.at(k) != tl.at(nb + k)) fail("sub-list tile differs", cnt, nb + k, sl.at(k));
                    expect = ne;
                }
                if (expect != cnt) fail("heavy chunks do not reach the end of the list", cnt, expect);
            }
            // split-KV: contiguous ranges covering [0, nt); lists concatenate
            for (int ns : kSplits) {
                int expect_b = 0;
                std::vector<int> cat;
                for (int sp = 0; sp < ns; ++sp) {
                    int32_t tb = -7, te = -7;
                    split_range(c.S_kv, BN, ns, sp, &tb, &te);
                    if (tb != expect_b || te < tb || te > nt) fail("split ranges do not partition the tiles", ns, sp, tb);
                    expect_b = te;
                    const TileList st = make_tile_list(s.Ck, true, band.lo, band.hi, BN, tb, te);
                    for (int n = 0; n < st.count(); ++n) {
                        const int t = st.at(n);
                        if (t < tb || t >= te) fail("split list leaves its range", ns, sp, t);
                        cat.push_back(t);
                    }
                }
                if (expect_b != nt) fail("split ranges do not reach the last tile", ns, expect_b, nt);
                if ((int)cat.size() != tl.count()) fail("split lists do not concatenate to the list", ns);
                for (int n = 0; n < tl.count(); ++n)
                    if (cat[n] != tl.at(n)) fail("split lists do not concatenate to the list", ns, n);
            }
        }
        if (counted != visible) fail("pair count by tile classes differs from the mask's", BM, BN, (int)(counted - visible));
    }
}

// decode_work over a whole grid, for every per-item order: each item (b, h,
// q-tile, split) of the problem exactly once, each (b, h) on one XCD (id % 8) in
// the orders that promise it, and the levels mapping q-tiles one to one.
void check_decode() {
    KernelParams p;
    std::memset(&p, 0, sizeof(p));
    for (int B = 1; B <= 5; ++B)
        for (int H = 1; H <= 3; ++H)
            for (int num_qt = 1; num_qt <= 5; ++num_qt)
                for (int mode = 0; mode < 4; ++mode)
                    for (int S = 1; S <= 4; ++S) {
                        const int heavy = mode == 3 ? (num_qt < 2 ? num_qt : 2) : 0;
                        if ((mode >= 2 && mode < 3 && S > 1) || (mode == 3 && S < 2)) continue;
                        p.B = B;
                        p.H = H;
                        p.bh_pad = (B * H + 7) / 8 * 8;
                        p.num_qt = num_qt;
                        p.num_splits = S;
                        p.schedule = mode == 0 ? 1 : 2;
                        p.levels = mode >= 2;
                        p.heavy = heavy;
                        const int64_t grid = grid_size(p);
                        const int64_t expect = (int64_t)p.bh_pad * (heavy ? num_qt + heavy * (S - 1) : num_qt * S);
                        if (grid != expect) fail("grid size", mode, (int)grid, (int)expect);
                        // seen[bh][qt or level][sp]
                        std::vector<int> seen((size_t)B * H * num_qt * S, 0);
                        for (int64_t w = 0; w < grid; ++w) {
                            const WorkItem it = decode_work(p, w);
                            const int64_t bh = (int64_t)it.b * H + it.h;
                            if (!it.valid) {
                                if (bh < (int64_t)B * H && mode != 0 && it.qt >= 0) fail("valid item marked invalid", mode, (int)w);
                                continue;
                            }
                            if (bh < 0 || bh >= (int64_t)B * H || it.qt < 0 || it.qt >= num_qt || it.sp < 0 || it.sp >= S)
                                fail("decoded item out of range", mode, (int)w, it.qt);
                            if (mode >= 1 && bh % 8 != w % 8) fail("(b, h) off its XCD", mode, (int)w, (int)bh);
                            if (heavy && it.qt >= heavy && it.sp != 0) fail("chunk slot past the cut levels", (int)w, it.qt, it.sp);
                            ++seen[((size_t)bh * num_qt + it.qt) * S + it.sp];
                        }
                        for (int64_t bh = 0; bh < (int64_t)B * H; ++bh)
                            for (int q = 0; q < num_qt; ++q)
                                for (int sp = 0; sp < S; ++sp) {
                                    const int want = (mode == 2) ? (sp == 0) : (mode == 3 ? (q < heavy || sp == 0) : 1);
                                    if (seen[((size_t)bh * num_qt + q) * S + sp] != want)
                                        fail("item not decoded exactly once", mode, q, sp);
                                }
                    }
    // levels onto q-tiles: a bijection of [0, num_qt) for every sequence length
    for (int num_qt = 1; num_qt <= 9; ++num_qt)
        for (int nq = 0; nq <= num_qt; ++nq) {
            std::vector<int> hit(num_qt, 0);
            for (int l = 0; l < num_qt; ++l) {
                const int q = level_qtile(l, nq);
                if (q < 0 || q >= num_qt) fail("level maps outside the q-tiles", l, nq, q);
                ++hit[q];
                if (l < nq && q != nq - 1 - l) fail("level is not counted from the end", l, nq, q);
            }
            for (int q = 0; q < num_qt; ++q)
                if (hit[q] != 1) fail("levels do not map one to one", q, nq, num_qt);
        }
}

}  // namespace

int main() {
    check_decode();
    Case c;
    while (std::scanf("%d %d %d %d %d %d %d %d", &c.S_q, &c.S_kv, &c.C, &c.T, &c.cross, &c.L, &c.M, &c.causal) == 8) {
        if (c.S_q < 0 || c.S_kv < 0 || c.S_q > 100000 || c.S_kv > 100000) fail("bad header");
        c.mask.assign((size_t)c.S_q * c.S_kv, 0);
        std::string line;
        line.resize((size_t)c.S_q * c.S_kv + 1);
        if (c.S_q * c.S_kv > 0) {
            if (std::scanf("%s", &line[0]) != 1) fail("missing mask");
            for (size_t k = 0; k < c.mask.size(); ++k) {
                if (line[k] != '0' && line[k] != '1') fail("bad mask character", (int)k);
                c.mask[k] = line[k] == '1';
            }
        } else {
            char dash[8];
            if (std::scanf("%7s", dash) != 1) fail("missing empty-mask marker");
        }
        check_case(c);
        ++g_case;
    }
    std::printf("checked %ld cases, %ld tiles\n", g_case, g_tiles);
    return 0;
}

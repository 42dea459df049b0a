// hstu_api.cpp - the C ABI of include/hstu.h: argument validation, default
// resolution (CK example README argument table: alpha = 0 -> 1/sqrt(hdim_qk),
// attn_scale = 0 -> 1/max_seqlen of Q's UIH), workspace sizing and dispatch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "hstu.h"
#include "hstu_api_internal.h"
#include "hstu_launch.h"
#include "hstu_plan.h"

namespace {

thread_local char g_last_error[512] = "";

hstu_status_t fail(hstu_status_t st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int64_t rows_q(const hstu_fwd_args_t *a) {
    return a->jagged ? (int64_t)a->total_q : (int64_t)a->batch * a->seqlen_q;
}

hstu_status_t validate(const hstu_fwd_args_t *a) {
    g_last_error[0] = '\0';
    if (!a) return fail(HSTU_ERR_INVALID_ARG, "args is NULL");
    if (a->dtype != HSTU_FP16 && a->dtype != HSTU_BF16)
        return fail(HSTU_ERR_INVALID_ARG, "dtype %d is neither HSTU_FP16 nor HSTU_BF16", a->dtype);
    if (a->batch < 0) return fail(HSTU_ERR_INVALID_ARG, "batch %d < 0", a->batch);
    if (a->nhead < 1) return fail(HSTU_ERR_INVALID_ARG, "nhead %d < 1", a->nhead);
    if (a->hdim_qk <= 0 || a->hdim_v <= 0)
        return fail(HSTU_ERR_INVALID_ARG, "head dims must be positive (%d, %d)", a->hdim_qk, a->hdim_v);
    {
        const int dq = a->hdim_qk, dv = a->hdim_v;
        const bool built = (dq == dv && (dq == 64 || dq == 96 || dq == 128 || dq == 256)) || (dq == 96 && dv == 64);
        if (!built)
            return fail(HSTU_ERR_UNSUPPORTED,
                        "head dims (%d, %d): built for 64/64, 96/96, 96/64, 128/128, 256/256", dq, dv);
    }
    for (int32_t f : {a->jagged, a->cross, a->causal, a->softmax})
        if (f != 0 && f != 1) return fail(HSTU_ERR_INVALID_ARG, "jagged/cross/causal/softmax must be 0 or 1");
    if (a->schedule < 0 || a->schedule > 3)
        return fail(HSTU_ERR_INVALID_ARG, "schedule %d not in 0..3", a->schedule);
    if (a->seqlen_q < 0 || a->seqlen_kv < 0)
        return fail(HSTU_ERR_INVALID_ARG, "negative seqlen (%d, %d)", a->seqlen_q, a->seqlen_kv);
    if (!a->jagged && !a->cross && a->seqlen_kv != a->seqlen_q)
        return fail(HSTU_ERR_INVALID_ARG, "batched self-attention needs seqlen_kv == seqlen_q (%d != %d)",
                    a->seqlen_kv, a->seqlen_q);
    if (a->jagged) {
        if (a->batch > 0 && !a->seq_offsets_q)
            return fail(HSTU_ERR_INVALID_ARG, "jagged mode needs seq_offsets_q");
        if (a->cross && a->batch > 0 && !a->seq_offsets_kv)
            return fail(HSTU_ERR_INVALID_ARG, "jagged cross-attention needs seq_offsets_kv");
        if (!a->cross && a->seq_offsets_kv)
            return fail(HSTU_ERR_INVALID_ARG, "seq_offsets_kv is for cross-attention only");
        if (a->total_q < 0) return fail(HSTU_ERR_INVALID_ARG, "total_q %d < 0", a->total_q);
    } else if (a->seq_offsets_q || a->seq_offsets_kv) {
        return fail(HSTU_ERR_INVALID_ARG, "seq_offsets are for jagged mode only");
    }
    if ((int64_t)a->batch * a->seqlen_q > INT32_MAX || (int64_t)a->batch * a->seqlen_kv > INT32_MAX)
        return fail(HSTU_ERR_INVALID_ARG, "token count exceeds int32");
    const bool work = rows_q(a) > 0 && a->batch > 0;
    if (work && (!a->q || !a->k || !a->v || !a->o))
        return fail(HSTU_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
    if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
        return fail(HSTU_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    const int64_t min_qk = (int64_t)a->nhead * a->hdim_qk, min_v = (int64_t)a->nhead * a->hdim_v;
    const int64_t strides[4] = {a->q_tok_stride, a->k_tok_stride, a->v_tok_stride, a->o_tok_stride};
    const int64_t mins[4] = {min_qk, min_qk, min_v, min_v};
    for (int i = 0; i < 4; ++i) {
        if (strides[i] == 0) continue;
        if (strides[i] < mins[i] || strides[i] % 8 != 0)
            return fail(HSTU_ERR_INVALID_ARG,
                        "token stride %lld must be 0 or a multiple of 8 that is >= nhead * hdim (%lld)",
                        (long long)strides[i], (long long)mins[i]);
    }
    {
        // the kernels address one (sequence, head) through 32-bit byte offsets,
        // including up to two key tiles (<= 256 rows) past its end
        const int64_t sq = (int64_t)a->seqlen_q + 512, skv = (a->cross ? (int64_t)a->seqlen_kv : (int64_t)a->seqlen_q) + 512;
        const int64_t qs = strides[0] ? strides[0] : mins[0], ks = strides[1] ? strides[1] : mins[1],
                      vs = strides[2] ? strides[2] : mins[2];
        if (sq * qs * 2 >= ((int64_t)1 << 32) || skv * ks * 2 >= ((int64_t)1 << 32) ||
            skv * vs * 2 >= ((int64_t)1 << 32))
            return fail(HSTU_ERR_UNSUPPORTED, "one sequence spans 4 GiB or more of q, k or v");
    }
    if (a->num_groups < 1 || a->num_groups > HSTU_MAX_GROUPS)
        return fail(HSTU_ERR_INVALID_ARG, "num_groups %d not in 1..%d", a->num_groups, HSTU_MAX_GROUPS);
    if (a->batch % a->num_groups != 0)
        return fail(HSTU_ERR_INVALID_ARG, "batch %d is not a multiple of num_groups %d", a->batch,
                    a->num_groups);
    if (!a->groups) return fail(HSTU_ERR_INVALID_ARG, "groups is NULL");
    for (int g = 0; g < a->num_groups; ++g) {
        const hstu_mask_group_t &m = a->groups[g];
        if (m.local_len < 0 || m.context_len < 0 || m.minfull_len < 0)
            return fail(HSTU_ERR_INVALID_ARG, "group %d: negative local/context/minfull length", g);
        if (!isfinite(m.attn_scale)) return fail(HSTU_ERR_INVALID_ARG, "group %d: attn_scale not finite", g);
        if (m.attn_scale == 0.0f && m.max_uih_q < 0)
            return fail(HSTU_ERR_INVALID_ARG, "group %d: attn_scale 0 needs max_uih_q >= 0", g);
    }
    if (!isfinite(a->alpha)) return fail(HSTU_ERR_INVALID_ARG, "alpha not finite");
    if (a->rab_timestamps || a->rab_pos) {
        if (a->cross) return fail(HSTU_ERR_UNSUPPORTED, "the relative attention bias is for self-attention");
        if (a->rab_timestamps && (!a->rab_time || ((uintptr_t)a->rab_time & 3u) ||
                                  ((uintptr_t)a->rab_timestamps & 3u)))
            return fail(HSTU_ERR_INVALID_ARG, "rab_timestamps needs a 4-byte aligned rab_time table");
        if (a->rab_pos && (a->rab_pos_len < 1 || a->rab_pos_len > HSTU_RAB_MAX_POS || ((uintptr_t)a->rab_pos & 3u)))
            return fail(HSTU_ERR_INVALID_ARG, "rab_pos_len %d not in 1..%d (or rab_pos misaligned)", a->rab_pos_len,
                        HSTU_RAB_MAX_POS);
    }
    if (a->lse && !a->softmax) return fail(HSTU_ERR_INVALID_ARG, "lse output is for the softmax variant");
    if (a->lse && ((uintptr_t)a->lse & 3u)) return fail(HSTU_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    return HSTU_OK;
}

void fill_params(const hstu_fwd_args_t *a, int32_t num_splits, hstu::KernelParams &p) {
    memset(&p, 0, sizeof(p));
    p.q = a->q;
    p.k = a->k;
    p.v = a->v;
    p.o = a->o;
    p.lse = a->lse;
    p.q_stride = a->q_tok_stride ? a->q_tok_stride : (int64_t)a->nhead * a->hdim_qk;
    p.k_stride = a->k_tok_stride ? a->k_tok_stride : (int64_t)a->nhead * a->hdim_qk;
    p.v_stride = a->v_tok_stride ? a->v_tok_stride : (int64_t)a->nhead * a->hdim_v;
    p.o_stride = a->o_tok_stride ? a->o_tok_stride : (int64_t)a->nhead * a->hdim_v;
    p.off_q = a->seq_offsets_q;
    p.off_kv = a->seq_offsets_kv;
    p.num_targets = a->num_targets;
    p.B = a->batch;
    p.H = a->nhead;
    p.seqlen_q = a->seqlen_q;
    p.seqlen_kv = a->cross ? a->seqlen_kv : a->seqlen_q;
    p.jagged = a->jagged;
    p.cross = a->cross;
    p.causal = a->causal;
    p.total_rows = (int32_t)rows_q(a);
    const int bm = hstu::block_m_for(a->hdim_qk);
    p.num_qt = (a->seqlen_q + bm - 1) / bm;
    const int64_t bh = (int64_t)a->batch * a->nhead;
    p.bh_pad = (int32_t)((bh + 7) / 8 * 8);
    p.num_splits = num_splits;
    p.schedule = a->schedule == 0 ? 2 : a->schedule;
    p.alpha = a->alpha != 0.0f ? a->alpha : (float)(1.0 / sqrt((double)a->hdim_qk));
    p.inv_alpha = (float)(1.0 / (double)p.alpha);
    p.rab_ts = a->rab_timestamps;
    p.rab_time = a->rab_timestamps ? a->rab_time : nullptr;
    p.rab_pos = a->rab_pos;
    p.rab_pos_len = a->rab_pos ? a->rab_pos_len : 0;
    p.G = a->num_groups;
    p.per_group = a->batch > 0 ? a->batch / a->num_groups : 1;
    for (int g = 0; g < a->num_groups; ++g) {
        const hstu_mask_group_t &m = a->groups[g];
        p.groups[g].local_len = m.local_len;
        p.groups[g].context_len = m.context_len;
        p.groups[g].minfull_len = m.minfull_len;
        p.groups[g].attn_scale =
            m.attn_scale != 0.0f ? m.attn_scale
                                 : (float)(1.0 / (double)(m.max_uih_q > 0 ? m.max_uih_q : 1));
    }
}

// Workspace layout: split-KV partial outputs (256-byte aligned), their LSEs
// (softmax), then, for the persistent schedule, the work queues.
size_t partial_bytes(const hstu_fwd_args_t *a, int32_t num_splits) {
    if (num_splits <= 1) return 0;
    const size_t rows = (size_t)rows_q(a) * (size_t)a->nhead * (size_t)num_splits;
    const size_t o_bytes = rows * (size_t)a->hdim_v * sizeof(float);
    const size_t lse_bytes = a->softmax ? rows * sizeof(float) : 0;
    return ((o_bytes + 255) / 256) * 256 + ((lse_bytes + 255) / 256) * 256;
}
bool wants_queue(const hstu_fwd_args_t *a) { return a->schedule == 0 || a->schedule == 3; }
// the persistent schedule's work queues (validated arguments)
size_t queue_bytes(const hstu_fwd_args_t *a, int32_t num_splits) {
    hstu::KernelParams p;
    fill_params(a, num_splits, p);
    return hstu::queue_bytes(p);
}
constexpr int64_t kPersistentItems = 2048;

// Heavy q-tiles.  When the per-item grid of an unsplit call (schedule left to
// the library) holds fewer work-groups than the chip runs at once, the kernel's
// time is that of its heaviest q-tile, under a causal mask one of a sequence's
// last (its min-full and target rows see the whole history; they may straddle
// two q-tiles).  The last kHeavyLevels q-tiles of every sequence, when their
// lists have more than a chunk of key tiles (heavy_tiles_for), are then cut into
// chunks that run side by side, and a combine pass adds the chunks' partials up.
// The chunk count is the largest (at most kHeavyMaxSplits) whose grid still fits
// the chip at once.  The workspace holds the partials (chunk count x cut levels
// per (b, h)) and each cut q-tile's record, after the rest.
constexpr size_t kHeavyMaxBytes = (size_t)512 << 20;
size_t align256(size_t b) { return (b + 255) / 256 * 256; }
size_t base_workspace_bytes(const hstu_fwd_args_t *a, int32_t num_splits) {
    return partial_bytes(a, num_splits) + (wants_queue(a) ? queue_bytes(a, num_splits) : 0);
}
int32_t heavy_tiles_for(const hstu_fwd_args_t *a) { return hstu::heavy_chunk_tiles(hstu::key_tile_for(a->hdim_qk)); }
// The cut (levels, chunk count) of a call, and the bytes of its partials and
// records; false when nothing is cut.
struct HeavyPlan {
    int32_t levels, splits;
    size_t o_bytes, lse_bytes, meta_bytes;
};
bool heavy_plan(const hstu_fwd_args_t *a, int32_t num_splits, HeavyPlan &h) {
    if (a->schedule != 0 || num_splits != 1) return false;
    hstu::KernelParams p;
    fill_params(a, 1, p);
    if (hstu::grid_size(p) >= kPersistentItems) return false;  // the persistent schedule runs
    const int32_t bn = hstu::key_tile_for(a->hdim_qk);
    if ((p.seqlen_kv + bn - 1) / bn <= heavy_tiles_for(a)) return false;  // no list is long enough
    const int64_t slots = (int64_t)hstu::kChipCUs * hstu::groups_per_cu_for(a->hdim_qk);
    p.heavy = p.num_qt < hstu::kHeavyLevels ? p.num_qt : hstu::kHeavyLevels;
    for (p.num_splits = hstu::kHeavyMaxSplits; p.num_splits >= 2; --p.num_splits)
        if (hstu::grid_size(p) < slots) break;
    if (p.heavy < 1 || p.num_splits < 2) return false;
    const size_t qtiles = (size_t)p.bh_pad * (size_t)p.heavy;
    const size_t rows = qtiles * (size_t)p.num_splits * (size_t)hstu::block_m_for(a->hdim_qk);
    h.levels = p.heavy;
    h.splits = p.num_splits;
    h.o_bytes = align256(rows * (size_t)a->hdim_v * sizeof(float));
    h.lse_bytes = a->softmax ? align256(rows * sizeof(float)) : 0;
    h.meta_bytes = align256(qtiles * 2 * sizeof(int32_t));
    return h.o_bytes + h.lse_bytes + h.meta_bytes <= kHeavyMaxBytes;
}
size_t heavy_bytes(const hstu_fwd_args_t *a, int32_t num_splits) {
    HeavyPlan h;
    return heavy_plan(a, num_splits, h) ? h.o_bytes + h.lse_bytes + h.meta_bytes : 0;
}
size_t workspace_bytes(const hstu_fwd_args_t *a, int32_t num_splits) {
    const size_t base = base_workspace_bytes(a, num_splits);
    const size_t heavy = heavy_bytes(a, num_splits);
    return heavy ? align256(base) + heavy : base;
}

// Schedule and work queues of one call: the persistent schedule (3) when it is
// asked for, or when the schedule is left to the library (0), the workspace
// holds the queues and the grid is large; else schedule 2 (0) or the one asked
// for.
hstu_status_t pick_schedule(const hstu_fwd_args_t *a, int32_t num_splits, void *ws, size_t ws_bytes,
                            hstu::KernelParams &p) {
    const size_t part = partial_bytes(a, num_splits), need = part + hstu::queue_bytes(p);
    const bool room = ws != nullptr && ws_bytes >= need && aligned16(ws);
    if (a->schedule == 3 && !room)
        return fail(HSTU_ERR_WORKSPACE, "schedule 3 needs a 16-byte aligned workspace of %zu bytes, %zu given",
                    need, ws ? ws_bytes : (size_t)0);
    // left to the library, the persistent grid runs only where its planning
    // kernel (one short launch) is small against the work: from kPersistentItems
    // possible items, four per resident work-group on a 256-CU part
    const bool worth = a->schedule == 3 || hstu::grid_size(p) >= kPersistentItems;
    if (wants_queue(a) && room && worth) {
        p.schedule = 3;
        p.queue = (uint32_t *)((char *)ws + part);
    } else {
        p.schedule = a->schedule == 0 ? 2 : a->schedule;
        p.queue = nullptr;
    }
    return HSTU_OK;
}

hstu_status_t check_grid(const hstu::KernelParams &p) {
    if (hstu::grid_size(p) > (int64_t)INT32_MAX)
        return fail(HSTU_ERR_INVALID_ARG, "problem too large for one launch");
    return HSTU_OK;
}

hstu_status_t hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return HSTU_OK;
    return fail(HSTU_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace hstu {
namespace api {

hstu_status_t fail(hstu_status_t st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}
void clear_error() { g_last_error[0] = '\0'; }
hstu_status_t validate_fwd(const hstu_fwd_args_t *a) { return validate(a); }
hstu_status_t hip_status(hipError_t e, const char *what) { return ::hip_status(e, what); }
int64_t rows_q(const hstu_fwd_args_t *a) { return ::rows_q(a); }

}  // namespace api
}  // namespace hstu

namespace {
// the caller's profiling event (hstu_fwd_args_t::prof_begin / prof_end), if any
hstu_status_t record_prof(void *ev, hipStream_t stream) {
    if (ev == nullptr) return HSTU_OK;
    return hip_status(hipEventRecord((hipEvent_t)ev, stream), "profiling event record");
}
}  // namespace

extern "C" {

hstu_status_t hstu_validate_args(const hstu_fwd_args_t *args) { return validate(args); }

size_t hstu_fwd_workspace_size(const hstu_fwd_args_t *args, int32_t num_splits) {
    if (validate(args) != HSTU_OK || num_splits < 1 || num_splits > HSTU_MAX_SPLITS) return 0;
    return workspace_bytes(args, num_splits);
}

hstu_status_t hstu_fwd(const hstu_fwd_args_t *args, void *ws, size_t ws_bytes, void *hip_stream) {
    hstu_status_t st = validate(args);
    if (st != HSTU_OK) return st;
    hstu::KernelParams p;
    fill_params(args, 1, p);
    if ((st = check_grid(p)) != HSTU_OK) return st;
    if ((st = pick_schedule(args, 1, ws, ws_bytes, p)) != HSTU_OK) return st;
    if (p.total_rows == 0 || p.B == 0) return HSTU_OK;
    // a small per-item grid left to the library runs in q-tile levels from each
    // sequence's end (the heaviest q-tiles dispatched first)
    if (args->schedule == 0 && p.queue == nullptr && hstu::grid_size(p) < kPersistentItems) p.levels = 1;
    // heavy q-tiles cut into chunks when the per-item grid runs and the workspace
    // holds the chunks' partials (hstu_fwd_workspace_size counts them)
    HeavyPlan hp;
    if (p.levels && heavy_plan(args, 1, hp) && ws != nullptr && aligned16(ws) &&
        ws_bytes >= workspace_bytes(args, 1)) {
        char *h = (char *)ws + align256(base_workspace_bytes(args, 1));
        p.heavy = hp.levels;
        p.heavy_tiles = heavy_tiles_for(args);
        p.num_splits = hp.splits;
        p.hpart_o = (float *)h;
        h += hp.o_bytes;
        if (args->softmax) p.hpart_lse = (float *)h;
        h += hp.lse_bytes;
        p.hmeta = (int32_t *)h;
        if ((st = check_grid(p)) != HSTU_OK) return st;
    }
    hipStream_t stream = (hipStream_t)hip_stream;
    if ((st = record_prof(args->prof_begin, stream)) != HSTU_OK) return st;
    st = hip_status(hstu::launch_forward(p, args->dtype, args->hdim_qk, args->hdim_v, args->softmax != 0, false, stream),
                    "forward kernel launch");
    if (st == HSTU_OK) st = record_prof(args->prof_end, stream);
    if (st != HSTU_OK || !p.heavy) return st;
    return hip_status(hstu::launch_heavy_combine(p, args->dtype, args->hdim_qk, args->hdim_v, args->softmax != 0, stream),
                      "heavy q-tile combine launch");
}

hstu_status_t hstu_fwd_splitkv(const hstu_fwd_args_t *args, int32_t num_splits, void *ws,
                               size_t ws_bytes, void *hip_stream) {
    hstu_status_t st = validate(args);
    if (st != HSTU_OK) return st;
    if (num_splits < 1 || num_splits > HSTU_MAX_SPLITS)
        return fail(HSTU_ERR_INVALID_ARG, "num_splits %d not in 1..%d", num_splits, HSTU_MAX_SPLITS);
    if (num_splits == 1) return hstu_fwd(args, ws, ws_bytes, hip_stream);
    const size_t need = partial_bytes(args, num_splits);
    if (!ws || ws_bytes < need)
        return fail(HSTU_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    ws ? ws_bytes : (size_t)0);
    if (!aligned16(ws)) return fail(HSTU_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    hstu::KernelParams p;
    fill_params(args, num_splits, p);
    if ((st = check_grid(p)) != HSTU_OK) return st;
    if ((st = pick_schedule(args, num_splits, ws, ws_bytes, p)) != HSTU_OK) return st;
    if (p.total_rows == 0 || p.B == 0) return HSTU_OK;
    const size_t rows = (size_t)p.total_rows * (size_t)p.H * (size_t)num_splits;
    p.part_o = (float *)ws;
    p.part_lse = args->softmax ? (float *)((char *)ws + ((rows * args->hdim_v * sizeof(float) + 255) / 256) * 256)
                               : nullptr;
    hipStream_t stream = (hipStream_t)hip_stream;
    if ((st = record_prof(args->prof_begin, stream)) != HSTU_OK) return st;
    st = hip_status(hstu::launch_forward(p, args->dtype, args->hdim_qk, args->hdim_v, args->softmax != 0, true, stream),
                    "split-KV kernel launch");
    if (st == HSTU_OK) st = record_prof(args->prof_end, stream);
    if (st != HSTU_OK) return st;
    return hip_status(hstu::launch_combine(p, args->dtype, args->hdim_v, args->softmax != 0, stream),
                      "combine kernel launch");
}

hstu_status_t hstu_fwd_splitkv_noalloc(const hstu_fwd_args_t *args, int32_t num_splits, void *hip_stream) {
    hstu_status_t st = validate(args);
    if (st != HSTU_OK) return st;
    if (num_splits < 1 || num_splits > HSTU_MAX_SPLITS)
        return fail(HSTU_ERR_INVALID_ARG, "num_splits %d not in 1..%d", num_splits, HSTU_MAX_SPLITS);
    // (the room for cutting heavy q-tiles is left out: hstu_fwd cuts them only
    // when the scratch holds that room too)
    const size_t need = base_workspace_bytes(args, num_splits);
    if (need > hstu::kScratchBytes)
        return fail(HSTU_ERR_WORKSPACE,
                    "this problem needs %zu bytes of workspace; the static scratch holds %zu (use hstu_fwd_splitkv "
                    "with a workspace of hstu_fwd_workspace_size bytes)",
                    need, hstu::kScratchBytes);
    if (rows_q(args) == 0 || args->batch == 0) return HSTU_OK;
    void *ws = nullptr;
    if ((st = hip_status(hstu::scratch_region(&ws), "static scratch address")) != HSTU_OK) return st;
    return hstu_fwd_splitkv(args, num_splits, ws, hstu::kScratchBytes, hip_stream);
}

hstu_status_t hstu_count_visible_pairs(const hstu_fwd_args_t *args, unsigned long long *d_count,
                                       void *hip_stream) {
    hstu_status_t st = validate(args);
    if (st != HSTU_OK) return st;
    if (!d_count) return fail(HSTU_ERR_INVALID_ARG, "d_count is NULL");
    hstu::KernelParams p;
    fill_params(args, 1, p);
    if ((st = check_grid(p)) != HSTU_OK) return st;
    if (p.B == 0) p.num_qt = 0;
    return hip_status(hstu::launch_count(p, args->hdim_qk, d_count, (hipStream_t)hip_stream),
                      "count kernel launch");
}

const char *hstu_status_string(hstu_status_t s) {
    switch (s) {
        case HSTU_OK: return "HSTU_OK";
        case HSTU_ERR_INVALID_ARG: return "HSTU_ERR_INVALID_ARG";
        case HSTU_ERR_UNSUPPORTED: return "HSTU_ERR_UNSUPPORTED";
        case HSTU_ERR_WORKSPACE: return "HSTU_ERR_WORKSPACE";
        case HSTU_ERR_HIP: return "HSTU_ERR_HIP";
    }
    return "HSTU_ERR_UNKNOWN";
}

const char *hstu_last_error(void) { return g_last_error; }

int32_t hstu_abi_version(void) { return HSTU_ABI_VERSION; }

}  // extern "C"

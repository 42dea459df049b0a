// hstu_params.h - the by-value argument block of the HSTU forward kernels,
// filled on the host from hstu_fwd_args_t (include/hstu.h) after validation and
// default resolution.
#pragma once

#include <stdint.h>

#include "hstu.h"

namespace hstu {

struct GroupDev {
    int32_t local_len, context_len, minfull_len;
    float attn_scale;  // resolved: a stored 0 has already been replaced by 1 / max UIH length
};

struct KernelParams {
    const void *q, *k, *v;
    void *o;
    float *lse;        // softmax LSE output or nullptr
    float *part_o;     // split-KV partial outputs [split][row][H][Dv] fp32
    float *part_lse;   // split-KV partial LSE     [split][row][H]    fp32
    int64_t q_stride, k_stride, v_stride, o_stride;  // elements between tokens
    const int32_t *off_q, *off_kv, *num_targets;
    int32_t B, H;
    int32_t seqlen_q, seqlen_kv;  // batched: physical; jagged: upper bounds
    int32_t jagged, cross, causal;
    int32_t total_rows;           // rows of o: jagged total_q, batched B * seqlen_q
    int32_t num_qt;               // q-tiles per sequence (upper bound)
    int32_t bh_pad;               // B * H rounded up to a multiple of 8
    int32_t num_splits;
    int32_t schedule;             // 1 or 2 (see decode_work)
    float alpha;                  // resolved QK scale
    float inv_alpha;              // 1 / alpha (the bias enters the score MFMAs divided by alpha)
    int32_t G, per_group;
    GroupDev groups[HSTU_MAX_GROUPS];
    // relative attention bias (nullptr: term absent)
    const int32_t *rab_ts;   // [tokens] timestamps
    const float *rab_time;   // [H][HSTU_RAB_TIME_BUCKETS]
    const float *rab_pos;    // [H][rab_pos_len]
    int32_t rab_pos_len;
    // persistent schedule: the per-XCD work queues (layout below), written by
    // the planning kernel before the launch; nullptr: one work item per
    // work-group, the work-group id
    uint32_t *queue;
    // per-item grid of an unsplit call: work-group ids run over q-tile levels
    // counted from each sequence's end (decode_work), so that the last q-tile of
    // every sequence, the heaviest under a causal mask, is dispatched first
    int32_t levels;
    // heavy q-tiles (with levels): heavy > 0 levels from each sequence's end are
    // cut; num_splits is the largest chunk count, and the split index of a work
    // item of those levels picks its chunk of the q-tile's key-tile list, cut
    // into chunks of at least heavy_tiles tiles; the chunks' fp32 partial
    // results (and LSEs) go to hpart_o [slot][BM rows][Dv] and hpart_lse
    // [slot][BM rows], slot = hq num_splits + chunk, hq = (b H + h) heavy +
    // level; hmeta [hq][2] holds that q-tile's chunk count | valid rows << 8 and
    // its first token
    int32_t heavy;
    int32_t heavy_tiles;
    float *hpart_o;
    float *hpart_lse;
    int32_t *hmeta;
};

// Work queues of the persistent schedule, in the caller's workspace:
//   words [0, 8)    take counter of XCD queue x (cleared by the planning kernel)
//   words [8, 16)   number of items in queue x
//   byte 256 on     queue x's items at kQueueHeader + 8 (x * per_queue + i):
//                   bh | (qt << 8 | split) << 32 (uint64), per_queue = grid / 8
constexpr size_t kQueueHeader = 256;
constexpr int kQueueCount = 8;  // word offset of the item counts

}  // namespace hstu

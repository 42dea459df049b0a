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
    int32_t G, per_group;
    GroupDev groups[HSTU_MAX_GROUPS];
    // relative attention bias (nullptr: term absent)
    const int32_t *rab_ts;   // [tokens] timestamps
    const float *rab_time;   // [H][HSTU_RAB_TIME_BUCKETS]
    const float *rab_pos;    // [H][rab_pos_len]
    int32_t rab_pos_len;
    // persistent schedule: kQueueWords work counters, zeroed before the launch
    // (nullptr: one work item per work-group, the work-group id)
    uint32_t *queue;
};

// work counters of the persistent schedule: one per XCD queue
constexpr int kQueueWords = 8;
constexpr size_t kQueueBytes = 256;  // workspace reserved for them

}  // namespace hstu

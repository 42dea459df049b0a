/*
 * hstu.h - C ABI of the MI355X (gfx950) HSTU attention forward library (libhstu.so).
 *
 * The operator (CK example README "18_hstu_attention", section "Forward
 * computation"; mask components from its "Masking" table, modes from "Modes of
 * operation", split-KV from "Split-KV"):
 *
 *   s[b,h,i,j] = alpha * q[b,i,h,:] . k[b,j,h,:]
 *   SiLU variant:    o[b,i,h,:] = attn_scale * sum_j vis(i,j) * SiLU(s[b,h,i,j]) * v[b,j,h,:]
 *   softmax variant: o[b,i,h,:] = attn_scale * sum_{j vis} softmax_j(s[b,h,i,:]) * v[b,j,h,:]
 *                    and optionally LSE[b,h,i] = ln sum_{j vis} exp(s[b,h,i,j])
 *
 * vis(i,j) is the composite functional mask.  Per sequence b with group g,
 * C = context_len, L = local_len, M = minfull_len, T = num_targets[b]:
 *   query rows  [context C | UIH U_q | targets T]          (S_q = C + U_q + T)
 *   key rows    [context C | UIH U_kv | targets T]  self-attention (S_kv = S_q)
 *               [context C | UIH U_kv]              cross-attention (S_kv = C + U_kv)
 *   - target keys are never attended; context keys are visible to every query;
 *   - a UIH query u sits at x = u + (U_kv - U_q) on the key-UIH axis, a target
 *     query at x = U_kv, a context query at x = -1 (under causal masking it sees
 *     only the context);
 *   - causal: UIH key v visible only if v <= x;
 *   - local window (L > 0): |x - v| <= L, except "full" rows: with M > 0 the last
 *     M UIH queries and all target queries see their whole causal history.
 *   Lengths that do not fit are clamped: C' = min(C, S), T' = min(T, S - C').
 *
 * Conventions (all entry points):
 *   - All tensors are caller-owned device memory; the library never allocates.
 *     Split-KV partial results live in a caller-provided workspace whose size
 *     hstu_fwd_workspace_size() returns.
 *   - Work is enqueued asynchronously on the caller's HIP stream (hipStream_t
 *     passed as void*; NULL = the null stream).  No host synchronisation.
 *   - Argument errors are detected on the host before any launch and returned as
 *     a status; hstu_last_error() then holds a message (thread-local).
 *   - Device-resident metadata (offsets, target counts) is not validated on the
 *     device; the kernels clamp lengths as above and never read or write outside
 *     [offset[b], offset[b+1]) of a sequence, but offsets must be non-decreasing
 *     and within the tensors.
 *   - Layout: q [tokens, nhead, hdim_qk], k [tokens, nhead, hdim_qk],
 *     v [tokens, nhead, hdim_v], o [tokens, nhead, hdim_v], each head's vector
 *     contiguous, heads contiguous within a token; the token stride is given in
 *     elements (0 = nhead * hdim).  Batched mode: token = b * seqlen + i.
 *     Jagged mode: token = seq_offsets[b] + i.  Rows must be 16-byte aligned
 *     (strides multiples of 8 elements, base pointers 16-byte aligned).
 *   - Accumulation and the non-linearity run in fp32; o is rounded to the input
 *     dtype (round-to-nearest-even).
 */
#ifndef HSTU_H
#define HSTU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSTU_ABI_VERSION 4
#define HSTU_MAX_GROUPS 64
#define HSTU_MAX_SPLITS 128
#define HSTU_RAB_TIME_BUCKETS 11 /* time-gap buckets of the relative attention bias */
#define HSTU_RAB_MAX_POS 2048    /* longest positional bias table */
#define HSTU_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20) /* static scratch of hstu_fwd_splitkv_noalloc */

typedef enum {
    HSTU_OK = 0,
    HSTU_ERR_INVALID_ARG = 1, /* a host-checkable argument is wrong */
    HSTU_ERR_UNSUPPORTED = 2, /* valid but not built (e.g. a head-dim pair) */
    HSTU_ERR_WORKSPACE = 3,   /* workspace missing or too small */
    HSTU_ERR_HIP = 4          /* a HIP runtime call failed (launch error) */
} hstu_status_t;

typedef enum { HSTU_FP16 = 0, HSTU_BF16 = 1 } hstu_dtype_t;

/* Per-group mask scalars (README "Attention variants": group HSTU passes one set
 * per group; no-group HSTU is num_groups = 1).  Sequences are grouped in
 * contiguous runs: sequence b belongs to group b / (batch / num_groups). */
typedef struct {
    int32_t local_len;   /* diagonal window; 0 disables the local mask */
    int32_t context_len; /* always-visible prefix length */
    int32_t minfull_len; /* tail of the UIH that attends the full history; 0 disables */
    float attn_scale;    /* post-non-linearity scale; 0 selects 1 / max(max_uih_q, 1) */
    int32_t max_uih_q;   /* largest UIH query length in the group; read only when attn_scale == 0.
                          * (CK README "Command-line arguments": an attn_scale of 0 means one over
                          * the max UIH length, derived there from the host-side lengths; here the
                          * lengths live on the device, so the caller states it, and 0 gives 1.) */
} hstu_mask_group_t;

typedef struct {
    int32_t dtype;     /* hstu_dtype_t of q, k, v and o */
    int32_t batch;     /* number of sequences B (>= 0) */
    int32_t nhead;     /* heads H (>= 1) */
    int32_t hdim_qk;   /* (hdim_qk, hdim_v) in {64/64, 96/96, 96/64, 128/128, 256/256} */
    int32_t hdim_v;    /* other pairs: HSTU_ERR_UNSUPPORTED */
    int32_t jagged;    /* 0: batched [B, S, H, D]; 1: jagged [1, total, H, D] + seq_offsets */
    int32_t cross;     /* 0: self-attention (k/v laid out like q, targets included); 1: cross */
    int32_t seqlen_q;  /* batched: physical S_q; jagged: an upper bound of every S_q (grid size) */
    int32_t seqlen_kv; /* batched: physical S_kv (== seqlen_q for self); jagged: upper bound */
    int32_t total_q;   /* jagged: seq_offsets_q[batch] (rows of o / lse); batched: ignored */
    const void *q;
    const void *k;
    const void *v;
    void *o;
    int64_t q_tok_stride; /* elements between consecutive tokens; 0 = nhead * hdim_qk */
    int64_t k_tok_stride;
    int64_t v_tok_stride; /* 0 = nhead * hdim_v */
    int64_t o_tok_stride;
    const int32_t *seq_offsets_q;  /* jagged: device [batch + 1], non-decreasing, [0] = 0 */
    const int32_t *seq_offsets_kv; /* jagged cross-attention: device [batch + 1]; else NULL */
    const int32_t *num_targets;    /* device [batch] target counts; NULL = no targets */
    int32_t causal;                /* 1: causal mask (README default) */
    int32_t softmax;               /* 0: SiLU; 1: softmax (with optional LSE) */
    float alpha;                   /* QK scale; 0 selects 1/sqrt(hdim_qk) */
    int32_t num_groups;            /* 1 ..= HSTU_MAX_GROUPS, batch % num_groups == 0 */
    const hstu_mask_group_t *groups; /* host array [num_groups], read during the call only */
    float *lse; /* softmax only, device, NULL = not saved: batched [B][H][S_q], jagged [H][total_q];
                   natural log; -inf for a row that sees no key */
    int32_t schedule; /* work order: 0 = library's choice (3 when the workspace holds the
                         work queues and there are at least 2048 possible items, else 2);
                         1 = q-tile levels heavy-first; 2 = per-XCD sequence groups (each
                         (b,h) kept on one XCD's L2), one work-group per q-tile; 3 = per
                         XCD, the (b,h) pairs longest first, taken from per-XCD work
                         queues by a persistent grid (one resident set of work-groups: no
                         launch gaps, no empty q-tiles, the tail stolen across XCDs; needs
                         the workspace) */
    /* Relative attention bias (HSTU explainer, "The layer, line by line" (b) and "The
     * relative attention bias"); self-attention only (HSTU_ERR_UNSUPPORTED with cross).
     * Added to the score before the mask and the non-linearity:
     *   s[b,h,i,j] = alpha q_i.k_j + rab_pos[h][min(|i - j|, rab_pos_len - 1)]
     *                              + rab_time[h][bucket(|ts_i - ts_j|)]
     * i, j: positions in the sequence; bucket(d): how many of the gap edges
     * 1, 5, 30, 60, 300, 1800, 3600, 86400, 604800, 2600000 (seconds) are <= d.
     * All NULL: no bias (the fields of ABI version 1 keep their meaning). */
    const int32_t *rab_timestamps; /* device [tokens of q] int32 seconds; NULL = no time term */
    const float *rab_time;         /* device [nhead][HSTU_RAB_TIME_BUCKETS], with rab_timestamps */
    const float *rab_pos;          /* device [nhead][rab_pos_len]; NULL = no positional term */
    int32_t rab_pos_len;           /* 1 ..= HSTU_RAB_MAX_POS when rab_pos is set */
    /* Profiling hooks (ABI version 4), for callers that time the main kernel alone
     * (the roofline of a benchmark): hipEvent_t handles, owned by the caller, that
     * the call records on its stream right before and right after launching its
     * main kernel (the forward kernel of hstu_fwd, the split kernel of
     * hstu_fwd_splitkv); the planning and combine passes fall outside them.  Not
     * recorded when the call launches nothing (an empty problem or an error).
     * NULL = no event. */
    void *prof_begin;
    void *prof_end;
} hstu_fwd_args_t;

/* Host-only argument check (no HIP call); also run by every entry point.  It covers
 * the operator's arguments as CK README "Command-line arguments" lists them (dtype,
 * batch and groups, jagged mode, heads, head dims, lengths, targets, softmax, causal,
 * the mask lengths, alpha and attn_scale) plus this boundary's own (pointers,
 * strides, alignment, schedule, bias).  Returns HSTU_OK, HSTU_ERR_INVALID_ARG (a
 * value out of its domain) or HSTU_ERR_UNSUPPORTED (valid, not built: a head-dim
 * pair, bias with cross-attention); hstu_last_error() then names the argument.
 * Reads args only; NULL args is HSTU_ERR_INVALID_ARG. */
hstu_status_t hstu_validate_args(const hstu_fwd_args_t *args);

/* Bytes of workspace for num_splits splits (num_splits == 1: hstu_fwd): the split-KV
 * partial results (README "Split-KV": fp32 partial rows and, for softmax, their LSEs),
 * plus, when args->schedule is 0 or 3, the work queues (256 bytes and 8 per possible
 * item: batch * nhead rounded up to 8, times the q-tiles of max_seqlen_q in 128 rows,
 * times num_splits), plus, for an unsplit call with schedule 0 whose per-item grid
 * is smaller than the chip's resident work-groups, room for cutting each
 * sequence's last two q-tiles into 2 to 4 chunks (an fp32 partial of 128 rows per
 * chunk, its LSEs for softmax, and an 8-byte record per cut q-tile; at most
 * 512 MiB, else the room is left out and nothing is cut).  Host-only; returns 0 on
 * invalid arguments. */
size_t hstu_fwd_workspace_size(const hstu_fwd_args_t *args, int32_t num_splits);

/* The forward operator: one fused kernel per call (plus, for schedule 3, an 8-work-
 * group kernel that writes the work queues; plus, when long q-tiles are cut into
 * chunks, a combine kernel).  ws may be NULL: then schedule 0 runs as 2, and
 * schedule 3 fails with HSTU_ERR_WORKSPACE.  Schedule 0 on a small per-item grid
 * runs the q-tiles in levels from each sequence's end, and, with room in ws, cuts
 * each sequence's last two q-tiles, when longer than 256 keys' worth of key tiles,
 * into up to 4 chunks whose fp32 partials a combine kernel adds up (same terms,
 * another order of addition).  A workspace of at least
 * hstu_fwd_workspace_size(args, 1) bytes, 16-byte aligned, is used by schedule 0
 * and 3; its contents need no initialisation; calls that share a workspace must
 * not overlap in time. */
hstu_status_t hstu_fwd(const hstu_fwd_args_t *args, void *ws, size_t ws_bytes, void *hip_stream);

/* Split-KV forward (README "Split-KV"): the key axis of every sequence is cut into
 * num_splits contiguous chunks processed by separate work-groups, which write fp32
 * partial outputs (and LSEs for softmax) into ws; a second kernel combines them into
 * o (and lse).  The result equals hstu_fwd's up to fp32 reassociation.
 * 1 <= num_splits <= HSTU_MAX_SPLITS; ws_bytes >= the partial results' share of
 * hstu_fwd_workspace_size() (without room for the work queues schedule 0 runs as
 * 2; schedule 3 needs it). */
hstu_status_t hstu_fwd_splitkv(const hstu_fwd_args_t *args, int32_t num_splits, void *ws,
                               size_t ws_bytes, void *hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that must not call hipMalloc, harnesses that forbid it):
 * hstu_fwd_splitkv (num_splits == 1: hstu_fwd) with its workspace - the split-KV
 * partial results and the persistent schedule's work queues - in a static device
 * array of HSTU_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends.  The caller passes inputs and outputs as for
 * hstu_fwd_splitkv; the call allocates and frees nothing.  A problem whose
 * workspace (hstu_fwd_workspace_size without the room for cutting long q-tiles
 * into chunks: that room is used only when the scratch holds it too) exceeds the
 * scratch is rejected with
 * HSTU_ERR_WORKSPACE before anything runs.  All calls on one GPU share its
 * scratch (each call's kernels overwrite what they use; nothing needs to start at
 * zero): calls that overlap in time on one GPU (other streams, other threads)
 * race and must be serialised by the caller.  The first call on a device looks
 * the scratch's address up (hipGetSymbolAddress) with that device current. */
hstu_status_t hstu_fwd_splitkv_noalloc(const hstu_fwd_args_t *args, int32_t num_splits, void *hip_stream);

/* Counts, on the device, the visible (b, h, i, j) pairs inside the key tiles the
 * forward kernel schedules, with the kernel's own mask predicate.  Equal to the
 * number of visible pairs of the mask exactly when no skipped tile holds one: the
 * check CK README "Test / Verify" makes against a CPU reference, here on the mask
 * alone, and the FLOP count of README "Benchmark" (the two GEMMs) restricted to
 * visible pairs.  d_count: device pointer to one uint64, overwritten (zeroed by
 * the library on the stream first); the call returns before the count is ready
 * (read it after synchronising hip_stream).  Errors as hstu_validate_args, plus
 * HSTU_ERR_INVALID_ARG for a NULL d_count and HSTU_ERR_HIP for a failed launch. */
hstu_status_t hstu_count_visible_pairs(const hstu_fwd_args_t *args, unsigned long long *d_count,
                                       void *hip_stream);

const char *hstu_status_string(hstu_status_t status);
const char *hstu_last_error(void);
int32_t hstu_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H */

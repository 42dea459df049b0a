/*
 * hstu_layer.h - C ABI of the HSTU layer around the attention operator
 * (libhstu.so; same status codes, dtypes and conventions as hstu.h).
 *
 * HSTU explainer, "The layer, line by line": one layer maps X [n, d_model] by
 *   (a) pointwise projection  Y = SiLU(X W1^T + b1), split along the features as
 *       [U | V | Q | K] (U, V: nhead * hdim_v wide; Q, K: nhead * hdim_qk wide);
 *   (b) spatial aggregation   A = the attention operator of hstu.h on Q, K, V
 *       (pointwise SiLU or softmax, functional mask, optional relative bias);
 *   (c) pointwise transformation with a residual around the block
 *       out = X + ((LayerNorm(A) * gamma + beta) * U) W2^T + b2.
 * The pages show the sub-layers' equations only as stripped images: the split
 * order, the layer norm (population variance, eps inside the square root, per-
 * feature affine) and the residual's place are this library's reading of the text.
 *
 * The three kernels are exported separately too (hstu_linear_fwd for (a) and
 * the f2 + residual part of (c), hstu_norm_gate_fwd for the gated norm), so a
 * caller can compose them with its own buffers.
 *
 * Conventions: device pointers, caller-owned memory, asynchronous on the given
 * HIP stream, host-side validation before any launch (status + hstu_last_error()).
 * Activations and weights are fp16 or bf16 (one dtype per call); biases and the
 * norm's affine are fp32.  Accumulation in fp32; outputs rounded to the dtype
 * (round-to-nearest-even).  Row strides are in elements, multiples of 8, and
 * every pointer is 16-byte aligned.
 */
#ifndef HSTU_LAYER_H
#define HSTU_LAYER_H

#include <stddef.h>
#include <stdint.h>

#include "hstu.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { HSTU_ACT_NONE = 0, HSTU_ACT_SILU = 1 } hstu_activation_t;

/* y = act(x w^T + bias) + residual   (explainer, "The layer, line by line" (a), (c))
 * x [rows][in_features] (row stride x_stride, 0 = in_features), w [out_features]
 * [in_features] contiguous (the layout of a torch Linear weight), bias [out_features]
 * fp32 or NULL, residual [rows][out_features] (stride residual_stride, 0 = dense) or
 * NULL, added after the activation; y [rows][out_features] (stride y_stride).
 * in_features % 64 == 0, out_features % 8 == 0, rows >= 0.  y must not overlap x,
 * w or residual. */
typedef struct {
    int32_t dtype;        /* HSTU_BF16 or HSTU_FP16: x, w, residual, y */
    int64_t rows;
    int32_t in_features;
    int32_t out_features;
    const void *x;
    int64_t x_stride;
    const void *w;
    const float *bias;
    int32_t activation;   /* hstu_activation_t */
    const void *residual;
    int64_t residual_stride;
    void *y;
    int64_t y_stride;
} hstu_linear_args_t;

hstu_status_t hstu_linear_fwd(const hstu_linear_args_t *args, void *hip_stream);

/* z = (LayerNorm(a) * gamma + beta) * u over `width` features per row
 * (explainer, "The layer, line by line" (c): the normalised attention output
 * gated by U).  LayerNorm: mean and population variance of the row, eps inside
 * the square root.  gamma/beta fp32 [width] or NULL (1 / 0).  width % 8 == 0,
 * width <= 4096.  z may be a (in place); u must not overlap z. */
typedef struct {
    int32_t dtype;
    int64_t rows;
    int32_t width;
    const void *a;
    int64_t a_stride;
    const void *u;
    int64_t u_stride;
    const float *gamma;
    const float *beta;
    float eps;            /* > 0 */
    void *z;
    int64_t z_stride;
} hstu_norm_gate_args_t;

hstu_status_t hstu_norm_gate_fwd(const hstu_norm_gate_args_t *args, void *hip_stream);

/* One whole layer.  attn describes the sequences (batched or jagged), heads, head
 * dims, mask, groups and optional relative bias exactly as for hstu_fwd; it must
 * be self-attention (cross = 0) and its q, k, v, o, token strides and lse are
 * ignored (the layer uses its own buffers); its profiling events, when set,
 * bracket the attention's forward kernel.  Tokens n = attn.total_q (jagged) or
 * batch * seqlen_q.  x, out [n][d_model] dense; w1 [2 H (dv + dqk)][d_model];
 * b1 [2 H (dv + dqk)]; w2 [d_model][H dv]; b2 [d_model]; ln_gamma, ln_beta [H dv]
 * or NULL.  d_model % 64 == 0; H dv a multiple of 64 (the input width of f2) and
 * <= 4096.  out must not overlap x.  Every launch's arguments are checked before
 * the first launch, so an argument error never leaves the layer half done.
 * The workspace (hstu_layer_workspace_size bytes, 256-byte aligned) holds the
 * projection [n][2 H (dv + dqk)] and the attention output [n][H dv]; with no
 * tokens (n = 0) nothing is launched and ws may be NULL. */
typedef struct {
    hstu_fwd_args_t attn;
    int32_t d_model;
    const void *x;
    const void *w1;
    const float *b1;
    const float *ln_gamma;
    const float *ln_beta;
    float ln_eps;
    const void *w2;
    const float *b2;
    void *out;
} hstu_layer_args_t;

/* 0 on invalid arguments. */
size_t hstu_layer_workspace_size(const hstu_layer_args_t *args);

/* Four launches on hip_stream: f1 + SiLU, the attention, norm * gate, f2 + residual. */
hstu_status_t hstu_layer_fwd(const hstu_layer_args_t *args, void *ws, size_t ws_bytes, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_LAYER_H */

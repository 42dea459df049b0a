// hstu_layer_api.cpp - the C ABI of include/hstu_layer.h: validation and the
// launch sequence of one HSTU layer (HSTU explainer, "The layer, line by line").
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include "hstu.h"
#include "hstu_api_internal.h"
#include "hstu_layer.h"
#include "hstu_layer_launch.h"
#include "hstu_params.h"

using hstu::api::fail;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// the linear kernel addresses one tile of up to 256 rows with 32-bit offsets and
// a 32-bit buffer range (256 rows x 2^22 elements x 2 bytes = 2^31)
constexpr int64_t kMaxStride = (int64_t)1 << 22;

hstu_status_t check_linear(const hstu_linear_args_t *a) {
    hstu::api::clear_error();
    if (!a) return fail(HSTU_ERR_INVALID_ARG, "args is NULL");
    if (a->dtype != HSTU_FP16 && a->dtype != HSTU_BF16)
        return fail(HSTU_ERR_INVALID_ARG, "dtype %d is neither HSTU_FP16 nor HSTU_BF16", a->dtype);
    if (a->rows < 0) return fail(HSTU_ERR_INVALID_ARG, "rows %lld < 0", (long long)a->rows);
    if (a->in_features <= 0 || a->in_features % 64 != 0)
        return fail(HSTU_ERR_UNSUPPORTED, "in_features %d: a positive multiple of 64 is needed", a->in_features);
    if (a->out_features <= 0 || a->out_features % 8 != 0)
        return fail(HSTU_ERR_UNSUPPORTED, "out_features %d: a positive multiple of 8 is needed", a->out_features);
    if (a->activation != HSTU_ACT_NONE && a->activation != HSTU_ACT_SILU)
        return fail(HSTU_ERR_INVALID_ARG, "activation %d unknown", a->activation);
    if (!a->x || !a->w || !a->y) return fail(HSTU_ERR_INVALID_ARG, "x, w and y are required");
    if (!aligned16(a->x) || !aligned16(a->w) || !aligned16(a->y) || !aligned16(a->bias) ||
        !aligned16(a->residual))
        return fail(HSTU_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    const int64_t xs = a->x_stride ? a->x_stride : a->in_features;
    const int64_t ys = a->y_stride ? a->y_stride : a->out_features;
    const int64_t rs = a->residual_stride ? a->residual_stride : a->out_features;
    if (xs < a->in_features || ys < a->out_features || (a->residual && rs < a->out_features))
        return fail(HSTU_ERR_INVALID_ARG, "a row stride is shorter than its row");
    if (xs % 8 || ys % 8 || rs % 8) return fail(HSTU_ERR_INVALID_ARG, "row strides must be multiples of 8");
    if (xs > kMaxStride || (int64_t)a->in_features > kMaxStride)
        return fail(HSTU_ERR_UNSUPPORTED, "row stride above %lld elements", (long long)kMaxStride);
    return HSTU_OK;
}

void fill_linear(const hstu_linear_args_t *a, hstu::layer::LinearParams &p) {
    p.x = (const uint16_t *)a->x;
    p.x_stride = a->x_stride ? a->x_stride : a->in_features;
    p.w = (const uint16_t *)a->w;
    p.bias = a->bias;
    p.res = (const uint16_t *)a->residual;
    p.r_stride = a->residual_stride ? a->residual_stride : a->out_features;
    p.y = (uint16_t *)a->y;
    p.y_stride = a->y_stride ? a->y_stride : a->out_features;
    p.M = a->rows;
    p.N = a->out_features;
    p.K = a->in_features;
    p.act = a->activation;
    p.m_tiles = (a->rows + 127) / 128;
    p.n_tiles = (a->out_features + 127) / 128;
}

hstu_status_t check_norm_gate(const hstu_norm_gate_args_t *a) {
    hstu::api::clear_error();
    if (!a) return fail(HSTU_ERR_INVALID_ARG, "args is NULL");
    if (a->dtype != HSTU_FP16 && a->dtype != HSTU_BF16)
        return fail(HSTU_ERR_INVALID_ARG, "dtype %d is neither HSTU_FP16 nor HSTU_BF16", a->dtype);
    if (a->rows < 0) return fail(HSTU_ERR_INVALID_ARG, "rows %lld < 0", (long long)a->rows);
    if (a->width <= 0 || a->width % 8 != 0 || a->width > 4096)
        return fail(HSTU_ERR_UNSUPPORTED, "width %d: a multiple of 8 up to 4096 is needed", a->width);
    if (!(a->eps > 0.0f) || !isfinite(a->eps)) return fail(HSTU_ERR_INVALID_ARG, "eps must be positive");
    if (!a->a || !a->u || !a->z) return fail(HSTU_ERR_INVALID_ARG, "a, u and z are required");
    if (!aligned16(a->a) || !aligned16(a->u) || !aligned16(a->z) || !aligned16(a->gamma) ||
        !aligned16(a->beta))
        return fail(HSTU_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    const int64_t as = a->a_stride ? a->a_stride : a->width, us = a->u_stride ? a->u_stride : a->width,
                  zs = a->z_stride ? a->z_stride : a->width;
    if (as < a->width || us < a->width || zs < a->width)
        return fail(HSTU_ERR_INVALID_ARG, "a row stride is shorter than its row");
    if (as % 8 || us % 8 || zs % 8) return fail(HSTU_ERR_INVALID_ARG, "row strides must be multiples of 8");
    if (a->z == a->a && zs != as) return fail(HSTU_ERR_INVALID_ARG, "in place needs z_stride == a_stride");
    return HSTU_OK;
}

void fill_norm_gate(const hstu_norm_gate_args_t *a, hstu::layer::NormGateParams &p) {
    p.a = (const uint16_t *)a->a;
    p.a_stride = a->a_stride ? a->a_stride : a->width;
    p.u = (const uint16_t *)a->u;
    p.u_stride = a->u_stride ? a->u_stride : a->width;
    p.gamma = a->gamma;
    p.beta = a->beta;
    p.eps = a->eps;
    p.z = (uint16_t *)a->z;
    p.z_stride = a->z_stride ? a->z_stride : a->width;
    p.M = a->rows;
    p.W = a->width;
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// widths of the layer: projection N1 = 2 H (dv + dqk), attention output H dv
struct LayerDims {
    int64_t n;
    int32_t n1, hv, hq;
    size_t aws;  // the attention's workspace
};

// projection [n][n1], attention output [n][H dv], the attention's own workspace
// (the persistent schedule's work queues)
size_t layer_ws(const LayerDims &d) {
    return align256((size_t)d.n * d.n1 * 2) + align256((size_t)d.n * d.hv * 2) + align256(d.aws);
}

// The argument blocks of the layer's four launches over the workspace ws:
// (a) Y = SiLU(X W1^T + b1) into ws, Y = [U | V | Q | K] per token;
// (b) the attention on views of Y (token stride n1) into A;
// (c) Z = Norm(A) * U in place; (d) out = X + Z W2^T + b2.
struct LayerLaunch {
    hstu_linear_args_t f1;
    hstu_fwd_args_t at;
    void *aws;  // the attention's workspace
    hstu_norm_gate_args_t ng;
    hstu_linear_args_t f2;
};

void layer_launch_args(const hstu_layer_args_t *args, const LayerDims &d, void *ws, LayerLaunch &ll) {
    const hstu_fwd_args_t &t = args->attn;
    uint16_t *y1 = (uint16_t *)ws;                                            // [n][n1]: U | V | Q | K
    uint16_t *ao = (uint16_t *)((char *)ws + align256((size_t)d.n * d.n1 * 2));  // [n][H dv]
    ll.f1 = hstu_linear_args_t{};
    ll.f1.dtype = t.dtype;
    ll.f1.rows = d.n;
    ll.f1.in_features = args->d_model;
    ll.f1.out_features = d.n1;
    ll.f1.x = args->x;
    ll.f1.w = args->w1;
    ll.f1.bias = args->b1;
    ll.f1.activation = HSTU_ACT_SILU;
    ll.f1.y = y1;

    ll.at = t;
    ll.at.v = y1 + d.hv;
    ll.at.q = y1 + 2 * d.hv;
    ll.at.k = y1 + 2 * d.hv + d.hq;
    ll.at.q_tok_stride = ll.at.k_tok_stride = ll.at.v_tok_stride = d.n1;
    ll.at.o = ao;
    ll.at.o_tok_stride = d.hv;
    ll.at.lse = nullptr;
    ll.aws = (char *)ao + align256((size_t)d.n * d.hv * 2);

    ll.ng = hstu_norm_gate_args_t{};
    ll.ng.dtype = t.dtype;
    ll.ng.rows = d.n;
    ll.ng.width = d.hv;
    ll.ng.a = ao;
    ll.ng.u = y1;
    ll.ng.u_stride = d.n1;
    ll.ng.gamma = args->ln_gamma;
    ll.ng.beta = args->ln_beta;
    ll.ng.eps = args->ln_eps;
    ll.ng.z = ao;

    ll.f2 = hstu_linear_args_t{};
    ll.f2.dtype = t.dtype;
    ll.f2.rows = d.n;
    ll.f2.in_features = d.hv;
    ll.f2.out_features = args->d_model;
    ll.f2.x = ao;
    ll.f2.w = args->w2;
    ll.f2.bias = args->b2;
    ll.f2.activation = HSTU_ACT_NONE;
    ll.f2.residual = args->x;
    ll.f2.y = args->out;
}

hstu_status_t check_layer(const hstu_layer_args_t *a, LayerDims &d) {
    hstu::api::clear_error();
    if (!a) return fail(HSTU_ERR_INVALID_ARG, "args is NULL");
    if (a->attn.cross) return fail(HSTU_ERR_UNSUPPORTED, "the layer is self-attention (attn.cross = 0)");
    if (a->d_model <= 0 || a->d_model % 64 != 0)
        return fail(HSTU_ERR_UNSUPPORTED, "d_model %d: a positive multiple of 64 is needed", a->d_model);
    if (!a->x || !a->w1 || !a->w2 || !a->out) return fail(HSTU_ERR_INVALID_ARG, "x, w1, w2 and out are required");
    if (!aligned16(a->x) || !aligned16(a->w1) || !aligned16(a->w2) || !aligned16(a->out) ||
        !aligned16(a->b1) || !aligned16(a->b2) || !aligned16(a->ln_gamma) || !aligned16(a->ln_beta))
        return fail(HSTU_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    if (!(a->ln_eps > 0.0f) || !isfinite(a->ln_eps)) return fail(HSTU_ERR_INVALID_ARG, "ln_eps must be positive");
    d.hv = a->attn.nhead * a->attn.hdim_v;
    d.hq = a->attn.nhead * a->attn.hdim_qk;
    d.n1 = 2 * (d.hv + d.hq);
    if (a->attn.nhead <= 0 || a->attn.hdim_v <= 0 || a->attn.hdim_qk <= 0)
        return fail(HSTU_ERR_INVALID_ARG, "nhead and head dims must be positive");
    if (d.hv > 4096) return fail(HSTU_ERR_UNSUPPORTED, "nhead * hdim_v = %d above 4096", d.hv);
    if (d.n1 > (1 << 22) || a->d_model > (1 << 22)) return fail(HSTU_ERR_UNSUPPORTED, "layer too wide");
    // the attention block exactly as hstu_layer_fwd will pass it (views of the
    // projection with its token stride), on placeholder buffers that are aligned
    // like the workspace's and never dereferenced: every check the attention would
    // make runs here, before the first launch
    hstu_fwd_args_t t = a->attn;
    const uintptr_t base = 256;
    t.v = (const void *)(base + 2 * (uintptr_t)d.hv);
    t.q = (const void *)(base + 4 * (uintptr_t)d.hv);
    t.k = (const void *)(base + 4 * (uintptr_t)d.hv + 2 * (uintptr_t)d.hq);
    t.q_tok_stride = t.k_tok_stride = t.v_tok_stride = d.n1;
    t.o = (void *)base;
    t.o_tok_stride = d.hv;
    t.lse = nullptr;
    hstu_status_t st = hstu::api::validate_fwd(&t);
    if (st != HSTU_OK) return st;
    d.n = hstu::api::rows_q(&a->attn);
    d.aws = hstu_fwd_workspace_size(&t, 1);
    // the two linear maps and the norm-gate exactly as the launches pass them
    // (placeholder buffers as above): a shape either kernel does not take (e.g.
    // H dv not a multiple of 64 for f2's input) fails here, before any launch
    LayerLaunch ll;
    layer_launch_args(a, d, (void *)base, ll);
    if ((st = check_linear(&ll.f1)) != HSTU_OK) return st;
    if ((st = check_norm_gate(&ll.ng)) != HSTU_OK) return st;
    if ((st = check_linear(&ll.f2)) != HSTU_OK) return st;
    return HSTU_OK;
}


}  // namespace

extern "C" {

hstu_status_t hstu_linear_fwd(const hstu_linear_args_t *args, void *hip_stream) {
    hstu_status_t st = check_linear(args);
    if (st != HSTU_OK) return st;
    if (args->rows == 0) return HSTU_OK;
    hstu::layer::LinearParams p;
    fill_linear(args, p);
    return hstu::api::hip_status(hstu::layer::launch_linear(p, args->dtype, (hipStream_t)hip_stream),
                                 "linear kernel launch");
}

hstu_status_t hstu_norm_gate_fwd(const hstu_norm_gate_args_t *args, void *hip_stream) {
    hstu_status_t st = check_norm_gate(args);
    if (st != HSTU_OK) return st;
    if (args->rows == 0) return HSTU_OK;
    hstu::layer::NormGateParams p;
    fill_norm_gate(args, p);
    return hstu::api::hip_status(hstu::layer::launch_norm_gate(p, args->dtype, (hipStream_t)hip_stream),
                                 "norm-gate kernel launch");
}

size_t hstu_layer_workspace_size(const hstu_layer_args_t *args) {
    LayerDims d;
    if (check_layer(args, d) != HSTU_OK) return 0;
    return layer_ws(d);
}

hstu_status_t hstu_layer_fwd(const hstu_layer_args_t *args, void *ws, size_t ws_bytes, void *hip_stream) {
    LayerDims d;
    hstu_status_t st = check_layer(args, d);
    if (st != HSTU_OK) return st;
    if (d.n == 0) return HSTU_OK;  // no tokens: nothing to launch, no workspace needed
    const size_t need = layer_ws(d);
    if (!ws || ws_bytes < need)
        return fail(HSTU_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
    if (((uintptr_t)ws & 255u) != 0) return fail(HSTU_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    LayerLaunch ll;
    layer_launch_args(args, d, ws, ll);
    if ((st = hstu_linear_fwd(&ll.f1, hip_stream)) != HSTU_OK) return st;
    if ((st = hstu_fwd(&ll.at, ll.aws, d.aws, hip_stream)) != HSTU_OK) return st;
    if ((st = hstu_norm_gate_fwd(&ll.ng, hip_stream)) != HSTU_OK) return st;
    return hstu_linear_fwd(&ll.f2, hip_stream);
}

}  // extern "C"

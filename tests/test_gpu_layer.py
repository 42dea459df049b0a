"""GPU parity of the HSTU layer kernels (HSTU explainer, "The layer, line by line")
against the oracle (oracle/layer.py): the linear map with each epilogue, the
gated layer norm, and whole layers (f1 + SiLU, the attention with mask and bias,
norm * gate, f2 + residual) through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import oracle.layer as OL
import recsys_attention_amd as hip
import workloads as W
from hip_runner import bits_to_device, compare, compare_rounded, layer_kwargs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hip._abi.load()  # raises when the library is missing: no silent fallback


def _log(msg):
    print(msg, flush=True)


def _host(t):
    return t.float().cpu().numpy()


# (M, K, N, dtype, activation, residual, x row stride padding)
LINEAR_CASES = [
    (1, 64, 8, "bf16", "silu", False, 0),
    (77, 512, 2048, "bf16", "silu", False, 0),
    (128, 128, 128, "fp16", "none", True, 0),
    (1000, 512, 136, "bf16", "none", True, 64),
    (4133, 1024, 512, "bf16", "silu", False, 8),
    (300, 256, 520, "fp16", "silu", True, 0),
    # enough rows for the persistent 256 x 256 tiles (two per CU: >= 512 of them),
    # ragged in M
    (33001, 512, 2048, "bf16", "silu", False, 0),
    (33001, 512, 2048, "fp16", "none", True, 8),
    # the layer's f2 shape class: two column tiles, residual (548 tiles)
    (70001, 512, 512, "bf16", "none", True, 0),
    # persistent kernel with fewer k-steps per tile than its prefetch depth, 7 column tiles
    (40000, 64, 1792, "bf16", "silu", True, 0),
]


@pytest.mark.parametrize("case", range(len(LINEAR_CASES)))
def test_linear(case):
    M, K, N, dt, act, use_res, pad = LINEAR_CASES[case]
    _log(f"linear M={M} K={K} N={N} {dt} act={act} residual={use_res} pad={pad}")
    rng = np.random.default_rng(900 + case)
    x32, xb = W.round_to_dtype(rng.standard_normal((M, K + pad)).astype(np.float32), dt)
    w32, wb = W.round_to_dtype((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32), dt)
    b = (0.1 * rng.standard_normal(N)).astype(np.float32)
    r32, rb = W.round_to_dtype(rng.standard_normal((M, N)).astype(np.float32), dt)
    x = bits_to_device(xb, dt)[:, :K]  # rows strided when pad > 0
    y = hip.hstu_linear(x, bits_to_device(wb, dt), torch.from_numpy(b).cuda(), activation=act,
                        residual=bits_to_device(rb, dt) if use_res else None)
    torch.cuda.synchronize()
    ref = OL.linear(x32[:, :K], w32, b)
    if act == "silu":
        ref = OL.silu(ref)
    if use_res:
        ref = ref + r32
    err = compare_rounded(_host(y), ref, dt, f"linear case {case}")
    _log(f"  max err {err:.3e}")


@pytest.mark.parametrize("width,inplace,affine,dt", [(64, False, True, "bf16"), (512, True, True, "bf16"),
                                                     (520, False, False, "fp16"), (4096, True, True, "bf16"),
                                                     (1024, False, True, "fp16"), (2048, False, True, "bf16")])
def test_norm_gate(width, inplace, affine, dt):
    _log(f"norm_gate width={width} inplace={inplace} affine={affine} {dt}")
    rng = np.random.default_rng(width + 7 * inplace)
    M = 333
    # attention outputs are small and offset: the normalisation must remove both
    a32, ab = W.round_to_dtype((0.01 * rng.standard_normal((M, width)) + 0.004).astype(np.float32), dt)
    u32, ub = W.round_to_dtype(rng.standard_normal((M, width + 16)).astype(np.float32), dt)
    g = (1 + 0.1 * rng.standard_normal(width)).astype(np.float32) if affine else None
    be = (0.1 * rng.standard_normal(width)).astype(np.float32) if affine else None
    a = bits_to_device(ab, dt)
    u = bits_to_device(ub, dt)[:, 8:8 + width]  # strided rows, offset start
    tg = None if g is None else torch.from_numpy(g).cuda()
    tb = None if be is None else torch.from_numpy(be).cuda()
    z = hip.hstu_norm_gate(a, u, tg, tb, 1e-6, out=a if inplace else None)
    torch.cuda.synchronize()
    ref = OL.norm_gate(a32, u32[:, 8:8 + width], g, be, 1e-6)
    err = compare_rounded(_host(z), ref, dt, f"norm_gate {width}", atol=2e-3)
    _log(f"  max err {err:.3e}")


def _layer_case(w, d_model, seed, rab=None):
    li = W.layer_inputs(w, d_model, seed)
    x, w1, b1, w2, b2, kw = layer_kwargs(w, li, rab)
    out = hip.hstu_layer(x, w1, b1, w2, b2, **kw)
    torch.cuda.synchronize()
    ref, _ = OL.hstu_layer(oracle.problem_of(w), li.x, li.w1, li.b1, li.w2, li.b2, li.gamma, li.beta,
                           li.eps, rab=rab)
    stats = compare(_host(out), ref, w.dtype, w.name)
    _log(f"  max err {stats['max_err']:.3e}, max |ref| {stats['scale']:.3e}")


@pytest.mark.parametrize("case", range(4))
def test_layer_random(case):
    """Whole layers: jagged and batched, every mask component, both bias terms or
    none, SiLU and softmax attention."""
    d, d_model, softmax, jagged, bias = [(128, 256, False, True, True), (64, 128, True, True, False),
                                         (128, 512, False, False, True), (96, 192, False, True, True)][case]
    w = W.random_workload(1000 + case, hdim_qk=d, hdim_v=d if d != 96 else 64, softmax=softmax,
                          jagged=jagged, max_uih=300, nhead=2)
    w.q = w.k = w.v = None
    rab = W.rab_inputs(w, 1100 + case, pos_len=256) if bias else None
    _log(f"layer case {case}: B={w.batch} H={w.nhead} d={w.hdim_qk}/{w.hdim_v} d_model={d_model} "
         f"tokens={w.total_q} softmax={softmax} bias={bias}")
    _layer_case(w, d_model, 1200 + case, rab)


def test_layer_edge_lengths():
    """Empty sequences, a one-token sequence, all-target and context-only sequences."""
    groups = [W.MaskGroup(local_len=3, context_len=4, minfull_len=2, attn_scale=0.0)]
    w = W.build("layer_edges", dtype="bf16", batch=6, nhead=2, hdim_qk=64, hdim_v=64, jagged=True,
                cross=False, causal=True, softmax=False, alpha=0.0, groups=groups,
                uih_q=[0, 0, 1, 0, 129, 3], targets=[0, 5, 0, 1, 2, 0], materialize=False)
    _layer_case(w, 128, 77, W.rab_inputs(w, 78, pos_len=16))


def test_layer_named_workload_sampled_rows():
    """The benchmark's layer workload at full size (83 302 tokens, d_model 512,
    4 heads of 128, both bias terms) in the benchmark's launch, against the oracle
    on sampled tokens: f1 over each sampled token's whole sequence, the attention
    of the sampled rows one by one, then the gated norm, f2 and the residual."""
    w, d_model, rab = W.layer_config("hstu_layer_bf16_d512_h4_causal_long")
    li = W.layer_inputs(w, d_model, W.LAYER_SEED)
    x, w1, b1, w2, b2, kw = layer_kwargs(w, li, rab)
    got = _host(hip.hstu_layer(x, w1, b1, w2, b2, **kw))
    H, dqk, dv = w.nhead, w.hdim_qk, w.hdim_v
    scale = 1.0 / max(max(w.uih_q), 1)  # the whole call's default attn_scale
    rng = np.random.default_rng(9)
    for b in rng.choice(w.batch, 3, replace=False):
        a, e = int(w.q_offsets[b]), int(w.q_offsets[b + 1])
        rows = np.sort(rng.choice(e - a, 6, replace=False))
        _log(f"sequence {b} ({e - a} tokens), rows {rows.tolist()}")
        sub = W.build("seq", dtype=w.dtype, batch=1, nhead=H, hdim_qk=dqk, hdim_v=dv, jagged=True,
                      cross=False, causal=True, softmax=False, alpha=0.0,
                      groups=[W.MaskGroup(g.local_len, g.context_len, g.minfull_len, scale)
                              for g in w.groups], uih_q=[w.uih_q[b]], targets=[w.targets[b]],
                      materialize=False)
        y = OL.silu(OL.linear(li.x[a:e], li.w1, li.b1))
        u, v, q, k = OL.split_uvqk(y, H, dqk, dv)
        rb = np.zeros(len(rows) * H, np.int32)
        rh = np.tile(np.arange(H, dtype=np.int32), len(rows))
        ri = np.repeat(rows, H).astype(np.int32)
        o, _ = oracle.rows_rab(oracle.problem_of(sub), q, k, v, rb, rh, ri,
                               timestamps=rab.timestamps[a:e], time_table=rab.time_table,
                               pos_table=rab.pos_table)
        z = OL.norm_gate(o.reshape(len(rows), H * dv), u[rows], li.gamma, li.beta, li.eps)
        ref = li.x[a + rows].astype(np.float64) + OL.linear(z, li.w2, li.b2)
        compare(got[a + rows], ref, w.dtype, f"sequence {b}")

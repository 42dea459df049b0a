"""GPU parity of the HIP HSTU forward against the CPU oracle (through the C ABI).

Every case draws seeded inputs (workloads), runs the HIP library on cuda:0 and
the oracle on the host from the same rounded bits, and compares elementwise with
the operator's tolerance (bf16: 2e-2 + 2e-2|ref|, fp16: 1e-2 + 1e-2|ref|) plus
scale-aware checks.  Visible-pair counts must match exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from hip_runner import DeviceInputs, compare, compare_lse, lse_tokens, o_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import recsys_attention_amd as hip
    hip._abi.load()  # raises when the library is missing: no silent fallback


def _log(msg):
    print(msg, flush=True)


def _check_full(w, num_splits=1, schedule=0, nthreads=0, elementwise=True):
    _log(f"case {w.name}: B={w.batch} H={w.nhead} d={w.hdim_qk} splits={num_splits} "
         f"schedule={schedule}")
    dev = DeviceInputs(w)
    res = dev.forward(num_splits=num_splits, schedule=schedule)
    torch.cuda.synchronize()
    o, lse = (res if w.softmax else (res, None))
    p = oracle.problem_of(w)
    o_ref, lse_ref, pairs = oracle.forward(p, w.q, w.k, w.v, nthreads=nthreads)
    stats = compare(o_tokens(w, o), o_ref, w.dtype, w.name, elementwise=elementwise)
    _log(f"  max err {stats['max_err']:.3e}, max |ref| {stats['scale']:.3e}, "
         f"worst row error / row max {stats['max_row_rel']:.2e}")
    if w.softmax:
        compare_lse(lse_tokens(w, lse), lse_ref, w.name)
    assert dev.count_pairs(schedule=schedule) == pairs
    return stats


@pytest.mark.parametrize("name", ["batched_silu_fp16_d64", "jagged_silu_bf16_d128_local",
                                  "group4_silu_bf16_d256"])
def test_config_parity(name):
    w = W.config(name)
    _check_full(w)


def test_config_parity_with_unit_attn_scale():
    """The configs' attn_scale makes |o| small; rerun them with attn_scale = 1 under the
    row-relative bound (the elementwise bound is stated for the configs' own scale)."""
    for name in ["batched_silu_fp16_d64", "jagged_silu_bf16_d128_local", "group4_silu_bf16_d256"]:
        w = W.config(name)
        for g in w.groups:
            g.attn_scale = 1.0
        _check_full(w, elementwise=False)


def test_cross_softmax_splitkv_config():
    w = W.config("cross_softmax_lse_splitkv16_bf16_d128")
    _check_full(w, num_splits=w.num_splits)
    _check_full(w, num_splits=1)


@pytest.fixture(scope="module")
def long_causal():
    """The full-size jagged causal workload (32 sequences of 1 k - 4 k events, 8 heads,
    d 128), on the device, with the oracle's whole output and pair count."""
    w = W.config("jagged_silu_bf16_d128_causal_long")
    _log(f"case {w.name}: full size, {w.total_q} tokens; oracle over every row")
    p = oracle.problem_of(w)
    o_ref, _, pairs = oracle.forward(p, w.q, w.k, w.v)
    return w, DeviceInputs(w), o_ref, pairs


@pytest.mark.parametrize("schedule", [0, 2])
def test_long_causal_config_full(long_causal, schedule):
    """Every output element of the long causal workload against the oracle, in the
    benchmark's launch (schedule 0: the persistent grid over planned per-XCD queues)
    and on the one-work-group-per-q-tile grid (2); exact visible-pair count."""
    w, dev, o_ref, pairs = long_causal
    _log(f"case {w.name}: schedule {schedule}")
    o = dev.forward(schedule=schedule)
    torch.cuda.synchronize()
    stats = compare(o_tokens(w, o), o_ref, w.dtype, f"{w.name} schedule {schedule}")
    _log(f"  max err {stats['max_err']:.3e}, max |ref| {stats['scale']:.3e}, "
         f"worst row error / row max {stats['max_row_rel']:.2e}")
    assert dev.count_pairs(schedule=schedule) == pairs


def test_long_causal_config_unit_attn_scale_full():
    """The long causal workload again with attn_scale = 1 (same mask), every element,
    under the row-relative and L2 bounds (the elementwise bound is stated for the
    workload's own scale, 1/4071)."""
    w1 = W.config("jagged_silu_bf16_d128_causal_long")
    for g in w1.groups:
        g.attn_scale = 1.0
    _check_full(w1, elementwise=False)


@pytest.mark.parametrize("seed", range(12))
def test_random_small_bf16_silu(seed):
    rng = np.random.default_rng(100 + seed)
    d = int(rng.choice([64, 128, 256]))
    w = W.random_workload(seed, dtype="bf16", hdim_qk=d, jagged=bool(seed % 2 == 0),
                          cross=bool(seed % 3 == 1), max_uih=int(rng.choice([40, 200, 400])))
    _check_full(w, schedule=1 + seed % 2)


@pytest.mark.parametrize("seed", range(8))
def test_random_small_softmax(seed):
    rng = np.random.default_rng(200 + seed)
    d = int(rng.choice([64, 128, 256]))
    dt = "fp16" if seed % 2 else "bf16"
    w = W.random_workload(50 + seed, dtype=dt, hdim_qk=d, softmax=True, jagged=bool(seed % 3),
                          cross=bool(seed % 4 == 3), max_uih=300)
    _check_full(w, num_splits=int(rng.choice([1, 2, 5])))


@pytest.mark.parametrize("seed", range(4))
def test_random_fp16_silu(seed):
    """fp16 SiLU at every head dim, jagged and batched (the d128 case runs the
    pipelined tile body)."""
    d = (64, 128, 256, 128)[seed]
    w = W.random_workload(400 + seed, dtype="fp16", hdim_qk=d, jagged=seed != 1, max_uih=500)
    _check_full(w)


@pytest.mark.parametrize("softmax", [False, True])
def test_groups_with_splitkv(softmax):
    """Group HSTU (per-group window, context, min-full tail and scale) through the
    split-KV path, against the oracle.  The scales stay in the operator's regime
    (the default 1/max UIH length, or 1/256): with attn_scale near 1 a long SiLU
    row is a small difference of terms summing to ~100 in magnitude, and the bf16
    rounding of P alone then moves it by more than the absolute bound (a CPU
    emulation of the kernel's arithmetic reproduces such a GPU value exactly)."""
    groups = [W.MaskGroup(3, 4, 2, 0.0), W.MaskGroup(0, 6, 0, 1.0 / 256), W.MaskGroup(40, 0, 9, 0.0)]
    w = W.build("groups_split", dtype="bf16", batch=6, nhead=2, hdim_qk=128, hdim_v=128, jagged=True,
                cross=False, causal=True, softmax=softmax, alpha=0.0, groups=groups,
                uih_q=[300, 17, 640, 0, 255, 129], targets=[3, 0, 12, 5, 1, 30], seed=17)
    _check_full(w, num_splits=4)


@pytest.mark.parametrize("dims", [(96, 96), (96, 64)])
@pytest.mark.parametrize("softmax", [False, True])
def test_hdim96(dims, softmax):
    """Head dims 96/96 and 96/64 (rows of 12 16-byte chunks, V narrower than Q/K):
    jagged self-attention with every mask component, then cross-attention through
    split-KV."""
    dqk, dv = dims
    w = W.random_workload(500 + dqk + dv + softmax, hdim_qk=dqk, hdim_v=dv, softmax=softmax,
                          max_uih=400)
    _check_full(w)
    w = W.random_workload(600 + dqk + dv + softmax, dtype="fp16", hdim_qk=dqk, hdim_v=dv,
                          softmax=softmax, cross=True, max_uih=300)
    _check_full(w, num_splits=3)


@pytest.mark.parametrize("softmax", [False, True])
def test_mfalcon_candidates_against_cached_history(softmax):
    """M-FALCON-style ranking (explainer "M-FALCON"): a user's history is a cached
    key/value sequence and the candidates are target queries of a cross-attention
    call with no query history.  Candidates never attend to each other, so scoring
    them all at once and in microbatches of 16 against the same cache gives the
    same rows bit for bit, and the oracle's values."""
    hist, cands = [700, 130, 1500], [37, 5, 64]
    groups = [W.MaskGroup(0, 0, 0, 1.0 / 512)]  # no query history to derive the scale from
    kw = dict(dtype="bf16", nhead=2, hdim_qk=128, hdim_v=128, jagged=True, cross=True, causal=True,
              softmax=softmax, alpha=0.0, groups=groups)
    w = W.build("mfalcon", batch=3, uih_q=[0, 0, 0], targets=cands, uih_kv=hist, seed=23, **kw)
    _check_full(w)
    res = DeviceInputs(w).forward()
    o_all = o_tokens(w, res[0] if softmax else res)
    lse_all = lse_tokens(w, res[1]) if softmax else None
    for b in range(w.batch):
        q0, k0, k1 = w.q_offsets[b], w.kv_offsets[b], w.kv_offsets[b + 1]
        for s0 in range(0, cands[b], 16):
            e0 = min(cands[b], s0 + 16)
            sub = W.build("mb", batch=1, uih_q=[0], targets=[e0 - s0], uih_kv=[hist[b]],
                          materialize=False, **kw)
            sub.q_bits = w.q_bits[q0 + s0:q0 + e0]
            sub.k_bits, sub.v_bits = w.k_bits[k0:k1], w.v_bits[k0:k1]
            r = DeviceInputs(sub).forward()
            torch.cuda.synchronize()
            assert np.array_equal(o_tokens(sub, r[0] if softmax else r), o_all[q0 + s0:q0 + e0]), (b, s0)
            if softmax:
                assert np.array_equal(lse_tokens(sub, r[1]), lse_all[q0 + s0:q0 + e0]), (b, s0)


@pytest.mark.parametrize("seed", range(4))
def test_random_non_causal(seed):
    w = W.random_workload(300 + seed, causal=False, softmax=bool(seed % 2), hdim_qk=128,
                          max_uih=150)
    _check_full(w)


@pytest.mark.parametrize("softmax", [False, True])
def test_splitkv_matches_unsplit(softmax):
    w = W.random_workload(11, softmax=softmax, hdim_qk=128, batch=3, nhead=2, max_uih=700,
                          groups=[W.MaskGroup(0, 6, 0, 0.0)])
    dev = DeviceInputs(w)
    base = dev.forward()
    base_o = o_tokens(w, base[0] if softmax else base)
    for ns in (1, 2, 3, 16, 64):
        _log(f"split {ns}")
        r = dev.forward(num_splits=ns)
        o = o_tokens(w, r[0] if softmax else r)
        compare(o, base_o, w.dtype, f"splits={ns}")
        if softmax:
            compare_lse(lse_tokens(w, r[1]), lse_tokens(w, base[1]), f"splits={ns}")


def test_schedules_agree_bitwise():
    """The work order moves work-groups, never the arithmetic of a row."""
    w = W.config("jagged_silu_bf16_d128_local")
    dev = DeviceInputs(w)
    a = dev.forward(schedule=1)
    for sched in (2,):
        b = dev.forward(schedule=sched)
        torch.cuda.synchronize()
        assert torch.equal(a, b), sched
        assert dev.count_pairs(schedule=sched) == dev.count_pairs(schedule=1)
    w2 = W.random_workload(11, softmax=True, hdim_qk=128, batch=3, nhead=2, max_uih=700,
                           groups=[W.MaskGroup(0, 6, 0, 0.0)])
    dev2 = DeviceInputs(w2)
    r1 = dev2.forward(num_splits=5, schedule=1)
    r3 = dev2.forward(num_splits=5, schedule=2)
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r3[0]) and torch.equal(r1[1], r3[1])


def test_jagged_equal_lengths_equals_batched():
    wb = W.random_workload(21, jagged=False, batch=3, nhead=2, hdim_qk=128, max_uih=190)
    wj = W.build("jag", dtype=wb.dtype, batch=3, nhead=2, hdim_qk=128, hdim_v=128, jagged=True,
                 cross=False, causal=True, softmax=False, alpha=0.0, groups=wb.groups,
                 uih_q=wb.uih_q, targets=wb.targets, materialize=False)
    wj.q, wj.k, wj.v = wb.q, wb.k, wb.v
    wj.q_bits, wj.k_bits, wj.v_bits = wb.q_bits, wb.k_bits, wb.v_bits
    ob = DeviceInputs(wb).forward()
    oj = DeviceInputs(wj).forward()
    torch.cuda.synchronize()
    assert torch.equal(ob.reshape(oj.shape), oj)


def test_group_equals_separate_calls():
    w = W.config("group4_silu_bf16_d256")
    # an explicit schedule (the per-item grid) on both sides: left to the library,
    # the small per-group calls would cut their long q-tiles into chunks, which
    # adds the same terms in another order
    full = o_tokens(w, DeviceInputs(w).forward(schedule=2))
    per = w.batch // len(w.groups)
    for g in range(len(w.groups)):
        bs = list(range(g * per, (g + 1) * per))
        sub = W.build("sub", dtype=w.dtype, batch=per, nhead=w.nhead, hdim_qk=w.hdim_qk,
                      hdim_v=w.hdim_v, jagged=True, cross=False, causal=True, softmax=False,
                      alpha=w.alpha, groups=[w.groups[g]], uih_q=[w.uih_q[b] for b in bs],
                      targets=[w.targets[b] for b in bs], materialize=False)
        t0, t1 = w.q_offsets[bs[0]], w.q_offsets[bs[-1] + 1]
        sub.q_bits, sub.k_bits, sub.v_bits = w.q_bits[t0:t1], w.k_bits[t0:t1], w.v_bits[t0:t1]
        # a single group's default scale uses the group's own max, which the full
        # call also uses, so the outputs must agree bit for bit
        got = o_tokens(sub, DeviceInputs(sub).forward(schedule=2))
        assert np.array_equal(got, full[t0:t1])


def test_edge_cases_jagged():
    """Empty sequences, all-target sequences, context longer than the sequence, one token."""
    groups = [W.MaskGroup(local_len=3, context_len=4, minfull_len=2, attn_scale=0.5)]
    for softmax in (False, True):
        w = W.build("edges", dtype="bf16", batch=6, nhead=2, hdim_qk=64, hdim_v=64, jagged=True,
                    cross=False, causal=True, softmax=softmax, alpha=0.0, groups=groups,
                    uih_q=[0, 0, 1, 0, 129, 3], targets=[0, 5, 0, 1, 2, 0], seed=5)
        # sequence 0 is only context (4 tokens); 1 has 4 context + 5 targets
        _check_full(w)


def test_fully_masked_rows_softmax():
    """Cross attention with U_q > U_kv and no context: leading rows see nothing:
    o = 0 and LSE = -inf there."""
    groups = [W.MaskGroup(0, 0, 0, 1.0)]
    w = W.build("masked", dtype="bf16", batch=2, nhead=2, hdim_qk=128, hdim_v=128, jagged=True,
                cross=True, causal=True, softmax=True, alpha=0.0, groups=groups,
                uih_q=[150, 40], targets=[0, 3], uih_kv=[20, 60], seed=9)
    _check_full(w)
    _check_full(w, num_splits=3)


def test_max_head_dim_and_ragged_tiles():
    """hdim 256 with lengths that leave ragged q and key tiles in every sequence."""
    groups = [W.MaskGroup(0, 6, 0, 0.0)]
    w = W.build("ragged256", dtype="bf16", batch=3, nhead=3, hdim_qk=256, hdim_v=256, jagged=True,
                cross=False, causal=True, softmax=False, alpha=0.0, groups=groups,
                uih_q=[1, 257, 300], targets=[31, 0, 7], seed=3)
    _check_full(w)


@pytest.mark.parametrize("softmax,local_len,context_len", [(False, 0, 6), (False, 5, 6), (True, 0, 6),
                                                           (True, 7, 0)])
def test_self_equals_cross_on_context_and_history_prefix(softmax, local_len, context_len):
    """Target keys are never attended (CK README "Masking": targets excluded from
    attention), so self-attention equals cross-attention whose keys and values are
    each sequence's [context | UIH] prefix, with the queries unchanged (the query
    history is then the whole key history: bottom-right alignment is the identity).
    The same key tiles in the same order: bit for bit."""
    groups = [W.MaskGroup(local_len, context_len, 4 if local_len else 0, 0.0)]
    kw = dict(dtype="bf16", batch=4, nhead=2, hdim_qk=128, hdim_v=128, jagged=True, causal=True,
              softmax=softmax, alpha=0.0, groups=groups)
    uih, tg = [300, 0, 129, 77], [5, 3, 0, 31]
    ws = W.build("self", cross=False, uih_q=uih, targets=tg, seed=61, **kw)
    wc = W.build("cross", cross=True, uih_q=uih, targets=tg, uih_kv=uih, materialize=False, **kw)
    keep = np.concatenate([np.arange(ws.q_offsets[b], ws.q_offsets[b] + context_len + uih[b])
                           for b in range(ws.batch)]).astype(np.int64)
    wc.q_bits = ws.q_bits
    wc.k_bits, wc.v_bits = ws.k_bits[keep], ws.v_bits[keep]
    assert len(keep) == wc.kv_offsets[-1]
    a = DeviceInputs(ws).forward()
    b = DeviceInputs(wc).forward()
    torch.cuda.synchronize()
    if softmax:
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    else:
        assert torch.equal(a, b)


@pytest.mark.parametrize("case", range(10))
def test_heavy_qtiles_cut_into_chunks(case):
    """Unsplit calls left to the library on a grid too small for the persistent
    schedule cut each sequence's last two q-tiles, when their key-tile lists are
    long (the min-full and target rows under a local window, the tail of a causal
    sequence), into chunks on separate work-groups, combined afterwards (CK README
    "Split-KV", applied per q-tile).  Cases 6 and 7 put the min-full and target
    rows across a q-tile boundary (1414 rows: 1402..1407 and 1408..1413); cases 8
    and 9 are batched (every sequence 1200 events and 6 targets).  Against the
    oracle, and against the uncut per-item grid (schedule 2) within the same
    tolerance; pair counts exact."""
    d, dv, softmax, L, M = [(128, 128, False, 5, 6), (128, 128, True, 5, 6), (256, 256, False, 0, 0),
                            (64, 64, True, 8, 16), (96, 64, False, 3, 9), (128, 128, False, 0, 0),
                            (128, 128, False, 5, 6), (128, 128, True, 5, 6), (128, 128, False, 5, 6),
                            (128, 128, True, 0, 0)][case]
    uih, tg, jagged = ([1402, 700, 90], [6, 3, 1], True) if case in (6, 7) else \
        (([1200] * 3, [6] * 3, False) if case >= 8 else ([1500, 700, 90], [6, 3, 1], True))
    groups = [W.MaskGroup(L, 6, M, 0.0)]
    w = W.build("heavy", dtype="bf16" if case % 2 == 0 else "fp16", batch=3, nhead=2, hdim_qk=d, hdim_v=dv,
                jagged=jagged, cross=False, causal=True, softmax=softmax, alpha=0.0, groups=groups,
                uih_q=uih, targets=tg, seed=300 + case)
    stats = _check_full(w, schedule=0)
    dev = DeviceInputs(w)
    a, b = dev.forward(schedule=0), dev.forward(schedule=2)
    torch.cuda.synchronize()
    oa = o_tokens(w, a[0] if softmax else a)
    ob = o_tokens(w, b[0] if softmax else b)
    compare(oa, ob, w.dtype, "cut vs uncut")
    if softmax:
        compare_lse(lse_tokens(w, a[1]), lse_tokens(w, b[1]), "cut vs uncut")


@pytest.mark.parametrize("name", ["batched_silu_fp16_d64", "jagged_silu_bf16_d128_local",
                                  "group4_silu_bf16_d256", "cross_softmax_lse_splitkv16_bf16_d128",
                                  "jagged_silu_bf16_d128_causal_long"])
def test_prepared_call_matches_binding(name):
    """hstu.prepare(): the argument block, output and workspace fixed once; every
    call (three in a row, then one on a side stream) gives bit for bit the output
    (and LSE) of the full binding call."""
    w = W.config(name)
    _log(f"case {name}: prepared call")
    dev = DeviceInputs(w)
    ref = dev.forward(num_splits=w.num_splits)
    pc = dev.prepare(num_splits=w.num_splits)
    side = torch.cuda.Stream()
    for i in range(4):
        if i == 3:
            side.wait_stream(torch.cuda.current_stream())
            got = pc(side)
            torch.cuda.current_stream().wait_stream(side)
        else:
            got = pc()
        torch.cuda.synchronize()
        if w.softmax:
            assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), i
        else:
            assert torch.equal(got, ref), i


@pytest.mark.parametrize("softmax", [False, True])
def test_most_groups_and_splits(softmax):
    """The largest group count (one sequence in each of 64 groups, every group
    with its own window, context, min-full tail and scale, the default scale
    among them) through split-KV with the largest split count (128: most
    chunks of the short sequences hold no key tile), then cross-attention over
    8 192 keys in 128 splits of one 64-key tile each."""
    from recsys_attention_amd import _abi
    ng, ns = _abi.HSTU_MAX_GROUPS, _abi.HSTU_MAX_SPLITS
    rng = np.random.default_rng(4242 + softmax)
    groups = [W.MaskGroup(int(rng.choice([0, 1, 5, 40])), int(rng.choice([0, 2, 7])),
                          int(rng.choice([0, 3, 30])), float(rng.choice([0.0, 1.0 / 128, 1.0 / 512])))
              for _ in range(ng)]
    w = W.build(f"groups{ng}_splits{ns}", dtype="bf16", batch=ng, nhead=2, hdim_qk=64, hdim_v=64,
                jagged=True, cross=False, causal=True, softmax=softmax, alpha=0.0, groups=groups,
                uih_q=rng.integers(0, 300, ng), targets=rng.integers(0, 6, ng), seed=4243 + softmax)
    _check_full(w, num_splits=ns)
    w = W.build(f"cross8192_splits{ns}", dtype="bf16", batch=2, nhead=2, hdim_qk=128, hdim_v=128,
                jagged=True, cross=True, causal=True, softmax=softmax, alpha=0.0,
                groups=[W.MaskGroup(0, 6, 0, 1.0 / 64)], uih_q=[64, 40], targets=[8, 3],
                uih_kv=[8192 - 6, 5000], seed=4245 + softmax)
    _check_full(w, num_splits=ns)


@pytest.mark.parametrize("name", ["jagged_silu_bf16_d128_local", "cross_softmax_lse_splitkv16_bf16_d128"])
def test_profiling_events_bracket_the_main_kernel(name):
    """The argument block's profiling hooks: the library records the caller's two
    events around its main kernel (forward, or split-KV), inside the call's own
    span, and the output is the same as without them."""
    w = W.config(name)
    dev = DeviceInputs(w)
    call = dev.prepare(num_splits=w.num_splits)
    _log(f"case {name}: profiling events")
    ref = call()
    ref = tuple(x.clone() for x in ref) if isinstance(ref, tuple) else ref.clone()
    s = torch.cuda.current_stream()
    b, e, t0, t1 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    b.record(s)
    e.record(s)
    torch.cuda.synchronize()
    t0.record(s)
    call.set_profiling_events(b, e)
    out = call()
    call.set_profiling_events(None, None)
    t1.record(s)
    torch.cuda.synchronize()
    if isinstance(out, tuple):
        assert all(torch.equal(x, y) for x, y in zip(out, ref))
    else:
        assert torch.equal(out, ref)
    k, step = b.elapsed_time(e), t0.elapsed_time(t1)
    assert 0.0 < k <= step, (k, step)
    assert t0.elapsed_time(b) >= 0.0 and e.elapsed_time(t1) >= 0.0

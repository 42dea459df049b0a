"""GPU parity of the relative attention bias (HSTU explainer, "The layer, line by
line" (b) and "The relative attention bias") against the oracle's biased forward.

Inputs: workloads.rab_inputs (int32 epoch-second timestamps whose gaps cover all
eleven time buckets, N(0, 1) float32 tables).  Same comparison rule as the
unbiased parity tests.
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


def _check(w, rab, num_splits=1, schedule=0):
    _log(f"case {w.name}: B={w.batch} H={w.nhead} d={w.hdim_qk}/{w.hdim_v} softmax={w.softmax} "
         f"splits={num_splits} time={rab.timestamps is not None} "
         f"P={None if rab.pos_table is None else rab.pos_table.shape[1]}")
    res = DeviceInputs(w).forward(num_splits=num_splits, schedule=schedule, rab=rab)
    torch.cuda.synchronize()
    o, lse = (res if w.softmax else (res, None))
    o_ref, lse_ref, _ = oracle.forward_rab(oracle.problem_of(w), w.q, w.k, w.v,
                                           timestamps=rab.timestamps, time_table=rab.time_table,
                                           pos_table=rab.pos_table)
    stats = compare(o_tokens(w, o), o_ref, w.dtype, w.name)
    _log(f"  max err {stats['max_err']:.3e}, max |ref| {stats['scale']:.3e}, "
         f"worst row error / row max {stats['max_row_rel']:.2e}")
    if w.softmax:
        compare_lse(lse_tokens(w, lse), lse_ref, w.name)
    return res


# (hdim_qk, hdim_v, softmax, dtype, jagged, terms, pos_len, shuffle, extremes)
CASES = [
    (128, 128, False, "bf16", True, "both", 64, False, False),
    (128, 128, True, "bf16", True, "both", 2048, True, False),
    (64, 64, False, "fp16", False, "time", None, True, True),
    (64, 64, True, "fp16", True, "pos", 1, False, False),
    (256, 256, False, "bf16", True, "both", 7, False, True),
    (256, 256, True, "bf16", False, "pos", 300, False, False),
    (96, 96, False, "bf16", True, "time", None, False, False),
    (96, 64, True, "fp16", True, "both", 100, True, False),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_bias_random(case):
    d, dv, softmax, dt, jagged, terms, P, shuffle, extremes = CASES[case]
    w = W.random_workload(700 + case, dtype=dt, hdim_qk=d, hdim_v=dv, softmax=softmax,
                          jagged=jagged, max_uih=400)
    rab = W.rab_inputs(w, 800 + case, time=terms in ("time", "both"),
                       pos_len=P if terms in ("pos", "both") else None, shuffle=shuffle,
                       extremes=extremes)
    _check(w, rab)


@pytest.mark.parametrize("softmax", [False, True])
def test_bias_with_groups_and_splitkv(softmax):
    """Group HSTU plus both bias terms through the split-KV path (the bias depends
    on absolute key positions, which each split must keep)."""
    groups = [W.MaskGroup(3, 4, 2, 0.0), W.MaskGroup(0, 6, 0, 1.0 / 256), W.MaskGroup(40, 0, 9, 0.0)]
    w = W.build("bias_groups_split", dtype="bf16", batch=6, nhead=2, hdim_qk=128, hdim_v=128,
                jagged=True, cross=False, causal=True, softmax=softmax, alpha=0.0, groups=groups,
                uih_q=[300, 17, 640, 0, 255, 129], targets=[3, 0, 12, 5, 1, 30], seed=19)
    rab = W.rab_inputs(w, 31, pos_len=500, shuffle=True)
    _check(w, rab, num_splits=4)
    _check(w, rab, num_splits=1)


def test_bias_long_sequences_full_positional_table():
    """Sequences longer than the largest positional table (2048 entries), so the
    clamp to the last entry is reached; non-causal rows see keys on both sides."""
    groups = [W.MaskGroup(0, 6, 0, 0.0)]
    for causal in (True, False):
        w = W.build("bias_long", dtype="bf16", batch=3, nhead=2, hdim_qk=128, hdim_v=128,
                    jagged=True, cross=False, causal=causal, softmax=False, alpha=0.0,
                    groups=groups, uih_q=[2600, 2047, 900], targets=[8, 1, 0], seed=41)
        _check(w, W.rab_inputs(w, 43, pos_len=2048))


def test_bias_schedules_agree_bitwise():
    """The work order moves work-groups, never the arithmetic of a biased row."""
    w = W.config("jagged_silu_bf16_d128_local")
    rab = W.rab_inputs(w, 53, pos_len=128)
    dev = DeviceInputs(w)
    a = dev.forward(schedule=1, rab=rab)
    b = dev.forward(schedule=2, rab=rab)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bias_named_workload_full():
    """The long causal workload (32 jagged sequences of 1 k - 4 k events, 8 heads,
    d 128) with both bias terms (2048-entry positional table), at full size in the
    benchmark's launch: every output element against the oracle's biased forward."""
    w = W.config("jagged_silu_bf16_d128_causal_long")
    _check(w, W.rab_inputs(w, 61, pos_len=2048))


@pytest.mark.parametrize("d,dv,softmax", [(128, 128, False), (128, 128, True), (64, 64, False), (256, 256, True)])
def test_zero_bias_tables_match_no_bias_bitwise(d, dv, softmax):
    """All-zero tables (both terms present) give bit for bit the output without
    bias: the bias enters the score MFMAs as their initial accumulator (divided by
    alpha), so zero tables leave every later step identical.  Long causal rows so
    that the d=128 SiLU case runs full key tiles through the pipelined body."""
    groups = [W.MaskGroup(0, 6, 0, 0.0)]
    w = W.build("bias_zero", dtype="bf16", batch=3, nhead=2, hdim_qk=d, hdim_v=dv, jagged=True,
                cross=False, causal=True, softmax=softmax, alpha=0.0, groups=groups,
                uih_q=[1500, 333, 70], targets=[7, 0, 3], seed=71)
    rab = W.rab_inputs(w, 73, pos_len=512)
    rab = W.RabInputs(rab.timestamps, np.zeros_like(rab.time_table), np.zeros_like(rab.pos_table))
    _log(f"case zero tables: d={d}/{dv} softmax={softmax}")
    dev = DeviceInputs(w)
    a = dev.forward(rab=rab)
    b = dev.forward()
    torch.cuda.synchronize()
    if softmax:
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    else:
        assert torch.equal(a, b)


@pytest.mark.parametrize("alpha,softmax", [(0.37, False), (-0.05, False), (0.37, True), (-0.05, True)])
def test_bias_explicit_alpha(alpha, softmax):
    """Explicit alpha, positive and negative: the bias enters the score MFMAs
    divided by alpha (1/alpha computed on the host), and alpha times the sum is
    the biased score, whatever alpha's sign.  Rows long enough for full key tiles
    (the pipelined body at hdim 128 with SiLU)."""
    groups = [W.MaskGroup(0, 6, 0, 0.0)]
    w = W.build("bias_alpha", dtype="bf16", batch=2, nhead=2, hdim_qk=128, hdim_v=128, jagged=True,
                cross=False, causal=True, softmax=softmax, alpha=alpha, groups=groups,
                uih_q=[900, 211], targets=[5, 2], seed=83)
    _check(w, W.rab_inputs(w, 89, pos_len=256, shuffle=True))

"""Seeded synthetic inputs for the HSTU attention forward operator.

This module is shared by the oracle-side tests and the HIP side.  It holds no
arithmetic of the operator itself: it only draws sequence lengths, target
counts and Q/K/V values from a seeded generator, rounds them once to the
storage dtype, and lays them out token-major.

Input recipe (every workload):
  * ``numpy.random.default_rng(seed)`` is created fresh per workload
    (default seed 13579, the CLI default of the CK example's argument list).
  * Draw order: UIH lengths -> target counts -> q -> k -> v.
  * Each tensor is drawn as float32 in token-major ``[tokens, H, D]`` order and
    rounded once, round-to-nearest-even, to fp16 or bf16.  The same bits go to
    the oracle (upcast) and to the GPU.
  * "uniform" means U[-1, 1] (the CK example's default init), "normal" N(0, 1)
    (its ``-norm_dist`` switch).

Physical sequence layout (CK example README, "Masking": physical length
formulas): a query sequence is ``[context | UIH | targets]`` with
``S_q = C + U_q + T``; self-attention keys have the same layout, cross-attention
keys are ``[context | UIH_kv]`` with ``S_kv = C + U_kv``.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

DEFAULT_SEED = 13579


@dataclasses.dataclass
class MaskGroup:
    """Per-group mask scalars (CK example README, "Attention variants": group HSTU)."""

    local_len: int
    context_len: int
    minfull_len: int
    attn_scale: float  # 0 -> 1 / (max UIH length of Q in the group)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str               # "fp16" | "bf16"
    batch: int
    nhead: int
    hdim_qk: int
    hdim_v: int
    jagged: bool
    cross: bool
    causal: bool
    softmax: bool
    alpha: float             # 0 -> 1/sqrt(hdim_qk)
    groups: List[MaskGroup]
    uih_q: List[int]
    targets: List[int]
    uih_kv: List[int]        # == uih_q for self-attention
    seqlen_q: List[int]      # physical, per sequence
    seqlen_kv: List[int]
    q_offsets: np.ndarray    # int64 [B+1] token offset of each sequence in q / o
    kv_offsets: np.ndarray   # int64 [B+1] token offset of each sequence in k / v
    num_splits: int = 1
    # token-major tensors: float32 values of the rounded inputs, and their raw bits
    q: Optional[np.ndarray] = None
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None

    @property
    def total_q(self) -> int:
        return int(self.q_offsets[-1])

    @property
    def total_kv(self) -> int:
        return int(self.kv_offsets[-1])

    @property
    def max_seqlen_q(self) -> int:
        return int(max(self.seqlen_q)) if self.seqlen_q else 0

    @property
    def max_seqlen_kv(self) -> int:
        return int(max(self.seqlen_kv)) if self.seqlen_kv else 0


# ----------------------------------------------------------------------------
# rounding (storage dtype); this is input preparation, not operator arithmetic
# ----------------------------------------------------------------------------

def round_to_dtype(x: np.ndarray, dtype: str):
    """Round float32 to fp16/bf16 (RNE). Returns (float32 values, uint16 bits)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        h = x.astype(np.float16)
        return h.astype(np.float32), h.view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        bits = u.astype(np.uint16)
        vals = (bits.astype(np.uint32) << 16).view(np.float32)
        return vals, bits
    raise ValueError(f"unknown dtype {dtype}")


def _draw(rng, shape, dist: str) -> np.ndarray:
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    if dist == "normal":
        return rng.standard_normal(size=shape, dtype=np.float32)
    raise ValueError(dist)


def _layout(uih_q, targets, uih_kv, groups, batch, cross, jagged, fixed_sq=None, fixed_skv=None):
    per = batch // len(groups)
    sq, skv = [], []
    for b in range(batch):
        c = groups[b // per].context_len
        sq.append(c + uih_q[b] + targets[b])
        skv.append(c + uih_kv[b] + (0 if cross else targets[b]))
    if not jagged:
        # batched: every sequence occupies the same physical length
        Sq = fixed_sq if fixed_sq is not None else max(sq)
        Skv = fixed_skv if fixed_skv is not None else (Sq if not cross else max(skv))
        assert all(s == Sq for s in sq), "batched mode needs equal physical q lengths"
        if not cross:
            Skv = Sq
        assert all(s == Skv for s in skv), "batched mode needs equal physical kv lengths"
    qo = np.zeros(batch + 1, np.int64)
    ko = np.zeros(batch + 1, np.int64)
    qo[1:] = np.cumsum(sq)
    ko[1:] = np.cumsum(skv)
    return sq, skv, qo, ko


def build(name, *, dtype, batch, nhead, hdim_qk, hdim_v, jagged, cross, causal, softmax,
          alpha, groups, uih_q, targets, uih_kv=None, dist="normal", seed=DEFAULT_SEED,
          rng=None, num_splits=1, materialize=True) -> Workload:
    """Assemble a workload from explicit lengths and draw its q/k/v."""
    if uih_kv is None:
        uih_kv = list(uih_q)
    uih_q = [int(u) for u in uih_q]
    targets = [int(t) for t in targets]
    uih_kv = [int(u) for u in uih_kv]
    sq, skv, qo, ko = _layout(uih_q, targets, uih_kv, groups, batch, cross, jagged)
    w = Workload(name=name, dtype=dtype, batch=batch, nhead=nhead, hdim_qk=hdim_qk,
                 hdim_v=hdim_v, jagged=jagged, cross=cross, causal=causal, softmax=softmax,
                 alpha=alpha, groups=groups, uih_q=uih_q, targets=targets, uih_kv=uih_kv,
                 seqlen_q=sq, seqlen_kv=skv, q_offsets=qo, kv_offsets=ko,
                 num_splits=num_splits)
    if materialize:
        if rng is None:
            rng = np.random.default_rng(seed)
        tq, tkv = int(qo[-1]), int(ko[-1])
        q32 = _draw(rng, (tq, nhead, hdim_qk), dist)
        k32 = _draw(rng, (tkv, nhead, hdim_qk), dist)
        v32 = _draw(rng, (tkv, nhead, hdim_v), dist)
        w.q, w.q_bits = round_to_dtype(q32, dtype)
        w.k, w.k_bits = round_to_dtype(k32, dtype)
        w.v, w.v_bits = round_to_dtype(v32, dtype)
    return w


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------

CONFIG_NAMES = (
    "batched_silu_fp16_d64",
    "jagged_silu_bf16_d128_local",
    "jagged_silu_bf16_d128_causal_long",
    "group4_silu_bf16_d256",
    "cross_softmax_lse_splitkv16_bf16_d128",
)


def config(name: str, seed: int = DEFAULT_SEED, materialize: bool = True) -> Workload:
    """The named workloads. Lengths drawn from the seed come first in the draw order."""
    rng = np.random.default_rng(seed)
    if name == "batched_silu_fp16_d64":
        # B=2, H=2, d=64, U=64, 4 targets per sequence, C=2, L=5, M=6, causal;
        # alpha = 1/sqrt(64), attn_scale = 1/64; physical length 70; uniform init.
        g = [MaskGroup(local_len=5, context_len=2, minfull_len=6, attn_scale=1.0 / 64)]
        return build(name, dtype="fp16", batch=2, nhead=2, hdim_qk=64, hdim_v=64,
                     jagged=False, cross=False, causal=True, softmax=False,
                     alpha=1.0 / 8.0, groups=g, uih_q=[64, 64], targets=[4, 4],
                     dist="uniform", rng=rng, materialize=materialize)
    if name == "jagged_silu_bf16_d128_local":
        # the CK README's jagged no-group example invocation
        U = [750, 730, 733, 860, 870, 788, 760, 821, 833, 779]
        T = [5, 5, 6, 6, 5, 6, 5, 6, 4, 6]
        g = [MaskGroup(local_len=5, context_len=6, minfull_len=6, attn_scale=0.0)]
        return build(name, dtype="bf16", batch=10, nhead=4, hdim_qk=128, hdim_v=128,
                     jagged=True, cross=False, causal=True, softmax=False, alpha=0.0,
                     groups=g, uih_q=U, targets=T, dist="normal", rng=rng,
                     materialize=materialize)
    if name == "jagged_silu_bf16_d128_causal_long":
        U = rng.integers(1024, 4096, size=32, endpoint=True)
        T = rng.integers(1, 32, size=32, endpoint=True)
        g = [MaskGroup(local_len=0, context_len=6, minfull_len=0, attn_scale=0.0)]
        return build(name, dtype="bf16", batch=32, nhead=8, hdim_qk=128, hdim_v=128,
                     jagged=True, cross=False, causal=True, softmax=False, alpha=0.0,
                     groups=g, uih_q=U, targets=T, dist="normal", rng=rng,
                     materialize=materialize)
    if name == "group4_silu_bf16_d256":
        U = rng.integers(256, 1024, size=16, endpoint=True)
        T = rng.integers(1, 16, size=16, endpoint=True)
        g = [MaskGroup(8, 4, 16, 1.0 / 1024), MaskGroup(32, 6, 0, 1.0 / 512),
             MaskGroup(0, 0, 0, 1.0 / 1024), MaskGroup(128, 8, 64, 1.0 / 256)]
        return build(name, dtype="bf16", batch=16, nhead=4, hdim_qk=256, hdim_v=256,
                     jagged=True, cross=False, causal=True, softmax=False, alpha=1.0 / 16,
                     groups=g, uih_q=U, targets=T, dist="normal", rng=rng,
                     materialize=materialize)
    if name == "cross_softmax_lse_splitkv16_bf16_d128":
        # batched cross attention: q [4, 6+64+8, 8, 128], k/v [4, 6+16384, 8, 128];
        # softmax with LSE, attn_scale = 1 (a convex combination is not shrunk).
        g = [MaskGroup(local_len=0, context_len=6, minfull_len=0, attn_scale=1.0)]
        return build(name, dtype="bf16", batch=4, nhead=8, hdim_qk=128, hdim_v=128,
                     jagged=False, cross=True, causal=True, softmax=True, alpha=0.0,
                     groups=g, uih_q=[64] * 4, targets=[8] * 4, uih_kv=[16384] * 4,
                     dist="normal", rng=rng, num_splits=16, materialize=materialize)
    raise KeyError(name)


def random_workload(seed: int, *, dtype="bf16", hdim_qk=128, hdim_v=None, batch=None,
                    nhead=None, jagged=True, cross=False, causal=True, softmax=False,
                    max_uih=300, groups=None, dist="normal", num_splits=1) -> Workload:
    """A small random case for sweeps: lengths, targets and mask scalars all from the seed."""
    rng = np.random.default_rng(seed)
    hdim_v = hdim_qk if hdim_v is None else hdim_v
    batch = int(rng.integers(1, 6)) if batch is None else batch
    nhead = int(rng.integers(1, 4)) if nhead is None else nhead
    if groups is None:
        groups = [MaskGroup(local_len=int(rng.choice([0, 1, 3, 17, 70])),
                            context_len=int(rng.choice([0, 1, 6, 40])),
                            minfull_len=int(rng.choice([0, 2, 9, 100])),
                            attn_scale=0.0)]
    if jagged:
        U = rng.integers(0, max_uih, size=batch, endpoint=True)
        T = rng.integers(0, 20, size=batch, endpoint=True)
    else:
        u = int(rng.integers(1, max_uih, endpoint=True))
        t = int(rng.integers(0, 20, endpoint=True))
        U, T = [u] * batch, [t] * batch
    if cross:
        if jagged:
            Ukv = rng.integers(0, 3 * max_uih, size=batch, endpoint=True)
        else:
            Ukv = [int(rng.integers(1, 3 * max_uih, endpoint=True))] * batch
    else:
        Ukv = None
    return build(f"random{seed}", dtype=dtype, batch=batch, nhead=nhead, hdim_qk=hdim_qk,
                 hdim_v=hdim_v, jagged=jagged, cross=cross, causal=causal, softmax=softmax,
                 alpha=0.0, groups=groups, uih_q=U, targets=T, uih_kv=Ukv, dist=dist, rng=rng,
                 num_splits=num_splits)


# ----------------------------------------------------------------------------
# relative attention bias inputs
# ----------------------------------------------------------------------------

# Gaps between consecutive events, in seconds: from same-second bursts to months,
# so that every time-gap bucket of the bias occurs within a sequence.
RAB_GAPS = (0, 1, 2, 4, 7, 20, 45, 100, 600, 2000, 5000, 40000, 200000, 900000, 3000000)
# relative frequencies (long gaps rarer; mean gap about 58000 s, so 8000 events
# stay well inside int32 epoch seconds)
RAB_GAP_WEIGHTS = (4, 4, 4, 4, 4, 4, 4, 4, 4, 4, 4, 3, 2, 1, 0.5)


@dataclasses.dataclass
class RabInputs:
    timestamps: Optional[np.ndarray]  # int32 [tokens of q], or None
    time_table: Optional[np.ndarray]  # float32 [H, 11], or None
    pos_table: Optional[np.ndarray]   # float32 [H, P], or None


def rab_inputs(w: Workload, seed: int, *, time=True, pos_len: Optional[int] = 64,
               shuffle=False, extremes=False) -> RabInputs:
    """Seeded bias inputs for a self-attention workload.

    Draw order: timestamps -> time table -> positional table, from
    ``numpy.random.default_rng(seed)``.  Timestamps of a sequence start at a
    random epoch second in [1.4e9, 1.6e9] and grow by gaps drawn from RAB_GAPS
    (shuffle: the sequence's timestamps are permuted, so gaps occur in both
    directions; extremes: the sequence's first two tokens are set to -2^31 and
    2^31 - 1).  Gaps are drawn with the relative frequencies RAB_GAP_WEIGHTS.  Tables are N(0, 1) float32 (the kernel's table dtype)."""
    rng = np.random.default_rng(seed)
    ts = None
    if time:
        ts = np.zeros(w.total_q, np.int64)
        for b in range(w.batch):
            a, e = int(w.q_offsets[b]), int(w.q_offsets[b + 1])
            n = e - a
            if n == 0:
                continue
            gp = np.asarray(RAB_GAP_WEIGHTS, np.float64)
            t = int(rng.integers(1_400_000_000, 1_600_000_000)) + np.concatenate(
                [[0], np.cumsum(rng.choice(RAB_GAPS, size=n - 1, p=gp / gp.sum()))])
            if shuffle:
                t = rng.permutation(t)
            if extremes and n >= 2:
                t[0], t[1] = -2 ** 31, 2 ** 31 - 1
            ts[a:e] = t
        assert ts.min() >= -2 ** 31 and ts.max() < 2 ** 31
        ts = ts.astype(np.int32)
    tt = rng.standard_normal((w.nhead, 11)).astype(np.float32) if time else None
    pt = rng.standard_normal((w.nhead, pos_len)).astype(np.float32) if pos_len else None
    return RabInputs(ts, tt, pt)


# ----------------------------------------------------------------------------
# HSTU layer inputs (the projections around the attention operator)
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class LayerInputs:
    d_model: int
    x: np.ndarray          # [tokens, d_model] float32 (rounded to the dtype)
    x_bits: np.ndarray
    w1: np.ndarray         # [2 H dv + 2 H dqk, d_model] (rounded)
    w1_bits: np.ndarray
    b1: np.ndarray         # [2 H dv + 2 H dqk] float32
    w2: np.ndarray         # [d_model, H dv] (rounded)
    w2_bits: np.ndarray
    b2: np.ndarray         # [d_model] float32
    gamma: np.ndarray      # [H dv] float32
    beta: np.ndarray       # [H dv] float32
    eps: float = 1e-6


def layer_inputs(w: Workload, d_model: int, seed: int) -> LayerInputs:
    """Seeded inputs of one layer over workload w's sequences (its q/k/v are not
    used: the layer makes them from X).  Draw order x -> w1 -> b1 -> w2 -> b2 ->
    gamma -> beta from ``numpy.random.default_rng(seed)``.  X ~ N(0, 1); weights
    N(0, 1/fan_in) (unit-variance pre-activations), rounded once to w.dtype like
    X; biases N(0, 0.1^2), gamma 1 + N(0, 0.1^2), beta N(0, 0.1^2) in float32."""
    rng = np.random.default_rng(seed)
    H, dqk, dv = w.nhead, w.hdim_qk, w.hdim_v
    n1 = 2 * H * (dv + dqk)
    x, xb = round_to_dtype(rng.standard_normal((w.total_q, d_model)).astype(np.float32), w.dtype)
    w1, w1b = round_to_dtype((rng.standard_normal((n1, d_model)) / np.sqrt(d_model)).astype(np.float32),
                             w.dtype)
    b1 = (0.1 * rng.standard_normal(n1)).astype(np.float32)
    w2, w2b = round_to_dtype((rng.standard_normal((d_model, H * dv)) / np.sqrt(H * dv)).astype(np.float32),
                             w.dtype)
    b2 = (0.1 * rng.standard_normal(d_model)).astype(np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(H * dv)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(H * dv)).astype(np.float32)
    return LayerInputs(d_model, x, xb, w1, w1b, b1, w2, w2b, b2, gamma, beta)


# the named HSTU layer workload: the long causal sequences with d_model 512 and
# 4 heads of 128 (H * d = d_model, as in the explainer's d = 512 example), both
# bias terms (positional table of 2048 entries)
LAYER_NAMES = ("hstu_layer_bf16_d512_h4_causal_long",)
LAYER_SEED = 2024
LAYER_RAB_SEED = 2025


def layer_config(name: str, seed: int = DEFAULT_SEED):
    """(attention Workload without q/k/v, d_model, RabInputs) of a named layer workload."""
    if name != "hstu_layer_bf16_d512_h4_causal_long":
        raise KeyError(name)
    w = config("jagged_silu_bf16_d128_causal_long", seed, materialize=False)
    w.name, w.nhead = name, 4
    return w, 512, rab_inputs(w, LAYER_RAB_SEED, pos_len=2048)

"""The oracle's own rounding: its single-precision build (scores, SiLU, softmax
sums and output accumulation in fp32) against the default double-precision build
on the same seeded inputs.  Their difference must stay a small fraction of the
parity tolerance the GPU path is held to (bf16: 2e-2 + 2e-2 |o_ref|, fp16:
1e-2 + 1e-2 |o_ref|), so that which of the two serves as the reference cannot
change a parity verdict; LSEs agree to well within the same margin."""
import numpy as np
import pytest

import oracle
import workloads as W

# the fp32 oracle's error may use at most this share of the parity tolerance
SHARE = 1e-3


def _tol(dtype):
    return 2e-2 if dtype == "bf16" else 1e-2


def _check(o32, o64, dtype, what):
    t = _tol(dtype)
    bound = SHARE * (t + t * np.abs(o64))
    err = np.abs(o32 - o64)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (what, float(err[worst]), float(bound[worst]), worst)


@pytest.fixture(scope="module")
def lib32():
    return oracle.load_fp32()


@pytest.mark.parametrize("name", ["batched_silu_fp16_d64", "jagged_silu_bf16_d128_local",
                                  "group4_silu_bf16_d256"])
def test_fp32_oracle_matches_fp64_on_named_workloads(name, lib32):
    w = W.config(name)
    p = oracle.problem_of(w)
    o64, _, n64 = oracle.forward(p, w.q, w.k, w.v)
    o32, _, n32 = oracle.forward(p, w.q, w.k, w.v, lib=lib32)
    assert n32 == n64
    _check(o32, o64, w.dtype, name)


def test_fp32_oracle_matches_fp64_on_split_kv_cross_rows(lib32):
    # rows of the 16 384-key cross-attention softmax workload (LSE included):
    # the longest sums of the named workloads
    w = W.config("cross_softmax_lse_splitkv16_bf16_d128")
    p = oracle.problem_of(w)
    rng = np.random.default_rng(5)
    n = 48
    rb = rng.integers(0, w.batch, n)
    rh = rng.integers(0, w.nhead, n)
    ri = np.array([rng.integers(0, w.seqlen_q[b]) for b in rb])
    o64, l64 = oracle.rows(p, w.q, w.k, w.v, rb, rh, ri)
    o32, l32 = oracle.rows(p, w.q, w.k, w.v, rb, rh, ri, lib=lib32)
    _check(o32, o64, w.dtype, "cross rows")
    assert np.max(np.abs(l32 - l64)) <= SHARE * _tol(w.dtype)


@pytest.mark.parametrize("seed", range(4))
def test_fp32_oracle_matches_fp64_on_random_problems_with_bias(seed, lib32):
    kw = [dict(softmax=False, jagged=True), dict(softmax=True, jagged=True),
          dict(softmax=False, jagged=False, causal=False), dict(softmax=True, jagged=False)][seed]
    w = W.random_workload(7100 + seed, hdim_qk=64, batch=4, nhead=2, max_uih=300, **kw)
    p = oracle.problem_of(w)
    o64, l64, _ = oracle.forward(p, w.q, w.k, w.v)
    o32, l32, _ = oracle.forward(p, w.q, w.k, w.v, lib=lib32)
    _check(o32, o64, w.dtype, f"random {seed}")
    if l64 is not None:
        fin = np.isfinite(l64)
        assert np.array_equal(fin, np.isfinite(l32))
        assert np.max(np.abs(l32[fin] - l64[fin]), initial=0.0) <= SHARE * _tol(w.dtype)
    rab = W.rab_inputs(w, 7200 + seed, pos_len=33)
    b64, _, _ = oracle.forward_rab(p, w.q, w.k, w.v, timestamps=rab.timestamps,
                                   time_table=rab.time_table, pos_table=rab.pos_table)
    b32, _, _ = oracle.forward_rab(p, w.q, w.k, w.v, timestamps=rab.timestamps,
                                   time_table=rab.time_table, pos_table=rab.pos_table, lib=lib32)
    _check(b32, b64, w.dtype, f"random {seed} with bias")


def test_fp32_oracle_is_a_different_build(lib32):
    # the two builds must not be the same library (a pin of this file's premise)
    w = W.config("jagged_silu_bf16_d128_local")
    p = oracle.problem_of(w)
    o64, _, _ = oracle.forward(p, w.q, w.k, w.v)
    o32, _, _ = oracle.forward(p, w.q, w.k, w.v, lib=lib32)
    assert not np.array_equal(o32, o64)
    assert np.array_equal(o32, o32.astype(np.float32).astype(np.float64))

"""Pins of the oracle's arithmetic (CPU only).

* The pages' worked example of un-normalised SiLU mass (HSTU explainer,
  section 3.4), stored under tests/golden/ with its citation.
* Special cases that reduce to library routines: with no context, no targets and
  no local window, the softmax variant is torch's scaled_dot_product_attention
  (causal or full) times attn_scale, and its LSE is torch.logsumexp; the SiLU
  variant is a masked dense product built from torch.nn.functional.silu.
* Structural identities: a grouped call == separate calls per group, the row
  API == the whole forward.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "silu_mass_example.json")


def _problem(B, H, D, Sq, Skv=None, *, T=0, C=0, L=0, M=0, cross=False, causal=True,
             softmax=False, alpha=0.0, a=1.0, Dv=None):
    Skv = Sq if Skv is None else Skv
    return oracle.Problem(batch=B, nhead=H, hdim_qk=D, hdim_v=Dv or D,
                          q_offsets=np.arange(B + 1) * Sq, kv_offsets=np.arange(B + 1) * Skv,
                          num_targets=[T] * B, cross=cross, causal=causal, softmax=softmax,
                          alpha=alpha, local_lens=[L], context_lens=[C], minfull_lens=[M],
                          attn_scales=[a])


def test_worked_example_silu_mass():
    """k identical keys at score 2: SiLU mass k*SiLU(2); softmax mass 1 (section 3.4)."""
    g = json.load(open(GOLDEN))
    D, U = 64, 24
    q = np.zeros((U, 1, D), np.float32)
    q[:, 0, 0] = 4.0
    k = q.copy()
    v = np.ones((U, 1, D), np.float32)
    alpha = 1.0 / 8.0  # alpha * (4 * 4) = 2
    tol = 0.5 * 10 ** -g["printed_decimals"]
    for L, kvis, key in ((2, 3, "mass_k3"), (19, 20, "mass_k20")):
        p = _problem(1, 1, D, U, L=L, alpha=alpha, a=1.0)
        o, _, _ = oracle.forward(p, q, k, v)
        row = o[U - 1, 0]  # the last row has L+1 visible keys
        assert np.allclose(row, row[0])
        assert abs(row[0] - g[key]) <= tol, (row[0], g[key])
        assert abs(row[0] / kvis / 2.0 - g["sigmoid_2"]) <= 0.5e-4
        ps = _problem(1, 1, D, U, L=L, alpha=alpha, a=1.0, softmax=True)
        os_, lse, _ = oracle.forward(ps, q, k, v)
        assert abs(os_[U - 1, 0, 0] - g["softmax_mass"]) <= tol
        assert abs(lse[U - 1, 0] - (2.0 + math.log(kvis))) < 1e-12
    o3 = 3 * 2 / (1 + math.exp(-2))
    o20 = 20 * 2 / (1 + math.exp(-2))
    assert round(o20 / o3, 1) == g["ratio_k20_over_k3"]


def _rand(shape, seed):
    return W.round_to_dtype(np.random.default_rng(seed).standard_normal(shape).astype(np.float32),
                            "bf16")[0]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D,Dv", [(64, 64), (32, 48)])
def test_softmax_equals_sdpa(causal, D, Dv):
    B, H, S = 2, 3, 37
    q, k, v = _rand((B * S, H, D), 1), _rand((B * S, H, D), 2), _rand((B * S, H, Dv), 3)
    alpha, a = 0.3, 0.7
    p = _problem(B, H, D, S, causal=causal, softmax=True, alpha=alpha, a=a, Dv=Dv)
    o, lse, pairs = oracle.forward(p, q, k, v)
    tq = torch.from_numpy(q).double().view(B, S, H, D).transpose(1, 2)
    tk = torch.from_numpy(k).double().view(B, S, H, D).transpose(1, 2)
    tv = torch.from_numpy(v).double().view(B, S, H, Dv).transpose(1, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                           scale=alpha) * a
    ref = ref.transpose(1, 2).reshape(B * S, H, Dv).numpy()
    assert np.abs(o - ref).max() < 1e-12
    s = alpha * (tq @ tk.transpose(-1, -2))
    if causal:
        s = s.masked_fill(~torch.ones(S, S, dtype=torch.bool).tril(), float("-inf"))
    ref_lse = torch.logsumexp(s, dim=-1).transpose(1, 2).reshape(B * S, H).numpy()
    assert np.abs(lse - ref_lse).max() < 1e-12
    assert pairs == B * H * (S * (S + 1) // 2 if causal else S * S)


def test_default_alpha_is_inverse_sqrt_hdim():
    B, H, D, S = 1, 2, 64, 20
    q, k, v = _rand((S, H, D), 4), _rand((S, H, D), 5), _rand((S, H, D), 6)
    o0, _, _ = oracle.forward(_problem(B, H, D, S, alpha=0.0), q, k, v)
    o1, _, _ = oracle.forward(_problem(B, H, D, S, alpha=1 / 8.0), q, k, v)
    assert np.array_equal(o0, o1)


@pytest.mark.parametrize("L,Dv", [(0, 32), (4, 32), (4, 48)])
def test_silu_equals_dense_masked_product(L, Dv):
    """No context/targets: o = a * (band ⊙ SiLU(alpha Q K^T)) V with torch's silu
    (also with a value head dim different from the query/key one)."""
    B, H, D, S = 2, 2, 32, 29
    q, k, v = _rand((B * S, H, D), 7), _rand((B * S, H, D), 8), _rand((B * S, H, Dv), 9)
    alpha, a = 0.4, 0.05
    o, _, pairs = oracle.forward(_problem(B, H, D, S, L=L, alpha=alpha, a=a, Dv=Dv), q, k, v)
    tq = torch.from_numpy(q).double().view(B, S, H, D).transpose(1, 2)
    tk = torch.from_numpy(k).double().view(B, S, H, D).transpose(1, 2)
    tv = torch.from_numpy(v).double().view(B, S, H, Dv).transpose(1, 2)
    band = torch.ones(S, S, dtype=torch.float64).tril()
    if L:
        band = band - torch.ones(S, S, dtype=torch.float64).tril(-L - 1)
    ref = a * (band * torch.nn.functional.silu(alpha * (tq @ tk.transpose(-1, -2)))) @ tv
    ref = ref.transpose(1, 2).reshape(B * S, H, Dv).numpy()
    assert np.abs(o - ref).max() < 1e-12
    assert pairs == B * H * int(band.sum())


def test_cross_attention_bottom_right_alignment():
    """Cross attention, no context/targets: the Q history is the tail of the KV history."""
    B, H, D, Sq, Skv = 1, 2, 16, 9, 23
    q, k, v = _rand((Sq, H, D), 10), _rand((Skv, H, D), 11), _rand((Skv, H, D), 12)
    p = _problem(B, H, D, Sq, Skv, cross=True, softmax=True, alpha=0.25, a=1.0)
    o, lse, _ = oracle.forward(p, q, k, v)
    m = torch.ones(Sq, Skv, dtype=torch.bool).tril(Skv - Sq)
    tq = torch.from_numpy(q).double().view(1, Sq, H, D).transpose(1, 2)
    tk = torch.from_numpy(k).double().view(1, Skv, H, D).transpose(1, 2)
    tv = torch.from_numpy(v).double().view(1, Skv, H, D).transpose(1, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=0.25)
    assert np.abs(o - ref.transpose(1, 2).reshape(Sq, H, D).numpy()).max() < 1e-12


def test_empty_rows():
    """A row with no visible key: o = 0 and, for softmax, LSE = -inf."""
    # C = 0, U = 0, T = 3: every row is a target row, every key a target key
    for softmax in (False, True):
        p = _problem(1, 1, 8, 3, T=3, softmax=softmax)
        q = np.ones((3, 1, 8), np.float32)
        o, lse, pairs = oracle.forward(p, q, q, q)
        assert pairs == 0 and not o.any()
        if softmax:
            assert np.all(np.isneginf(lse))
    # cross attention with U_q > U_kv and no context: the first rows see nothing
    p = _problem(1, 1, 8, 6, 2, cross=True, softmax=True)
    q = np.ones((6, 1, 8), np.float32)
    o, lse, _ = oracle.forward(p, q, q[:2], q[:2])
    assert np.all(np.isneginf(lse[:4])) and not o[:4].any() and np.isfinite(lse[4:]).all()


def test_rows_equal_forward():
    """The row API evaluates the same rule and arithmetic as the whole forward."""
    w = W.random_workload(3, jagged=True, batch=3, nhead=2, hdim_qk=32, max_uih=40,
                          groups=[W.MaskGroup(3, 2, 4, 0.0)])
    p = oracle.problem_of(w)
    o, _, _ = oracle.forward(p, w.q, w.k, w.v)
    rb, rh, ri = [0, 1, 2, 2], [1, 0, 1, 0], [0, 5, w.seqlen_q[2] - 1, 3]
    orow, _ = oracle.rows(p, w.q, w.k, w.v, rb, rh, ri)
    for n in range(4):
        tok = w.q_offsets[rb[n]] + ri[n]
        assert np.array_equal(orow[n], o[tok, rh[n]])


def test_group_call_equals_separate_calls():
    """Group HSTU: sequences of group g use group g's scalars (contiguous groups)."""
    groups = [W.MaskGroup(2, 1, 0, 0.5), W.MaskGroup(0, 3, 0, 0.0), W.MaskGroup(5, 0, 3, 0.25)]
    w = W.random_workload(5, batch=6, nhead=2, hdim_qk=16, max_uih=30, groups=groups)
    o, _, pairs = oracle.forward(oracle.problem_of(w), w.q, w.k, w.v)
    total = 0
    for g in range(3):
        bs = [2 * g, 2 * g + 1]
        sub = W.build("sub", dtype=w.dtype, batch=2, nhead=2, hdim_qk=16, hdim_v=16, jagged=True,
                      cross=False, causal=True, softmax=False, alpha=0.0, groups=[groups[g]],
                      uih_q=[w.uih_q[b] for b in bs], targets=[w.targets[b] for b in bs],
                      materialize=False)
        t0, t1 = w.q_offsets[bs[0]], w.q_offsets[bs[1] + 1]
        og, _, pg = oracle.forward(oracle.problem_of(sub), w.q[t0:t1], w.k[t0:t1], w.v[t0:t1])
        assert np.array_equal(o[t0:t1], og)
        total += pg
    assert total == pairs


def test_attn_scale_default_is_inverse_max_uih_of_group():
    groups = [W.MaskGroup(0, 2, 0, 0.0), W.MaskGroup(0, 2, 0, 0.0)]
    w = W.build("s", dtype="bf16", batch=4, nhead=1, hdim_qk=8, hdim_v=8, jagged=True,
                cross=False, causal=True, softmax=False, alpha=0.0, groups=groups,
                uih_q=[5, 9, 7, 3], targets=[1, 0, 2, 2], materialize=False)
    info, scale = oracle.seq_info(oracle.problem_of(w))
    assert list(info[:, 1]) == [5, 9, 7, 3]
    assert np.allclose(scale, [1 / 9, 1 / 9, 1 / 7, 1 / 7])

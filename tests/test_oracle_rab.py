"""Pins of the oracle's relative attention bias (HSTU explainer, "The layer, line
by line" (b) and "The relative attention bias"): the time-gap buckets against the
page's bucket table, and the biased forward against independent evaluations
(torch SDPA with an additive float mask; the dense SiLU product)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rab_time_buckets.json")


def _rand(shape, seed):
    return W.round_to_dtype(np.random.default_rng(seed).standard_normal(shape).astype(np.float32),
                            "bf16")[0]


def _problem(B, H, D, S, *, causal=True, softmax=False, alpha=0.0, a=1.0):
    return oracle.Problem(batch=B, nhead=H, hdim_qk=D, hdim_v=D, q_offsets=np.arange(B + 1) * S,
                          kv_offsets=np.arange(B + 1) * S, num_targets=[0] * B, cross=False,
                          causal=causal, softmax=softmax, alpha=alpha, local_lens=[0],
                          context_lens=[0], minfull_lens=[0], attn_scales=[a])


def test_time_buckets_match_the_table():
    g = json.load(open(GOLDEN))
    assert g["buckets"] == len(g["edges"])
    for d, b in g["cases"]:
        assert oracle.rab_bucket(d) == b, (d, b)
    for b, e in enumerate(g["edges"]):
        assert oracle.rab_bucket(e) == b
        if e > 0:
            assert oracle.rab_bucket(e - 1) == b - 1


def _bias(S, H, ts, time_tab, pos_tab, B):
    """The bias matrix [B, H, S, S] written out from the page's definition."""
    edges = np.array(json.load(open(GOLDEN))["edges"][1:], np.int64)
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    out = np.zeros((B, H, S, S))
    for b in range(B):
        t = ts[b * S:(b + 1) * S].astype(np.int64)
        bucket = np.searchsorted(edges, np.abs(t[:, None] - t[None, :]), side="right")
        for h in range(H):
            if pos_tab is not None:
                out[b, h] += pos_tab[h][np.minimum(np.abs(i - j), pos_tab.shape[1] - 1)]
            if time_tab is not None:
                out[b, h] += time_tab[h][bucket]
    return out


def _inputs(B, H, D, S, seed):
    q, k, v = _rand((B * S, H, D), seed), _rand((B * S, H, D), seed + 1), _rand((B * S, H, D), seed + 2)
    rng = np.random.default_rng(seed + 3)
    # increasing timestamps with gaps from seconds to weeks
    ts = np.cumsum(rng.choice([0, 1, 3, 20, 45, 200, 1000, 3000, 50000, 400000, 3000000],
                              size=B * S)).astype(np.int32)
    time_tab = rng.standard_normal((H, 11))
    pos_tab = rng.standard_normal((H, 9))
    return q, k, v, ts, time_tab, pos_tab


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("terms", ["pos", "time", "both"])
def test_softmax_with_bias_equals_sdpa(causal, terms):
    B, H, D, S = 2, 3, 32, 41
    q, k, v, ts, time_tab, pos_tab = _inputs(B, H, D, S, 11)
    tt = time_tab if terms in ("time", "both") else None
    pt = pos_tab if terms in ("pos", "both") else None
    alpha, a = 0.3, 0.7
    p = _problem(B, H, D, S, causal=causal, softmax=True, alpha=alpha, a=a)
    o, lse, _ = oracle.forward_rab(p, q, k, v, timestamps=ts if tt is not None else None,
                                   time_table=tt, pos_table=pt)
    bias = torch.from_numpy(_bias(S, H, ts, tt, pt, B))
    if causal:
        bias = bias.masked_fill(~torch.ones(S, S, dtype=torch.bool).tril(), float("-inf"))
    tq = torch.from_numpy(q).double().view(B, S, H, D).transpose(1, 2)
    tk = torch.from_numpy(k).double().view(B, S, H, D).transpose(1, 2)
    tv = torch.from_numpy(v).double().view(B, S, H, D).transpose(1, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=bias, scale=alpha) * a
    assert np.abs(o - ref.transpose(1, 2).reshape(B * S, H, D).numpy()).max() < 1e-12
    ref_lse = torch.logsumexp(alpha * (tq @ tk.transpose(-1, -2)) + bias, dim=-1)
    assert np.abs(lse - ref_lse.transpose(1, 2).reshape(B * S, H).numpy()).max() < 1e-12


def test_silu_with_bias_equals_dense_product():
    B, H, D, S = 2, 2, 32, 37
    q, k, v, ts, time_tab, pos_tab = _inputs(B, H, D, S, 21)
    alpha, a = 0.4, 0.05
    p = _problem(B, H, D, S, causal=True, softmax=False, alpha=alpha, a=a)
    o, _, _ = oracle.forward_rab(p, q, k, v, timestamps=ts, time_table=time_tab, pos_table=pos_tab)
    tq = torch.from_numpy(q).double().view(B, S, H, D).transpose(1, 2)
    tk = torch.from_numpy(k).double().view(B, S, H, D).transpose(1, 2)
    tv = torch.from_numpy(v).double().view(B, S, H, D).transpose(1, 2)
    s = alpha * (tq @ tk.transpose(-1, -2)) + torch.from_numpy(_bias(S, H, ts, time_tab, pos_tab, B))
    band = torch.ones(S, S, dtype=torch.float64).tril()
    ref = a * (band * torch.nn.functional.silu(s)) @ tv
    assert np.abs(o - ref.transpose(1, 2).reshape(B * S, H, D).numpy()).max() < 1e-12


def test_constant_positional_bias_only_shifts_softmax():
    """A constant bias leaves the softmax weights alone and shifts the LSE by it."""
    B, H, D, S = 1, 2, 32, 30
    q, k, v, _, _, _ = _inputs(B, H, D, S, 31)
    p = _problem(B, H, D, S, causal=True, softmax=True, alpha=0.2)
    o0, lse0, _ = oracle.forward(p, q, k, v)
    o1, lse1, _ = oracle.forward_rab(p, q, k, v, pos_table=np.full((H, 4), 2.5))
    assert np.abs(o1 - o0).max() < 1e-12
    assert np.abs(lse1 - lse0 - 2.5).max() < 1e-12


def test_cross_attention_is_rejected():
    p = oracle.Problem(batch=1, nhead=1, hdim_qk=32, hdim_v=32, q_offsets=[0, 4], kv_offsets=[0, 9],
                       num_targets=[0], cross=True, causal=True, softmax=False, alpha=0.0,
                       local_lens=[0], context_lens=[0], minfull_lens=[0], attn_scales=[1.0])
    q, k, v = _rand((4, 1, 32), 1), _rand((9, 1, 32), 2), _rand((9, 1, 32), 3)
    with pytest.raises(ValueError):
        oracle.forward_rab(p, q, k, v, pos_table=np.zeros((1, 3)))


def test_selected_rows_with_bias_equal_whole_forward():
    """The oracle's row-at-a-time entry (used for sampled parity at full size) gives
    the whole forward's rows, bias included."""
    B, H, D, S = 2, 3, 32, 41
    q, k, v, ts, time_tab, pos_tab = _inputs(B, H, D, S, 71)
    for softmax in (False, True):
        p = _problem(B, H, D, S, causal=True, softmax=softmax, alpha=0.3, a=0.5)
        o, lse, _ = oracle.forward_rab(p, q, k, v, timestamps=ts, time_table=time_tab,
                                       pos_table=pos_tab)
        rb, rh, ri = [0, 1, 1, 0], [2, 0, 1, 1], [40, 0, 17, 5]
        orow, lrow = oracle.rows_rab(p, q, k, v, rb, rh, ri, timestamps=ts, time_table=time_tab,
                                     pos_table=pos_tab)
        for n, (b, h, i) in enumerate(zip(rb, rh, ri)):
            assert np.array_equal(orow[n], o[b * S + i, h])
            if softmax:
                assert lrow[n] == lse[b * S + i, h]

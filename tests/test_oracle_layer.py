"""Pins of the oracle's HSTU layer (HSTU explainer, "The layer, line by line"):
an independent torch float64 evaluation of the whole layer on a causal special
case, the identities of a zero gate and a zero f2, the norm against torch's
layer_norm, and planted mistakes in the oracle's source that a pin must catch."""
import importlib.util
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.layer as OL
import workloads as W

SRC = os.path.join(os.path.dirname(oracle.__file__), "layer.py")


def _case(seed=3, B=2, S=24, H=2, D=16, d_model=32):
    """Causal self-attention without context or targets (every key up to the row),
    explicit attn_scale, and seeded layer inputs."""
    w = W.build("layer_pin", dtype="bf16", batch=B, nhead=H, hdim_qk=D, hdim_v=D, jagged=True,
                cross=False, causal=True, softmax=False, alpha=0.0,
                groups=[W.MaskGroup(0, 0, 0, 0.125)], uih_q=[S] * B, targets=[0] * B,
                materialize=False)
    li = W.layer_inputs(w, d_model, seed)
    return w, li


def _torch_layer(w, li, S, alpha):
    """The layer written with torch's own primitives, dense attention per sequence."""
    H, D = w.nhead, w.hdim_qk
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    x = t(li.x)
    y = F.silu(F.linear(x, t(li.w1), t(li.b1)))
    u, v, q, k = torch.split(y, [H * D, H * D, H * D, H * D], dim=1)
    outs = []
    for b in range(w.batch):
        sl = slice(b * S, (b + 1) * S)
        qb = q[sl].view(S, H, D).transpose(0, 1)
        kb = k[sl].view(S, H, D).transpose(0, 1)
        vb = v[sl].view(S, H, D).transpose(0, 1)
        s = alpha * (qb @ kb.transpose(-1, -2))
        p = F.silu(s) * torch.ones(S, S, dtype=torch.float64).tril() * w.groups[0].attn_scale
        outs.append((p @ vb).transpose(0, 1).reshape(S, H * D))
    o = torch.cat(outs)
    z = F.layer_norm(o, (H * D,), t(li.gamma), t(li.beta), li.eps) * u
    return (x + F.linear(z, t(li.w2), t(li.b2))).numpy()


def test_layer_equals_torch_dense():
    w, li = _case()
    out, mid = OL.hstu_layer(oracle.problem_of(w), li.x, li.w1, li.b1, li.w2, li.b2, li.gamma,
                             li.beta, li.eps)
    ref = _torch_layer(w, li, 24, 1.0 / np.sqrt(w.hdim_qk))
    # the attention oracle takes Q, K, V as float32 (one rounding, relative 6e-8)
    assert np.abs(out - ref).max() < 1e-6
    assert np.abs(out - li.x).max() > 0.1  # the block contributes


def test_zero_gate_leaves_residual_plus_f2_bias():
    w, li = _case(seed=5)
    H, D = w.nhead, w.hdim_v
    w1 = li.w1.copy()
    b1 = li.b1.copy()
    w1[:H * D] = 0.0
    b1[:H * D] = 0.0  # U = SiLU(0) = 0
    out, _ = OL.hstu_layer(oracle.problem_of(w), li.x, w1, b1, li.w2, li.b2, li.gamma, li.beta,
                           li.eps)
    assert np.array_equal(out, li.x.astype(np.float64) + li.b2.astype(np.float64))


def test_zero_f2_leaves_residual_plus_bias():
    w, li = _case(seed=7)
    out, _ = OL.hstu_layer(oracle.problem_of(w), li.x, li.w1, li.b1, np.zeros_like(li.w2), li.b2,
                           li.gamma, li.beta, li.eps)
    assert np.array_equal(out, li.x.astype(np.float64) + li.b2.astype(np.float64))


def test_norm_gate_matches_torch():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((9, 64)) * 1e-2 + 3e-3
    u = rng.standard_normal((9, 64))
    g, b = 1 + 0.1 * rng.standard_normal(64), 0.1 * rng.standard_normal(64)
    ref = F.layer_norm(torch.from_numpy(o), (64,), torch.from_numpy(g), torch.from_numpy(b), 1e-6)
    assert np.abs(OL.norm_gate(o, u, g, b, 1e-6) - (ref.numpy() * u)).max() < 1e-12


PINS = [test_layer_equals_torch_dense, test_zero_gate_leaves_residual_plus_f2_bias,
        test_zero_f2_leaves_residual_plus_bias, test_norm_gate_matches_torch]

MUTATIONS = {
    "residual_dropped": ("out = np.asarray(x, np.float64) + linear(z, w2, b2)", "out = linear(z, w2, b2)"),
    "split_uv_swapped": ("return (y[:, :a], y[:, a:b].reshape(n, H, dv)",
                         "return (y[:, a:b], y[:, :a].reshape(n, H, dv)"),
    "split_qk_swapped": ("y[:, b:c].reshape(n, H, dqk),\n            y[:, c:].reshape(n, H, dqk))",
                         "y[:, c:].reshape(n, H, dqk),\n            y[:, b:c].reshape(n, H, dqk))"),
    "eps_outside_sqrt": ("np.sqrt(var + eps)", "(np.sqrt(var) + eps)"),
    "no_mean_subtraction": ("y = (z - mean) / np.sqrt", "y = z / np.sqrt"),
    "sample_variance": ("((z - mean) ** 2).mean(axis=-1, keepdims=True)",
                        "((z - mean) ** 2).sum(axis=-1, keepdims=True) / (z.shape[-1] - 1)"),
    "gate_before_norm": ("return layer_norm(o, gamma, beta, eps) * np.asarray(u, np.float64)",
                         "return layer_norm(o * np.asarray(u, np.float64), gamma, beta, eps)"),
    "b1_dropped": ("y = silu(linear(x, w1, b1))", "y = silu(linear(x, w1))"),
    "silu_sign": ("return x / (1.0 + np.exp(-x))", "return x / (1.0 + np.exp(x))"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_in_layer_is_caught(name, monkeypatch):
    find, repl = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation anchor for {name} not unique"
    spec = importlib.util.spec_from_loader("oracle._layer_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    exec(compile(src.replace(find, repl), SRC, "exec"), mod.__dict__)
    monkeypatch.setattr(OL, "hstu_layer", mod.hstu_layer)
    monkeypatch.setattr(OL, "norm_gate", mod.norm_gate)
    caught = False
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught = True
            break
    assert caught, f"no pin fails for the planted mistake {name}"

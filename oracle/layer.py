"""CPU oracle of one HSTU layer around the attention operator (numpy, float64).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the smoke
check and the benchmark's cpu_baseline leg may use it; the product path never
imports it.

HSTU explainer, "The layer, line by line": given X [n, d_model] one layer is
  (a) pointwise projection: one linear map f1, SiLU, split four ways into
      U, V, Q, K;
  (b) spatial aggregation: the attention operator (pointwise SiLU, the
      functional mask, optionally the relative attention bias) on Q, K, V;
  (c) pointwise transformation: the attention output normalised, gated by U,
      mapped back by a second linear map f2, with a residual around the block.
The pages print the sub-layers' equations as stripped images, so the following
reading is taken (each part is the plainest one the text supports):
  * f1(X) = X W1^T + b1 with W1 [2 H dv + 2 H dqk, d_model]; SiLU elementwise;
    the split order along the features is [U | V | Q | K] (U and V H*dv wide,
    Q and K H*dqk wide), heads contiguous inside each part ([n, H, d]);
  * Norm is a layer norm over the H*dv features of a token, with the
    population variance, eps inside the square root, and a per-feature affine
    gamma, beta;
  * out = X + f2(Norm(A V) * U), f2(Z) = Z W2^T + b2 with W2 [d_model, H dv].
The attention step goes through the C oracle, which takes Q, K, V as float32:
they are rounded once there (relative 2^-24), the rest stays in float64.
Parity status: pinned by an independent torch float64 evaluation (torch's
linear, silu, layer_norm and a dense masked attention) on a causal special case,
and by the identities a zero gate and a zero f2 give (out = X + b2).
"""
from __future__ import annotations

import numpy as np

from . import forward, forward_rab


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(x) = x * sigmoid(x) = x / (1 + exp(-x))."""
    return x / (1.0 + np.exp(-x))


def linear(x: np.ndarray, w: np.ndarray, b=None) -> np.ndarray:
    """x W^T (+ b): x [n, in], w [out, in], b [out]."""
    y = np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
    if b is not None:
        y = y + np.asarray(b, np.float64)
    return y


def layer_norm(z: np.ndarray, gamma=None, beta=None, eps: float = 1e-6) -> np.ndarray:
    """Normalise each row to zero mean and unit (population) variance, then affine."""
    z = np.asarray(z, np.float64)
    mean = z.mean(axis=-1, keepdims=True)
    var = ((z - mean) ** 2).mean(axis=-1, keepdims=True)
    y = (z - mean) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, np.float64)
    if beta is not None:
        y = y + np.asarray(beta, np.float64)
    return y


def split_uvqk(y: np.ndarray, H: int, dqk: int, dv: int):
    """[n, 2 H dv + 2 H dqk] -> U [n, H dv], V [n, H, dv], Q [n, H, dqk], K [n, H, dqk]."""
    n = y.shape[0]
    a, b, c = H * dv, 2 * H * dv, 2 * H * dv + H * dqk
    assert y.shape[1] == c + H * dqk
    return (y[:, :a], y[:, a:b].reshape(n, H, dv), y[:, b:c].reshape(n, H, dqk),
            y[:, c:].reshape(n, H, dqk))


def norm_gate(o: np.ndarray, u: np.ndarray, gamma=None, beta=None, eps: float = 1e-6) -> np.ndarray:
    """Norm(A V) * U, both [n, H dv]."""
    return layer_norm(o, gamma, beta, eps) * np.asarray(u, np.float64)


def hstu_layer(p, x, w1, b1, w2, b2, gamma=None, beta=None, eps: float = 1e-6, rab=None,
               nthreads: int = 0):
    """One layer.  p: oracle.Problem of the attention (self-attention; its q_offsets
    delimit the sequences of X's rows).  rab: workloads.RabInputs-like object or None.
    Returns (out [n, d_model], intermediates dict with y (after SiLU), o, z)."""
    H, dqk, dv = p.H, p.Dqk, p.Dv
    y = silu(linear(x, w1, b1))
    u, v, q, k = split_uvqk(y, H, dqk, dv)
    if rab is None:
        o, _, _ = forward(p, q, k, v, nthreads=nthreads)
    else:
        o, _, _ = forward_rab(p, q, k, v, timestamps=rab.timestamps, time_table=rab.time_table,
                              pos_table=rab.pos_table, nthreads=nthreads)
    o = o.reshape(o.shape[0], H * dv)
    z = norm_gate(o, u, gamma, beta, eps)
    out = np.asarray(x, np.float64) + linear(z, w2, b2)
    return out, dict(y=y, o=o, z=z)

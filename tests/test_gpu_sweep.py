"""Randomised GPU parity sweep against the oracle: each seed draws one combination
of every feature (head-dim pair, dtype, SiLU / softmax, jagged / batched, self /
cross, causal or not, groups, mask scalars, split-KV, both bias terms), so feature
interactions that the targeted tests do not pair up are exercised too."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from hip_runner import DeviceInputs, compare, compare_lse, lse_tokens, o_tokens

pytestmark = pytest.mark.gpu

DIMS = [(64, 64), (96, 96), (96, 64), (128, 128), (256, 256)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import recsys_attention_amd as hip
    hip._abi.load()  # raises when the library is missing: no silent fallback


def _case(seed):
    rng = np.random.default_rng(5000 + seed)
    dqk, dv = DIMS[int(rng.integers(len(DIMS)))]
    softmax = bool(rng.integers(2))
    cross = bool(rng.integers(4) == 0)
    G = int(rng.choice([1, 2, 3]))
    B = G * int(rng.integers(1, 3))
    groups = [W.MaskGroup(local_len=int(rng.choice([0, 1, 5, 33])), context_len=int(rng.choice([0, 2, 9])),
                          minfull_len=int(rng.choice([0, 3, 40])),
                          attn_scale=float(rng.choice([0.0, 1.0 / 128])) if not softmax else
                          float(rng.choice([0.0, 1.0]))) for _ in range(G)]
    jagged = bool(rng.integers(3)) or cross
    if not jagged:  # batched: one physical length, so one context length
        groups = [W.MaskGroup(g.local_len, groups[0].context_len, g.minfull_len, g.attn_scale) for g in groups]
    if jagged:
        U = rng.integers(0, 300, size=B, endpoint=True)
        T = rng.integers(0, 12, size=B, endpoint=True)
    else:
        U, T = [int(rng.integers(1, 300))] * B, [int(rng.integers(0, 12))] * B
    Ukv = rng.integers(0, 500, size=B, endpoint=True) if cross else None
    w = W.build(f"sweep{seed}", dtype="fp16" if rng.integers(3) == 0 else "bf16", batch=B,
                nhead=int(rng.integers(1, 4)), hdim_qk=dqk, hdim_v=dv, jagged=jagged, cross=cross,
                causal=bool(rng.integers(5)), softmax=softmax, alpha=0.0, groups=groups, uih_q=U,
                targets=T, uih_kv=Ukv, seed=6000 + seed)
    splits = int(rng.choice([1, 1, 2, 7]))
    rab = None
    if not cross and rng.integers(2):
        rab = W.rab_inputs(w, 7000 + seed, time=bool(rng.integers(4)),
                           pos_len=int(rng.choice([1, 16, 300])), shuffle=bool(rng.integers(2)))
    return w, splits, rab


@pytest.mark.parametrize("seed", range(24))
def test_random_feature_mix(seed):
    w, splits, rab = _case(seed)
    print(f"case {w.name}: B={w.batch} H={w.nhead} d={w.hdim_qk}/{w.hdim_v} {w.dtype} softmax={w.softmax} "
          f"jagged={w.jagged} cross={w.cross} causal={w.causal} groups={len(w.groups)} splits={splits} "
          f"bias={rab is not None}", flush=True)
    res = DeviceInputs(w).forward(num_splits=splits, rab=rab)
    torch.cuda.synchronize()
    o, lse = (res if w.softmax else (res, None))
    p = oracle.problem_of(w)
    if rab is None:
        o_ref, lse_ref, _ = oracle.forward(p, w.q, w.k, w.v)
    else:
        o_ref, lse_ref, _ = oracle.forward_rab(p, w.q, w.k, w.v, timestamps=rab.timestamps,
                                               time_table=rab.time_table, pos_table=rab.pos_table)
    compare(o_tokens(w, o), o_ref, w.dtype, w.name)
    if w.softmax:
        compare_lse(lse_tokens(w, lse), lse_ref, w.name)

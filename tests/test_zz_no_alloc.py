"""The allocation-free entry point (hstu_fwd_splitkv_noalloc: split-KV partials and
work queues in the library's static scratch) against hstu_fwd_splitkv with a
caller workspace, through the C ABI.  Same kernels, same work order, same
arithmetic: the outputs must agree bit for bit, call after call, whatever an
earlier call left in the scratch."""
import numpy as np
import pytest
import torch

import oracle
import recsys_attention_amd as hip
import workloads as W
from hip_runner import DeviceInputs, compare, compare_lse, lse_tokens, o_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hip._abi.load()  # raises when the library is missing: no silent fallback


def _noalloc_vs_workspace(w, num_splits):
    print(f"case {w.name}: B={w.batch} H={w.nhead} d={w.hdim_qk} splits={num_splits} "
          f"softmax={w.softmax}", flush=True)
    dev = DeviceInputs(w)
    ref = dev.forward(num_splits=num_splits)
    ref_o, ref_lse = (ref if w.softmax else (ref, None))
    out = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_lse, float("nan")) if w.softmax else None
    res = hip.hstu_fwd_splitkv_noalloc(dev.q, dev.k, dev.v, num_splits, out=out, lse_out=lse,
                                       return_lse=w.softmax, **dev.kw)
    torch.cuda.synchronize()
    o, l = (res if w.softmax else (res, None))
    assert o.data_ptr() == out.data_ptr()
    assert torch.equal(o, ref_o)
    if w.softmax:
        assert torch.equal(l, ref_lse)
    return o, l


def test_noalloc_matches_workspace_entry_point_call_after_call():
    # 1: the split-KV cross-attention workload, 16 splits (about 20 MB of partials)
    big = W.config("cross_softmax_lse_splitkv16_bf16_d128")
    _noalloc_vs_workspace(big, big.num_splits)
    # 2: a smaller input right after it (stale partials of call 1 in the scratch),
    #    also against the oracle
    small = W.random_workload(31, softmax=True, hdim_qk=128, batch=3, nhead=2, max_uih=300,
                              groups=[W.MaskGroup(4, 6, 2, 0.0)])
    o, l = _noalloc_vs_workspace(small, 5)
    o_ref, lse_ref, _ = oracle.forward(oracle.problem_of(small), small.q, small.k, small.v)
    compare(o_tokens(small, o), o_ref, small.dtype, small.name)
    compare_lse(lse_tokens(small, l), lse_ref, small.name)
    # 3: the long causal workload unsplit (the persistent schedule's work queues in
    #    the scratch), then 4: a smaller SiLU problem split 3 ways
    _noalloc_vs_workspace(W.config("jagged_silu_bf16_d128_causal_long"), 1)
    tiny = W.random_workload(32, softmax=False, hdim_qk=64, batch=2, nhead=2, max_uih=90)
    o, _ = _noalloc_vs_workspace(tiny, 3)
    o_ref, _, _ = oracle.forward(oracle.problem_of(tiny), tiny.q, tiny.k, tiny.v)
    compare(o_tokens(tiny, o), o_ref, tiny.dtype, tiny.name)


def test_noalloc_rejects_problems_beyond_the_scratch():
    """A workspace need above the static scratch is an error before any launch."""
    w = W.config("cross_softmax_lse_splitkv16_bf16_d128")
    dev = DeviceInputs(w)
    out = torch.empty((w.batch, w.seqlen_q[0], w.nhead, w.hdim_v), dtype=torch.bfloat16,
                      device="cuda")
    lse = torch.empty((w.batch, w.nhead, w.seqlen_q[0]), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="static scratch"):
        hip.hstu_fwd_splitkv_noalloc(dev.q, dev.k, dev.v, 128, out=out, lse_out=lse,
                                     return_lse=True, **dev.kw)

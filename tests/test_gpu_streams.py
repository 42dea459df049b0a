"""Calls on a side stream (stream=): the binding enqueues the kernels there and
makes the call's own allocations (output, LSE, workspace) on that stream, so the
caching allocator cannot hand those blocks to other streams while the kernels
still run.  Each call runs on a side stream while the current stream allocates
and overwrites a large buffer at the same time; the results must equal the
current-stream results bit for bit."""
import pytest
import torch

import recsys_attention_amd as hip
import workloads as W
from hip_runner import DeviceInputs, layer_kwargs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hip._abi.load()


def _churn():
    # allocations and writes on the current stream while the side stream runs
    for _ in range(4):
        t = torch.empty(64 << 20, dtype=torch.int32, device="cuda")
        t.fill_(-1)
        del t


def _on_side(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    res = fn(side)
    _churn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("name", ["jagged_silu_bf16_d128_local", "cross_softmax_lse_splitkv16_bf16_d128",
                                  "jagged_silu_bf16_d128_causal_long"])
def test_forward_on_side_stream(name):
    """hstu_fwd (the per-item grid with cut q-tiles; the persistent schedule) and
    hstu_fwd_splitkv, each with the workspace the binding allocates."""
    w = W.config(name)
    print(f"case {name}: side stream", flush=True)
    dev = DeviceInputs(w)
    ref = dev.forward(num_splits=w.num_splits)
    torch.cuda.synchronize()
    rl = w.softmax
    if w.num_splits == 1:
        got = _on_side(lambda st: hip.hstu_fwd(dev.q, dev.k, dev.v, return_lse=rl, stream=st, **dev.kw))
    else:
        got = _on_side(lambda st: hip.hstu_fwd_splitkv(dev.q, dev.k, dev.v, w.num_splits, return_lse=rl,
                                                       stream=st, **dev.kw))
    if rl:
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    else:
        assert torch.equal(got, ref)


def test_layer_on_side_stream():
    """hstu_layer with its projection workspace allocated by the binding."""
    w = W.random_workload(1000, hdim_qk=128, hdim_v=128, jagged=True, max_uih=300, nhead=2)
    w.q = w.k = w.v = None
    li = W.layer_inputs(w, 256, 1200)
    rab = W.rab_inputs(w, 1100, pos_len=256)
    x, w1, b1, w2, b2, kw = layer_kwargs(w, li, rab)
    print(f"case layer: {w.total_q} tokens, side stream", flush=True)
    ref = hip.hstu_layer(x, w1, b1, w2, b2, **kw)
    torch.cuda.synchronize()
    got = _on_side(lambda st: hip.hstu_layer(x, w1, b1, w2, b2, stream=st, **kw))
    assert torch.equal(got, ref)

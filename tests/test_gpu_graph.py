"""The library's launch sequences captured into a HIP graph and replayed.

The planning kernel clears the persistent schedule's take counters and writes its
queues on every call (a kernel, not a memset), and every other buffer a call uses
is fully rewritten, so a captured call can be replayed.  Each replay, with the
program's own eager work between replays, must give bit for bit the eager
result (the persistent grid's item-to-work-group assignment varies from run to
run, but every item's arithmetic is fixed)."""
import pytest
import torch

import workloads as W
from hip_runner import DeviceInputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import recsys_attention_amd as hip
    hip._abi.load()


# the persistent schedule with its planning kernel (long causal), heavy q-tile
# chunks with their combine kernel (local window), split-KV with its combine
# (cross softmax with LSE), hdim 256 groups
@pytest.mark.parametrize("name", ["jagged_silu_bf16_d128_causal_long", "jagged_silu_bf16_d128_local",
                                  "cross_softmax_lse_splitkv16_bf16_d128", "group4_silu_bf16_d256"])
def test_graph_replays_equal_eager(name):
    w = W.config(name)
    print(f"case {name}: graph capture and replay", flush=True)
    dev = DeviceInputs(w)
    ref = dev.forward(num_splits=w.num_splits)
    torch.cuda.synchronize()
    ref = tuple(t.clone() for t in ref) if isinstance(ref, tuple) else (ref.clone(),)
    pc = dev.prepare(num_splits=w.num_splits)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pc(side)  # warm-up on the capture's stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = pc()
    out = out if isinstance(out, tuple) else (out,)
    for r in range(3):
        for t in out:
            t.fill_(0)  # eager work between replays; the replay must rewrite everything
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(a, b), f"replay {r}"
        dev.forward(num_splits=w.num_splits)  # an eager call in between
        torch.cuda.synchronize()

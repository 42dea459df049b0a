"""The persistent schedule (3: a resident grid taking work items from planned
per-XCD queues) against the one-work-group-per-item schedule (2).  Both run the
same per-item code on the same items (in different orders, and no item's result
depends on another's), so their outputs must agree bit for bit.  The other GPU
tests compare the default schedule with the oracle: 3 for grids of at least
2048 possible items (the binding provides the workspace), 2 below."""
import pytest
import torch

import workloads as W
from hip_runner import DeviceInputs
from test_gpu_sweep import _case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import recsys_attention_amd as hip
    hip._abi.load()  # raises when the library is missing: no silent fallback


def _both(dev, **kw):
    a = dev.forward(schedule=2, **kw)
    b = dev.forward(schedule=3, **kw)
    torch.cuda.synchronize()
    return (a if isinstance(a, tuple) else (a,)), (b if isinstance(b, tuple) else (b,))


def _same(a, b, what):
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.float32 else x.view(torch.int32),
                           y.view(torch.uint8) if y.dtype != torch.float32 else y.view(torch.int32)), what


@pytest.mark.parametrize("seed", range(12))
def test_persistent_matches_per_item_grid_random(seed):
    w, splits, rab = _case(seed)
    print(f"case {w.name}: d={w.hdim_qk}/{w.hdim_v} softmax={w.softmax} jagged={w.jagged} "
          f"cross={w.cross} splits={splits} bias={rab is not None}", flush=True)
    a, b = _both(DeviceInputs(w), num_splits=splits, rab=rab)
    _same(a, b, w.name)


@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_persistent_matches_per_item_grid_named(name):
    w = W.config(name)
    print(f"case {name}", flush=True)
    a, b = _both(DeviceInputs(w), num_splits=w.num_splits)
    _same(a, b, name)


def test_persistent_with_bias_long_causal():
    w = W.config("jagged_silu_bf16_d128_causal_long")
    rab = W.rab_inputs(w, 11, pos_len=2048)
    print("case jagged_silu_bf16_d128_causal_long + bias", flush=True)
    a, b = _both(DeviceInputs(w), rab=rab)
    _same(a, b, "long causal + bias")


def test_workspace_reused_across_calls():
    # the planning kernel rewrites the queues before every launch: a workspace
    # left with another call's queues (or garbage) serves the next one
    import recsys_attention_amd as hip
    w1, w2 = W.config("jagged_silu_bf16_d128_local"), W.config("group4_silu_bf16_d256")
    d1, d2 = DeviceInputs(w1), DeviceInputs(w2)
    need = max(hip.workspace_size(d.q, d.k, d.v, 1, **d.kw) for d in (d1, d2))
    ws = torch.full((need,), 0x5a, dtype=torch.uint8, device="cuda")
    print("case reuse", flush=True)
    outs = []
    for dev in (d1, d2, d1):
        outs.append(hip.hstu_fwd(dev.q, dev.k, dev.v, schedule=3, workspace=ws, **dev.kw))
    torch.cuda.synchronize()
    _same((outs[0],), (d1.forward(schedule=2),), "first call")
    _same((outs[1],), (d2.forward(schedule=2),), "second call")
    _same((outs[2],), (outs[0],), "third call")


def test_empty_and_tiny_grids():
    # fewer items than resident work-groups, and sequences without q-tiles
    w = W.build("tiny", dtype="bf16", batch=3, nhead=1, hdim_qk=128, hdim_v=128, jagged=True,
                cross=False, causal=True, softmax=False, alpha=0.0,
                groups=[W.MaskGroup(0, 0, 0, 0.0)], uih_q=[0, 5, 0], targets=[0, 1, 0], seed=3)
    print("case tiny", flush=True)
    a, b = _both(DeviceInputs(w))
    _same(a, b, "tiny")


def test_persistent_schedule_in_a_graph():
    # the planning kernel (not a memset node) rewrites the queues on every
    # replay; each replay, with eager work and synchronisations in between, must
    # reproduce the eager result bit for bit
    import recsys_attention_amd as hip
    w = W.config("jagged_silu_bf16_d128_causal_long")
    dev = DeviceInputs(w)
    eager = dev.forward(schedule=3)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    ws = torch.empty(hip.workspace_size(dev.q, dev.k, dev.v, 1, **dev.kw), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        hip.hstu_fwd(dev.q, dev.k, dev.v, schedule=3, out=out, workspace=ws, **dev.kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print("case graph capture", flush=True)
    with torch.cuda.graph(g):
        hip.hstu_fwd(dev.q, dev.k, dev.v, schedule=3, out=out, workspace=ws, **dev.kw)
    for r in range(4):
        out.zero_()
        ws.fill_(0x5a)  # garbage in the queues: the replay must rewrite them
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same((out,), (eager,), f"replay {r}")
        dev.forward(schedule=2)  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("batch,nhead", [(200, 4), (4200, 4)])
def test_many_pairs(batch, nhead):
    # more (b, h) pairs per XCD queue than one wave ranks (100: the bitonic sort
    # in LDS) and than are sorted at all (2100: the pairs keep their order)
    import numpy as np
    rng = np.random.default_rng(batch)
    U = rng.integers(0, 200 if batch < 1000 else 6, size=batch, endpoint=True)
    T = rng.integers(0, 3, size=batch, endpoint=True)
    w = W.build(f"pairs{batch}", dtype="bf16", batch=batch, nhead=nhead, hdim_qk=64, hdim_v=64,
                jagged=True, cross=False, causal=True, softmax=False, alpha=0.0,
                groups=[W.MaskGroup(0, 2, 0, 0.0)], uih_q=U, targets=T, seed=batch)
    print(f"case pairs{batch}", flush=True)
    a, b = _both(DeviceInputs(w))
    _same(a, b, w.name)


def test_two_streams_at_once():
    # calls that overlap in time, each with its own workspace, do not interfere
    import recsys_attention_amd as hip
    w1 = W.config("jagged_silu_bf16_d128_causal_long")
    w2 = W.build("streams2", dtype="bf16", batch=16, nhead=8, hdim_qk=128, hdim_v=128, jagged=True,
                 cross=False, causal=True, softmax=False, alpha=0.0,
                 groups=[W.MaskGroup(0, 6, 0, 0.0)], uih_q=[1500 + 97 * i for i in range(16)],
                 targets=[3] * 16, seed=77)
    d1, d2 = DeviceInputs(w1), DeviceInputs(w2)
    ref1, ref2 = d1.forward(schedule=2), d2.forward(schedule=2)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    print("case two streams", flush=True)
    for _ in range(3):
        with torch.cuda.stream(s1):
            o1 = hip.hstu_fwd(d1.q, d1.k, d1.v, schedule=3, **d1.kw)
        with torch.cuda.stream(s2):
            o2 = hip.hstu_fwd(d2.q, d2.k, d2.v, schedule=3, **d2.kw)
        outs.append((o1, o2))
    torch.cuda.synchronize()
    for o1, o2 in outs:
        _same((o1,), (ref1,), "stream 1")
        _same((o2,), (ref2,), "stream 2")


def _expected_queues(w, per_queue):
    """The planning kernel's contract, written out: queue x holds the (b, h) pairs
    with b*H + h = x (mod 8), longest first (cost = q-tiles x keys, ties by pair
    index; in natural order when a queue has more than 2048 pairs), each pair's
    q-tiles from the last to the first, then "no item" entries."""
    import numpy as np
    off = np.asarray(w.q_offsets, dtype=np.int64)
    lens = off[1:] - off[:-1]
    BH = w.batch * w.nhead
    bh_pad = (BH + 7) // 8 * 8
    queues, counts = [], []
    for x in range(8):
        pairs = []
        for k in range((bh_pad - x + 7) // 8):
            bh = x + 8 * k
            if bh >= BH:
                continue
            S = int(lens[bh // w.nhead])
            nq = (S + 127) // 128
            pairs.append((k, bh, nq, float(np.float32(nq) * np.float32(S))))
        if bh_pad // 8 <= 2048:
            pairs.sort(key=lambda t: (-t[3], t[0]))
        ent = [bh | (qt << 8) << 32 for _, bh, nq, _ in pairs for qt in range(nq - 1, -1, -1)]
        counts.append(len(ent))
        queues.append(np.array(ent + [0xFFFFFFFF] * (per_queue - len(ent)), dtype=np.uint64))
    return queues, counts


@pytest.mark.parametrize("batch,nhead,maxlen", [(7, 3, 700), (32, 8, 3000), (200, 4, 300), (4200, 4, 6)])
def test_planned_queues_hold_every_item_once_in_order(batch, nhead, maxlen):
    # the queues the planning kernel leaves in the workspace, entry by entry
    # (the forward kernel only advances the take counters in the header)
    import numpy as np
    import recsys_attention_amd as hip
    rng = np.random.default_rng(batch + nhead)
    U = rng.integers(0, maxlen, size=batch, endpoint=True)
    T = rng.integers(0, 3, size=batch, endpoint=True)
    w = W.build(f"queues{batch}", dtype="bf16", batch=batch, nhead=nhead, hdim_qk=64, hdim_v=64,
                jagged=True, cross=False, causal=True, softmax=False, alpha=0.0,
                groups=[W.MaskGroup(0, 2, 0, 0.0)], uih_q=U, targets=T, seed=batch)
    dev = DeviceInputs(w)
    need = hip.workspace_size(dev.q, dev.k, dev.v, 1, **dev.kw)
    ws = torch.full((need,), 0x5a, dtype=torch.uint8, device="cuda")
    print(f"case queues{batch}x{nhead}", flush=True)
    hip.hstu_fwd(dev.q, dev.k, dev.v, schedule=3, workspace=ws, **dev.kw)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    header = raw[:256].view(np.uint32)
    # one entry per possible item (8 queues of (b, h) pairs x q-tiles); the
    # workspace may hold more after the queues (a small unsplit grid: room for
    # cutting heavy q-tiles when the library picks the schedule)
    per_queue = (batch * nhead + 7) // 8 * ((w.max_seqlen_q + 127) // 128)
    assert need >= 256 + 64 * per_queue
    lists = raw[256:256 + 64 * per_queue].view(np.uint64).reshape(8, per_queue)
    queues, counts = _expected_queues(w, per_queue)
    for x in range(8):
        assert int(header[8 + x]) == counts[x], f"queue {x} count"
        assert np.array_equal(lists[x], queues[x]), f"queue {x} entries"

"""Benchmark of the HSTU attention forward on one MI355X.

A step is one call of the forward operator over the whole workload (every
sequence and head): the mask, the non-linearity and both products run inside
the timed kernels; inputs are resident in HBM before timing starts.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--schedule S]
                    [--rab none|pos|time|both]

Prints one JSON line: effective TFLOP/s counting 2 * (hdim_qk + hdim_v) FLOPs
per visible (b, h, i, j) pair over the median of the per-step HIP-event times
(minimum, mean and the shader clock are logged beside it), the roofline of the
dominant kernel (its own duration from events the library records around its
launch, in a second loop of the same steps), and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)

METRIC = "HSTU fwd effective TFLOP/s (visible pairs) and % of bf16 MFMA peak, 1 GPU"
DEFAULT_WORKLOAD = "jagged_silu_bf16_d128_causal_long"
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
RAB_SEED = 61          # bias inputs of the --rab runs
RAB_POS_LEN = 2048     # positional table entries (the largest the kernel takes)
KERNEL_SOURCES = [os.path.join(ROOT, "recsys_attention_amd", "csrc", f)
                  for f in ("hstu_fwd_kernels.hip", "hstu_plan.h", "hstu_params.h")]


def cpu_model() -> str:
    """The host CPU's model name (the oracle baseline runs there)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def device_info(torch) -> dict:
    """Name, architecture and compute units of cuda:0 (as the runtime reports them)."""
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""), "compute_units": pr.multi_processor_count}


def sclk_reader(torch):
    """A function returning the shader clock (MHz) the driver reports as current for
    cuda:0 (sysfs pp_dpm_sclk of its PCI device), or None where it is not readable."""
    try:
        pr = torch.cuda.get_device_properties(0)
        path = (f"/sys/bus/pci/devices/{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:"
                f"{pr.pci_device_id:02x}.0/pp_dpm_sclk")
        open(path).read()
    except (OSError, AttributeError):
        return lambda: None

    def read():
        try:
            for line in open(path):
                if line.rstrip().endswith("*"):
                    return int("".join(c for c in line.split(":", 1)[1] if c.isdigit()))
        except (OSError, ValueError, IndexError):
            pass
        return None
    return read


def timed_steps(torch, step, steps: int, warmup: int, warmup_s: float, stream):
    """W warm-up steps, then more until warmup_s seconds of back-to-back launches
    have passed (the first launches after idle run at a lower clock), then exactly
    `steps` steps with a HIP event pair around each one, on the launch stream,
    bracketed by device synchronisations.  The shader clock is sampled while the
    timed steps run.  Returns per-step milliseconds and a record of the run."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    extra, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < warmup_s:
        for _ in range(20):
            step()
        extra += 20
        torch.cuda.synchronize()
    read_clock = sclk_reader(torch)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(steps):
        step()
        evs[i + 1].record(stream)
    clocks = [read_clock()]
    torch.cuda.synchronize()
    clocks.append(read_clock())
    wall = time.perf_counter() - t0
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    per_sorted = sorted(per)
    med = per_sorted[steps // 2] if steps % 2 else 0.5 * (per_sorted[steps // 2 - 1] + per_sorted[steps // 2])
    rec = {"ms_median": round(med, 4), "ms_min": round(per_sorted[0], 4),
           "ms_mean": round(sum(per) / steps, 4), "ms_max": round(per_sorted[-1], 4),
           "ms_total_timed": round(evs[0].elapsed_time(evs[-1]), 4),
           "warmup_extra_steps": extra, "warmup_s": warmup_s,
           "sclk_mhz_during": clocks[0], "sclk_mhz_after": clocks[1], "wall_s_timed": round(wall, 3)}
    return med, rec


def main_kernel_times(torch, call, steps: int, stream):
    """Durations of the step's main kernel alone (the forward kernel, or the split
    kernel of a split-KV step): a loop of its own after the timed one, in which the
    library records one event pair per step right around that kernel's launch (the
    argument block's profiling hooks), on the launch stream.  Returns the median
    milliseconds and a record of the run."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for b, e in evs:  # an event exists once it has been recorded
        b.record(stream)
        e.record(stream)
    torch.cuda.synchronize()
    for b, e in evs:
        call.set_profiling_events(b, e)
        call()
    call.set_profiling_events(None, None)
    torch.cuda.synchronize()
    per = sorted(b.elapsed_time(e) for b, e in evs)
    med = per[steps // 2] if steps % 2 else 0.5 * (per[steps // 2 - 1] + per[steps // 2])
    return med, {"ms_median": round(med, 4), "ms_min": round(per[0], 4),
                 "ms_mean": round(sum(per) / steps, 4), "ms_max": round(per[-1], 4)}


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--warmup-s", type=float, default=1.0,
                    help="after the --warmup steps, keep warming up until this many seconds "
                         "of back-to-back launches have passed (clock ramp)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--launch", choices=("prepared", "binding"), default="prepared",
                    help="prepared: hstu.prepare() once, then one C call per step; binding: "
                         "the full hstu_fwd binding (checks, allocations) every step")
    ap.add_argument("--schedule", type=int, default=0)
    ap.add_argument("--splits", type=int, default=0, help="0: the workload's own split count")
    ap.add_argument("--rab", choices=("none", "pos", "time", "both"), default="none",
                    help="relative attention bias terms (self-attention workloads)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample (0 disables cpu_baseline)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a device copy of this size (counter calibration) and exit")
    return ap.parse_args()


def copy_probe(mib: int):
    """A plain device-to-device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "launches": 3}), flush=True)


def cpu_baseline(w, budget_s: float, rab=None):
    """The oracle, untuned, on whole sequences of the workload (all heads) until
    about budget_s of wall time; returns TFLOP/s over the visible pairs done.
    rab: the workload's bias inputs (workloads.RabInputs) or None."""
    import numpy as np

    import oracle
    import workloads as W
    lib = oracle.load()
    done_pairs, secs, seqs = 0, 0.0, 0
    order = list(range(w.batch))
    for b in order:
        sub = W.build("sample", dtype=w.dtype, batch=1, nhead=w.nhead, hdim_qk=w.hdim_qk,
                      hdim_v=w.hdim_v, jagged=True, cross=w.cross, causal=w.causal,
                      softmax=w.softmax, alpha=w.alpha, groups=[w.groups[0]] if len(w.groups) == 1
                      else [w.groups[b // (w.batch // len(w.groups))]],
                      uih_q=[w.uih_q[b]], targets=[w.targets[b]], uih_kv=[w.uih_kv[b]],
                      materialize=False)
        q0, q1 = w.q_offsets[b], w.q_offsets[b + 1]
        k0, k1 = w.kv_offsets[b], w.kv_offsets[b + 1]
        p = oracle.problem_of(sub)
        if len(w.groups) == 1 and w.groups[0].attn_scale == 0.0:
            # keep the whole workload's default scale (it does not change the work)
            p.ga = np.array([1.0 / max(w.uih_q)], np.float64)
        t0 = time.perf_counter()
        if rab is None:
            _, _, pairs = oracle.forward(p, w.q[q0:q1], w.k[k0:k1], w.v[k0:k1], lib=lib)
        else:
            ts = None if rab.timestamps is None else rab.timestamps[q0:q1]
            _, _, pairs = oracle.forward_rab(p, w.q[q0:q1], w.k[k0:k1], w.v[k0:k1], timestamps=ts,
                                             time_table=rab.time_table, pos_table=rab.pos_table,
                                             lib=lib)
        secs += time.perf_counter() - t0
        done_pairs += pairs
        seqs += 1
        if secs >= budget_s:
            break
    flops = done_pairs * 2.0 * (w.hdim_qk + w.hdim_v)
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(lib),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"first {seqs} of {w.batch} sequences, all {w.nhead} heads "
                      f"({done_pairs} visible pairs, {secs:.1f} s, fp64 C loops)"}


def algorithmic_bytes(w, rab=None) -> int:
    """q, k and v read once, o (and the softmax LSE) written once; with the bias,
    the timestamps and tables read once."""
    b = 2 * (w.total_q * w.nhead * (w.hdim_qk + w.hdim_v) + w.total_kv * w.nhead * (w.hdim_qk + w.hdim_v))
    if w.softmax:
        b += 4 * w.total_q * w.nhead
    if rab is not None:
        for a in (rab.timestamps, rab.time_table, rab.pos_table):
            b += 0 if a is None else a.nbytes
    return b


def roofline(w, splits, flops, ms, traffic, rab=None, kernel_ms=None):
    """Roofline of the step's dominant kernel, the forward kernel (the split kernel
    of a split-KV step): `achieved` is the step's algorithmic FLOPs or bytes over
    that kernel's own median duration (kernel_ms, events the library records
    around its launch), or over the whole step when that was not measured.  A
    workload with few query rows per key (the split-KV cross-attention one: ~72
    FLOP per byte, far below the ~310 FLOP/B balance point of the chip) is bounded
    by HBM, the others by the MFMA."""
    peak = PEAK_TFLOPS[w.dtype]
    t = kernel_ms if kernel_ms else ms
    name = "hstu_fwd_kernel" + (f" (split, {splits} splits)" if splits > 1 else "")
    covers = (f"{name} alone, HIP events around its launch" if kernel_ms else
              "whole step" + (f" (split kernel + combine, {splits} splits)" if splits > 1 else ""))
    nbytes = algorithmic_bytes(w, rab)
    if flops / nbytes < peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        gbs = nbytes / (t * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel_ms": round(t, 4),
                "covers": covers,
                "traffic_unit": "bytes per launch of the forward kernel (FETCH_SIZE+WRITE_SIZE, copy-calibrated)"}
    tflops = flops / (t * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4), "traffic": traffic, "kernel_ms": round(t, 4),
            "covers": covers,
            "traffic_unit": "bytes per launch (FETCH_SIZE+WRITE_SIZE, copy-calibrated)"}


def layer_flops(w, d_model, pairs) -> float:
    """f1 (2 n d_model N1) + the attention (2 (dqk + dv) per visible pair) + f2 (2 n H dv d_model)."""
    n, H = w.total_q, w.nhead
    n1 = 2 * H * (w.hdim_qk + w.hdim_v)
    return 2.0 * n * d_model * n1 + pairs * 2.0 * (w.hdim_qk + w.hdim_v) + 2.0 * n * H * w.hdim_v * d_model


def layer_cpu_baseline(w, d_model, li, rab, budget_s: float):
    """The oracle layer (numpy float64 projections, the C attention oracle), untuned,
    on whole sequences until about budget_s of wall time."""
    import numpy as np

    import oracle
    import oracle.layer as OL
    import workloads as W
    lib = oracle.load()
    flops, secs, seqs = 0.0, 0.0, 0
    scale = 1.0 / max(max(w.uih_q), 1)
    for b in range(w.batch):
        sub = W.build("sample", dtype=w.dtype, batch=1, nhead=w.nhead, hdim_qk=w.hdim_qk,
                      hdim_v=w.hdim_v, jagged=True, cross=False, causal=w.causal, softmax=w.softmax,
                      alpha=w.alpha, groups=[W.MaskGroup(g.local_len, g.context_len, g.minfull_len,
                                                         g.attn_scale or scale) for g in w.groups[:1]],
                      uih_q=[w.uih_q[b]], targets=[w.targets[b]], materialize=False)
        q0, q1 = w.q_offsets[b], w.q_offsets[b + 1]
        r = W.RabInputs(None if rab.timestamps is None else rab.timestamps[q0:q1], rab.time_table,
                        rab.pos_table)
        p = oracle.problem_of(sub)
        t0 = time.perf_counter()
        OL.hstu_layer(p, li.x[q0:q1], li.w1, li.b1, li.w2, li.b2, li.gamma, li.beta, li.eps, rab=r)
        secs += time.perf_counter() - t0
        flops += layer_flops(sub, d_model, int(oracle.count_pairs(p, lib=lib).sum()) * w.nhead)
        seqs += 1
        if secs >= budget_s:
            break
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(lib),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"first {seqs} of {w.batch} sequences, whole layer, all {w.nhead} heads "
                      f"({secs:.1f} s; numpy float64 projections, C float64 attention)"}


def layer_main(args, torch):
    """One step = one hstu_layer call over the whole workload.  A second timed loop
    runs the same four kernels through their own entry points with HIP events
    between them, for the per-kernel durations of the roofline."""
    import recsys_attention_amd as hip
    import workloads as W
    from hip_runner import layer_kwargs

    w, d_model, rab = W.layer_config(args.workload)
    li = W.layer_inputs(w, d_model, W.LAYER_SEED)
    x, w1, b1, w2, b2, kw = layer_kwargs(w, li, rab)
    n, H, dqk, dv = w.total_q, w.nhead, w.hdim_qk, w.hdim_v
    hv, hq, n1 = H * dv, H * dqk, 2 * H * (dv + dqk)
    print(f"bench: {w.name}, {n} tokens, d_model {d_model}", file=sys.stderr, flush=True)
    ws = torch.empty(hip.hstu_layer_workspace_size(x, w1, b1, w2, b2, **kw), dtype=torch.uint8,
                     device=x.device)
    out = torch.empty_like(x)
    # views of the workspace as the layer lays it out: [U | V | Q | K] and the attention output
    y1 = ws[:n * n1 * 2].view(x.dtype).view(n, n1)
    off = (n * n1 * 2 + 255) // 256 * 256
    ao = ws[off:off + n * hv * 2].view(x.dtype).view(n, hv)
    attn_kw = {k: kw[k] for k in ("num_targets", "causal", "softmax", "alpha", "groups", "seq_offsets",
                                  "rab_timestamps", "rab_time", "rab_pos")}
    attn_kw["max_seqlen_q"] = kw["max_seqlen"]
    q = y1[:, 2 * hv:2 * hv + hq].view(n, H, dqk)
    k = y1[:, 2 * hv + hq:].view(n, H, dqk)
    v = y1[:, hv:2 * hv].view(n, H, dv)
    o = ao.view(n, H, dv)
    pairs = hip.hstu_count_visible_pairs(q, k, v, **{a: b for a, b in attn_kw.items()
                                                     if not a.startswith("rab_")})
    flops = layer_flops(w, d_model, pairs)
    stream = torch.cuda.current_stream()

    def step():
        hip.hstu_layer(x, w1, b1, w2, b2, workspace=ws, out=out, **kw)

    kernels = [
        ("linear_f1_silu", lambda: hip.hstu_linear(x, w1, b1, activation="silu", out=y1),
         2.0 * n * d_model * n1, 2 * (n * d_model + n1 * d_model + n * n1)),
        ("hstu_fwd_kernel", lambda: hip.hstu_fwd(q, k, v, out=o, **attn_kw),
         pairs * 2.0 * (dqk + dv), 2 * n * (2 * hq + 2 * hv)),
        ("norm_gate", lambda: hip.hstu_norm_gate(ao, y1[:, :hv], kw["ln_gamma"], kw["ln_beta"],
                                                 kw["ln_eps"], out=ao), 0.0, 2 * 3 * n * hv),
        ("linear_f2_residual", lambda: hip.hstu_linear(ao, w2, b2, residual=x, out=out),
         2.0 * n * hv * d_model, 2 * (n * hv + hv * d_model + 2 * n * d_model)),
    ]
    ms, timing = timed_steps(torch, step, args.steps, args.warmup, args.warmup_s, stream)
    # per-kernel durations: events between the four launches of each step
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(args.steps)]
    for e in evs:
        e[0].record(stream)
        for i, (_, fn, _, _) in enumerate(kernels):
            fn()
            e[i + 1].record(stream)
    torch.cuda.synchronize()
    per = []
    for i, (name, _, kf, kb) in enumerate(kernels):
        kms = sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps
        per.append({"kernel": name, "ms": round(kms, 4), "tflops": round(kf / (kms * 1e-3) / 1e12, 2),
                    "gbs": round(kb / (kms * 1e-3) / 1e9, 1)})
    dom = max(range(len(kernels)), key=lambda i: per[i]["ms"])
    name, _, kf, kb = kernels[dom]
    kms = per[dom]["ms"]
    if kf / kb >= PEAK_TFLOPS[w.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": per[dom]["tflops"], "peak": PEAK_TFLOPS[w.dtype],
                "unit": "TFLOP/s", "frac": round(per[dom]["tflops"] / PEAK_TFLOPS[w.dtype], 4)}
    else:
        roof = {"bound": "hbm", "achieved": per[dom]["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(per[dom]["gbs"] / PEAK_HBM_GBS, 4)}
    roof.update({"kernel": name, "traffic": None, "per_kernel": per})
    tflops = flops / (ms * 1e-3) / 1e12
    out_line = {
        "metric": "HSTU layer fwd effective TFLOP/s (f1, attention over visible pairs, f2), 1 GPU",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "nhead": H, "hdim_qk": dqk, "hdim_v": dv,
                   "d_model": d_model, "total_tokens": n, "visible_pairs": pairs, "rab": "both",
                   "pct_of_bf16_peak": round(100.0 * tflops / PEAK_TFLOPS[w.dtype], 2)},
        "roofline": roof,
        "device": device_info(torch),
        "timing": timing,
    }
    if args.cpu_seconds > 0:
        out_line["cpu_baseline"] = layer_cpu_baseline(w, d_model, li, rab, args.cpu_seconds)
    print(json.dumps(out_line), flush=True)


def schedule_run(w, splits, schedule):
    """The work order the library picks for schedule 0 (its rule: the persistent
    grid, 3, from 2048 possible items when the workspace holds the queues, which
    the binding provides; else the per-item grid, 2, unsplit in q-tile levels
    from each sequence's end, and with each sequence's last two q-tiles cut into
    2 to 4 chunks when that grid (at least one chunk slot more per cut q-tile)
    holds fewer work-groups than the chip runs at once (256 CUs, two per CU, one
    for hdim 256) and a sequence has more than 256 keys)."""
    if schedule != 0:
        return schedule
    bh_pad = (w.batch * w.nhead + 7) // 8 * 8
    items = bh_pad * ((w.max_seqlen_q + 127) // 128) * splits
    if items >= 2048:
        return 3
    bn = 128 if w.hdim_qk <= 64 else 64
    chunk = 1 if bn >= 256 else 256 // bn
    kv = w.max_seqlen_kv if w.cross else w.max_seqlen_q
    slots = 256 * (1 if w.hdim_qk >= 256 else 2)
    nq = (w.max_seqlen_q + 127) // 128
    if splits == 1 and bh_pad * (nq + min(nq, 2)) < slots and (kv + bn - 1) // bn > chunk:
        return "2 (levels, last q-tiles cut)"
    return "2 (levels)" if splits == 1 else 2


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "this operator's multi-GPU sharding is described, not built.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    import torch

    import workloads as W
    from hip_runner import DeviceInputs, rab_kwargs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload in W.LAYER_NAMES:
        layer_main(args, torch)
        return
    w = W.config(args.workload)
    splits = args.splits or w.num_splits
    label = w.name if args.rab == "none" else f"{w.name}+rab_{args.rab}"
    print(f"bench: {label}, {w.total_q} q tokens, splits={splits}", file=sys.stderr, flush=True)
    dev = DeviceInputs(w)
    rab = None
    if args.rab != "none":
        # bias inputs drawn once (seeded) and resident on the device like q/k/v
        rab = W.rab_inputs(w, RAB_SEED, time=args.rab in ("time", "both"),
                           pos_len=RAB_POS_LEN if args.rab in ("pos", "both") else None)
        dev.kw.update(rab_kwargs(rab))
    stream = torch.cuda.current_stream()
    pairs = dev.count_pairs(schedule=args.schedule)
    flops = pairs * 2.0 * (w.hdim_qk + w.hdim_v)

    if args.launch == "prepared":
        # the argument block, output and workspace fixed once: each step is one C
        # call (the binding's own per-call checks and allocations cost ~20 us of
        # host time, more than the small workloads' kernels)
        step = dev.prepare(num_splits=splits, schedule=args.schedule)
    else:
        def step():
            return dev.forward(num_splits=splits, schedule=args.schedule)

    ms, timing = timed_steps(torch, step, args.steps, args.warmup, args.warmup_s, stream)
    timing["launch"] = args.launch
    kernel_ms = None
    if args.launch == "prepared":
        kernel_ms, timing["main_kernel"] = main_kernel_times(torch, step, args.steps, stream)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]

    traffic = None
    tf = os.path.join(ROOT, "profiles", f"traffic_{label}.json")
    if os.path.exists(tf):
        rec = json.load(open(tf))
        if rec.get("kernel_hash") == kernel_hash():
            traffic = rec.get("hbm_bytes_per_launch")

    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": label, "batch": w.batch, "nhead": w.nhead,
                   "hdim_qk": w.hdim_qk, "hdim_v": w.hdim_v, "total_tokens": w.total_q,
                   "max_seqlen": w.max_seqlen_q, "visible_pairs": pairs,
                   "splits": splits, "schedule": args.schedule,
                   "schedule_run": schedule_run(w, splits, args.schedule),
                   "pct_of_bf16_peak": round(100.0 * tflops / peak, 2)},
        "roofline": roofline(w, splits, flops, ms, traffic, rab, kernel_ms),
        "device": device_info(torch),
        "timing": timing,
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, rab)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

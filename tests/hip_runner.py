"""Runs a workloads.Workload through the HIP library and compares with the oracle.

Used by the GPU tests, the smoke check and the benchmark.  The oracle and the
HIP path receive the same rounded input bits; nothing of either side's
arithmetic lives here, only marshalling and the comparison rule.
"""
from __future__ import annotations

import numpy as np
import torch

import recsys_attention_amd as hip


def to_device(bits: np.ndarray, dtype: str, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.to(device)


def hip_groups(w):
    mx = hip.group_max_uih(w.uih_q, len(w.groups))
    return [hip.HstuGroup(g.local_len, g.context_len, g.minfull_len, g.attn_scale, mx[i])
            for i, g in enumerate(w.groups)]


class DeviceInputs:
    """q/k/v and metadata of a workload on the device, in the layout the ABI takes."""

    def __init__(self, w, device="cuda"):
        self.w = w
        q = to_device(w.q_bits, w.dtype, device)
        k = to_device(w.k_bits, w.dtype, device)
        v = to_device(w.v_bits, w.dtype, device)
        H = w.nhead
        if w.jagged:
            self.q, self.k, self.v = q, k, v
            self.kw = dict(seq_offsets=torch.tensor(w.q_offsets, dtype=torch.int32, device=device),
                           max_seqlen_q=w.max_seqlen_q)
            if w.cross:
                self.kw.update(seq_offsets_kv=torch.tensor(w.kv_offsets, dtype=torch.int32,
                                                           device=device),
                               max_seqlen_kv=w.max_seqlen_kv)
        else:
            B, Sq, Skv = w.batch, w.seqlen_q[0] if w.batch else 0, w.seqlen_kv[0] if w.batch else 0
            self.q = q.view(B, Sq, H, w.hdim_qk)
            self.k = k.view(B, Skv, H, w.hdim_qk)
            self.v = v.view(B, Skv, H, w.hdim_v)
            self.kw = {}
        self.kw.update(num_targets=torch.tensor(w.targets, dtype=torch.int32, device=device),
                       cross=w.cross, causal=w.causal, softmax=w.softmax, alpha=w.alpha,
                       groups=hip_groups(w))

    def forward(self, num_splits=1, schedule=0, return_lse=None, out=None, workspace=None,
                rab=None):
        rl = self.w.softmax if return_lse is None else return_lse
        kw = dict(self.kw)
        if rab is not None:
            kw.update(rab_kwargs(rab, self.q.device))
        if num_splits == 1:
            return hip.hstu_fwd(self.q, self.k, self.v, return_lse=rl, schedule=schedule, out=out,
                                **kw)
        return hip.hstu_fwd_splitkv(self.q, self.k, self.v, num_splits, return_lse=rl,
                                    schedule=schedule, out=out, workspace=workspace, **kw)

    def prepare(self, num_splits=1, schedule=0, return_lse=None):
        """The same call as forward(), argument block and buffers fixed once."""
        rl = self.w.softmax if return_lse is None else return_lse
        return hip.prepare(self.q, self.k, self.v, num_splits, return_lse=rl, schedule=schedule,
                           **self.kw)

    def count_pairs(self, schedule=0):
        return hip.hstu_count_visible_pairs(self.q, self.k, self.v, schedule=schedule, **self.kw)


def rab_kwargs(rab, device="cuda"):
    """workloads.RabInputs -> the binding's rab_* arguments (device tensors)."""
    def dev(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return dict(rab_timestamps=dev(rab.timestamps), rab_time=dev(rab.time_table),
                rab_pos=dev(rab.pos_table))


def o_tokens(w, o: torch.Tensor) -> np.ndarray:
    """Output as float32 numpy [total_q, H, Dv] (token-major like the oracle's)."""
    return o.float().reshape(-1, w.nhead, w.hdim_v).cpu().numpy()


def lse_tokens(w, lse: torch.Tensor) -> np.ndarray:
    """LSE as [total_q, H] (batched [B,H,S] and jagged [H,total] both re-laid out)."""
    x = lse.cpu().numpy()
    if w.jagged:
        return x.T
    return x.transpose(0, 2, 1).reshape(-1, w.nhead)


def tolerances(dtype: str):
    """The operator's stated elementwise bound, plus scale-free checks.

    row_rel: per output row, max|o - ref| <= row_rel * max|ref_row|.  The kernel
    rounds P to the input dtype before P.V (one rounding of 2^-9 relative for
    bf16, 2^-11 for fp16 per term); over n visible keys that error grows like a
    random walk, about 0.05 % of the row's largest element for the longest rows
    of the workloads, so row_rel leaves a wide margin while still catching a
    missing or doubled key tile (several percent).
    """
    if dtype == "bf16":
        return dict(atol=2e-2, rtol=2e-2, row_rel=1e-2, rel_l2=1e-2)
    return dict(atol=1e-2, rtol=1e-2, row_rel=4e-3, rel_l2=5e-3)


def compare(o: np.ndarray, ref: np.ndarray, dtype: str, what="", elementwise=True):
    """Compare an output [rows, H, Dv] (or [rows, Dv]) with the oracle's.

    elementwise: max|o - ref| <= atol + rtol |ref| (the operator's stated bound;
    meaningful at the workloads' own attn_scale, which keeps |o| small).
    Always: the per-row relative bound above, exact zeros where the reference
    row is zero, and relative L2 over everything <= rel_l2."""
    tol = tolerances(dtype)
    o = np.asarray(o, np.float64)
    ref = np.asarray(ref, np.float64)
    assert o.shape == ref.shape, (o.shape, ref.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - ref)
    if elementwise:
        bound = tol["atol"] + tol["rtol"] * np.abs(ref)
        worst = np.unravel_index(np.argmax(err - bound), err.shape) if err.size else None
        assert (err <= bound).all(), \
            f"{what}: elementwise bound fails at {worst}: {o[worst]} vs {ref[worst]}"
    rerr = err.max(axis=-1) if err.size else err
    rmax = np.abs(ref).max(axis=-1) if ref.size else ref
    zero = rmax == 0
    assert (rerr[zero] == 0).all(), f"{what}: rows with a zero reference are not zero"
    ratio = np.where(zero, 0.0, rerr / np.where(zero, 1.0, rmax))
    if ratio.size:
        worst = np.unravel_index(np.argmax(ratio), ratio.shape)
        assert ratio.max() <= tol["row_rel"], \
            f"{what}: row {worst} error {rerr[worst]} vs row max {rmax[worst]} ({ratio.max():.2e})"
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    if scale > 0:
        rl2 = np.linalg.norm(o - ref) / np.linalg.norm(ref)
        assert rl2 <= tol["rel_l2"], f"{what}: relative L2 {rl2}"
    return dict(max_err=float(err.max(initial=0.0)), scale=scale,
                max_row_rel=float(ratio.max(initial=0.0)))


def compare_lse(lse: np.ndarray, ref: np.ndarray, what=""):
    """|lse - ref| <= 1e-3 + 1e-4 |ref|; -inf exactly where the reference row is empty."""
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(lse), ninf), f"{what}: -inf rows differ"
    d = np.abs(lse[~ninf] - ref[~ninf])
    assert (d <= 1e-3 + 1e-4 * np.abs(ref[~ninf])).all(), f"{what}: lse err {d.max(initial=0)}"


def bits_to_device(bits: np.ndarray, dtype: str, device="cuda"):
    """Rounded bits (uint16) -> a device tensor of the dtype, same shape."""
    return to_device(bits, dtype, device).view(bits.shape)


def layer_kwargs(w, li, rab=None, device="cuda"):
    """workloads.Workload + LayerInputs (+ RabInputs) -> (x, w1, b1, w2, b2, kwargs) for
    recsys_attention_amd.hstu_layer."""
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    x = bits_to_device(li.x_bits, w.dtype, device)
    w1 = bits_to_device(li.w1_bits, w.dtype, device)
    w2 = bits_to_device(li.w2_bits, w.dtype, device)
    kw = dict(nhead=w.nhead, hdim_qk=w.hdim_qk, hdim_v=w.hdim_v, ln_gamma=f32(li.gamma),
              ln_beta=f32(li.beta), ln_eps=li.eps,
              num_targets=torch.tensor(w.targets, dtype=torch.int32, device=device),
              causal=w.causal, softmax=w.softmax, alpha=w.alpha, groups=hip_groups(w))
    if w.jagged:
        kw.update(seq_offsets=torch.tensor(w.q_offsets, dtype=torch.int32, device=device),
                  max_seqlen=w.max_seqlen_q)
    else:
        kw.update(batch=w.batch)
    if rab is not None:
        kw.update(rab_kwargs(rab, device))
    return x, w1, f32(li.b1), w2, f32(li.b2), kw


def compare_rounded(o: np.ndarray, ref: np.ndarray, dtype: str, what="", atol=1e-3):
    """One rounding of an fp32 result to the dtype: |o - ref| <= 2^-8 |ref| (bf16;
    2^-10 for fp16) + atol."""
    o = np.asarray(o, np.float64)
    ref = np.asarray(ref, np.float64)
    assert o.shape == ref.shape, (o.shape, ref.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    rt = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -10
    err = np.abs(o - ref)
    bound = atol + rt * np.abs(ref)
    if err.size:
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert (err <= bound).all(), f"{what}: bound fails at {worst}: {o[worst]} vs {ref[worst]}"
    return float(err.max(initial=0.0))

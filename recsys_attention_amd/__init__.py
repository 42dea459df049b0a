"""MI355X-native HSTU attention forward (Python binding of libhstu.so).

Thin marshalling layer over the C ABI of include/hstu.h: tensors are torch
device tensors (PyTorch supplies device memory and the current stream), every
step of the operator runs in the HIP kernels.  Without the built library every
entry point raises.

    o = hstu_fwd(q, k, v, seq_offsets=off, max_seqlen_q=S, num_targets=t,
                 groups=[HstuGroup(local_len=5, context_len=6, minfull_len=6,
                                   attn_scale=0.0, max_uih_q=870)])
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional, Sequence

import torch

from . import _abi

__all__ = ["HstuGroup", "hstu_fwd", "hstu_fwd_splitkv", "hstu_count_visible_pairs",
           "workspace_size", "group_max_uih", "is_available", "library_path"]


@dataclasses.dataclass
class HstuGroup:
    """Mask scalars of one group (no-group HSTU: a single group)."""

    local_len: int = 5
    context_len: int = 6
    minfull_len: int = 6
    attn_scale: float = 0.0   # 0 -> 1 / max(max_uih_q, 1)
    max_uih_q: int = -1       # needed when attn_scale == 0


def group_max_uih(uih_lengths: Sequence[int], num_groups: int):
    """Largest UIH query length of each contiguous group of sequences."""
    B = len(uih_lengths)
    per = B // num_groups if num_groups else 0
    return [max(uih_lengths[g * per:(g + 1) * per], default=0) for g in range(num_groups)]


def is_available() -> bool:
    try:
        _abi.load()
        return True
    except (RuntimeError, OSError):
        return False


def library_path() -> str:
    return _abi.LIB_PATH


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _abi.HSTU_BF16
    if t.dtype == torch.float16:
        return _abi.HSTU_FP16
    raise ValueError(f"q/k/v must be bfloat16 or float16, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _tok_stride(t: torch.Tensor, name: str) -> int:
    if t.stride(-1) != 1 or t.stride(-2) != t.shape[-1]:
        raise ValueError(f"{name}: each head's vector and the heads of a token must be contiguous")
    if t.dim() == 4 and t.shape[0] > 1 and t.stride(0) != t.shape[1] * t.stride(1):
        raise ValueError(f"{name}: batched tokens must be evenly strided")
    return t.stride(-3)


def _groups_c(groups):
    if not groups:
        raise ValueError("at least one mask group is required")
    arr = (_abi.MaskGroupC * len(groups))()
    for i, g in enumerate(groups):
        arr[i].local_len = int(g.local_len)
        arr[i].context_len = int(g.context_len)
        arr[i].minfull_len = int(g.minfull_len)
        arr[i].attn_scale = float(g.attn_scale)
        arr[i].max_uih_q = int(getattr(g, "max_uih_q", -1))
    return arr


class _Call:
    """The hstu_fwd_args_t of one call plus the objects it points into."""

    def __init__(self, q, k, v, *, seq_offsets, seq_offsets_kv, num_targets, max_seqlen_q,
                 max_seqlen_kv, cross, causal, softmax, alpha, groups, return_lse, out, schedule,
                 rab_timestamps=None, rab_time=None, rab_pos=None):
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            if not t.is_cuda:
                raise ValueError(f"{n} must be a device tensor")
            if t.dim() not in (3, 4):
                raise ValueError(f"{n} must be [B, S, H, D] or [total, H, D]")
        dt = _dtype_code(q)
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise ValueError("q, k and v must share one dtype")
        jagged = seq_offsets is not None
        H, Dqk, Dv = q.shape[-2], q.shape[-1], v.shape[-1]
        if k.shape[-2] != H or v.shape[-2] != H or k.shape[-1] != Dqk:
            raise ValueError("q/k/v head counts or q/k head dims differ")
        if jagged:
            if seq_offsets.dtype != torch.int32 or not seq_offsets.is_cuda:
                raise ValueError("seq_offsets must be an int32 device tensor")
            B = seq_offsets.numel() - 1
            if max_seqlen_q is None:
                raise ValueError("jagged mode needs max_seqlen_q (an upper bound of the lengths)")
            total_q = q.shape[-3] if q.dim() == 3 else q.shape[0] * q.shape[1]
            Sq = int(max_seqlen_q)
            if cross:
                if seq_offsets_kv is None or max_seqlen_kv is None:
                    raise ValueError("jagged cross-attention needs seq_offsets_kv and max_seqlen_kv")
                Skv = int(max_seqlen_kv)
            else:
                Skv = Sq
            o_shape = (*q.shape[:-1], Dv)
            lse_shape = (H, total_q)
        else:
            if q.dim() != 4:
                raise ValueError("batched mode needs [B, S, H, D] tensors")
            B, Sq = q.shape[0], q.shape[1]
            Skv = k.shape[1]
            cross = bool(cross) or Skv != Sq
            total_q = B * Sq
            o_shape = (B, Sq, H, Dv)
            lse_shape = (B, H, Sq)
        if num_targets is not None and (num_targets.dtype != torch.int32 or not num_targets.is_cuda):
            raise ValueError("num_targets must be an int32 device tensor")
        if out is None:
            out = torch.empty(o_shape, dtype=q.dtype, device=q.device)
        self.lse = None
        if return_lse:
            if not softmax:
                raise ValueError("return_lse is for the softmax variant")
            self.lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
        self.out = out
        self.groups = _groups_c(groups)
        _check_rab(rab_timestamps, rab_time, rab_pos, H, total_q)
        self.keep = (q, k, v, seq_offsets, seq_offsets_kv, num_targets, rab_timestamps, rab_time, rab_pos)
        a = _abi.FwdArgsC()
        a.dtype, a.batch, a.nhead, a.hdim_qk, a.hdim_v = dt, B, H, Dqk, Dv
        a.jagged, a.cross = int(jagged), int(bool(cross))
        a.seqlen_q, a.seqlen_kv, a.total_q = Sq, Skv, total_q
        a.q, a.k, a.v, a.o = _ptr(q), _ptr(k), _ptr(v), _ptr(out)
        a.q_tok_stride = _tok_stride(q, "q")
        a.k_tok_stride = _tok_stride(k, "k")
        a.v_tok_stride = _tok_stride(v, "v")
        a.o_tok_stride = _tok_stride(out, "out")
        a.seq_offsets_q = _ptr(seq_offsets)
        a.seq_offsets_kv = _ptr(seq_offsets_kv) if (jagged and cross) else None
        a.num_targets = _ptr(num_targets)
        a.causal, a.softmax, a.alpha = int(bool(causal)), int(bool(softmax)), float(alpha)
        a.num_groups = len(groups)
        a.groups = ctypes.cast(self.groups, ctypes.POINTER(_abi.MaskGroupC))
        a.lse = _ptr(self.lse)
        a.schedule = int(schedule)
        a.rab_timestamps = _ptr(rab_timestamps)
        a.rab_time = _ptr(rab_time)
        a.rab_pos = _ptr(rab_pos)
        a.rab_pos_len = 0 if rab_pos is None else int(rab_pos.shape[-1])
        self.args = a
        self.device = q.device

    def stream(self, stream):
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        return ctypes.c_void_p(stream.cuda_stream)


def _check_rab(ts, tt, pt, H, total_q):
    """Shapes and types of the relative attention bias inputs (the library checks the rest)."""
    if ts is not None:
        if ts.dtype != torch.int32 or not ts.is_cuda or not ts.is_contiguous() or ts.numel() != total_q:
            raise ValueError("rab_timestamps must be a contiguous int32 device tensor, one per q token")
        if tt is None:
            raise ValueError("rab_timestamps needs rab_time")
    if tt is not None and (tt.dtype != torch.float32 or not tt.is_cuda or not tt.is_contiguous()
                           or tuple(tt.shape) != (H, _abi.HSTU_RAB_TIME_BUCKETS)):
        raise ValueError(f"rab_time must be a contiguous float32 device tensor [{H}, "
                         f"{_abi.HSTU_RAB_TIME_BUCKETS}]")
    if pt is not None and (pt.dtype != torch.float32 or not pt.is_cuda or not pt.is_contiguous()
                           or pt.dim() != 2 or pt.shape[0] != H):
        raise ValueError(f"rab_pos must be a contiguous float32 device tensor [{H}, P]")


def _result(call, return_lse):
    return (call.out, call.lse) if return_lse else call.out


def hstu_fwd(q, k, v, *, seq_offsets=None, seq_offsets_kv=None, num_targets=None,
             max_seqlen_q=None, max_seqlen_kv=None, cross=False, causal=True, softmax=False,
             alpha=0.0, groups=(HstuGroup(),), return_lse=False, out=None, schedule=0,
             rab_timestamps=None, rab_time=None, rab_pos=None, stream=None):
    """HSTU attention forward.  Batched: q [B, S_q, H, Dqk], k [B, S_kv, H, Dqk],
    v [B, S_kv, H, Dv].  Jagged: q/k/v [total, H, D] with int32 seq_offsets [B+1]
    (device) and max_seqlen_q.  Returns o (and the LSE when return_lse).
    Relative attention bias (self-attention): rab_timestamps int32 [tokens of q]
    with rab_time float32 [H, 11] (time-gap buckets), rab_pos float32 [H, P]
    (positional, indexed by min(|i - j|, P - 1))."""
    lib = _abi.load()
    c = _Call(q, k, v, seq_offsets=seq_offsets, seq_offsets_kv=seq_offsets_kv,
              num_targets=num_targets, max_seqlen_q=max_seqlen_q, max_seqlen_kv=max_seqlen_kv,
              cross=cross, causal=causal, softmax=softmax, alpha=alpha, groups=groups,
              return_lse=return_lse, out=out, schedule=schedule, rab_timestamps=rab_timestamps,
              rab_time=rab_time, rab_pos=rab_pos)
    _abi.check(lib.hstu_fwd(ctypes.byref(c.args), None, 0, c.stream(stream)))
    return _result(c, return_lse)


def workspace_size(q, k, v, num_splits, **kw) -> int:
    lib = _abi.load()
    c = _Call(q, k, v, **_call_kw(kw))
    return int(lib.hstu_fwd_workspace_size(ctypes.byref(c.args), int(num_splits)))


def _call_kw(kw):
    d = dict(seq_offsets=None, seq_offsets_kv=None, num_targets=None, max_seqlen_q=None,
             max_seqlen_kv=None, cross=False, causal=True, softmax=False, alpha=0.0,
             groups=(HstuGroup(),), return_lse=False, out=None, schedule=0, rab_timestamps=None,
             rab_time=None, rab_pos=None)
    d.update(kw)
    return d


def hstu_fwd_splitkv(q, k, v, num_splits, *, workspace=None, stream=None, **kw):
    """Split-KV forward: partial results per key chunk in a workspace, then a combine
    kernel.  Same arguments and result as hstu_fwd.  The workspace (a uint8 device
    tensor of at least workspace_size() bytes) is allocated when not given."""
    lib = _abi.load()
    d = _call_kw(kw)
    c = _Call(q, k, v, **d)
    need = int(lib.hstu_fwd_workspace_size(ctypes.byref(c.args), int(num_splits)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _abi.check(lib.hstu_fwd_splitkv(ctypes.byref(c.args), int(num_splits), ws_ptr, ws_bytes,
                                    c.stream(stream)))
    return _result(c, d["return_lse"])


def hstu_count_visible_pairs(q, k, v, *, stream=None, **kw) -> int:
    """Visible (b, h, i, j) pairs inside the key tiles the forward kernel schedules,
    counted on the device with the kernel's own predicate."""
    lib = _abi.load()
    c = _Call(q, k, v, **_call_kw(kw))
    cnt = torch.zeros(1, dtype=torch.int64, device=q.device)
    _abi.check(lib.hstu_count_visible_pairs(ctypes.byref(c.args), ctypes.c_void_p(cnt.data_ptr()),
                                            c.stream(stream)))
    return int(cnt.item())

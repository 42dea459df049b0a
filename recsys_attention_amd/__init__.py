"""MI355X-native HSTU attention forward (Python binding of libhstu.so).

Thin marshalling layer over the C ABI of include/hstu.h: tensors are torch
device tensors (PyTorch supplies device memory and the current stream), every
step of the operator runs in the HIP kernels.  Without the built library every
entry point raises.

    o = hstu_fwd(q, k, v, seq_offsets=off, max_seqlen_q=S, num_targets=t,
                 groups=[HstuGroup(local_len=5, context_len=6, minfull_len=6,
                                   attn_scale=0.0, max_uih_q=870)])

Every entry point takes stream= (a torch.cuda.Stream; default the current
stream): the kernels are enqueued there and the call's own allocations (output,
LSE, workspace) are made there, so the caching allocator reuses them in that
stream's order.  Ordering the inputs' producers before that stream is the
caller's part, as for any torch operation on a side stream.
"""
from __future__ import annotations

import contextlib
import ctypes
import dataclasses
from typing import Optional, Sequence

import torch

from . import _abi

__all__ = ["HstuGroup", "hstu_fwd", "hstu_fwd_splitkv", "hstu_fwd_splitkv_noalloc",
           "hstu_count_visible_pairs", "prepare", "PreparedCall",
           "workspace_size", "group_max_uih", "is_available", "library_path",
           "hstu_linear", "hstu_norm_gate", "hstu_layer", "hstu_layer_workspace_size"]


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
                 rab_timestamps=None, rab_time=None, rab_pos=None, lse_out=None):
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
            if lse_out is None:
                lse_out = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
            if (lse_out.dtype != torch.float32 or tuple(lse_out.shape) != tuple(lse_shape)
                    or not lse_out.is_contiguous()):
                raise ValueError(f"lse_out must be a contiguous float32 tensor {list(lse_shape)}")
            self.lse = lse_out
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
             rab_timestamps=None, rab_time=None, rab_pos=None, workspace=None, stream=None):
    """HSTU attention forward.  Batched: q [B, S_q, H, Dqk], k [B, S_kv, H, Dqk],
    v [B, S_kv, H, Dv].  Jagged: q/k/v [total, H, D] with int32 seq_offsets [B+1]
    (device) and max_seqlen_q.  Returns o (and the LSE when return_lse).
    Relative attention bias (self-attention): rab_timestamps int32 [tokens of q]
    with rab_time float32 [H, 11] (time-gap buckets), rab_pos float32 [H, P]
    (positional, indexed by min(|i - j|, P - 1)).
    schedule 0 and 3 use a small workspace (uint8 device tensor of workspace_size(...,
    num_splits=1) bytes) for the persistent schedule's work queues; it is allocated
    when not given."""
    lib = _abi.load()
    with _on(stream):
        c = _Call(q, k, v, seq_offsets=seq_offsets, seq_offsets_kv=seq_offsets_kv,
                  num_targets=num_targets, max_seqlen_q=max_seqlen_q, max_seqlen_kv=max_seqlen_kv,
                  cross=cross, causal=causal, softmax=softmax, alpha=alpha, groups=groups,
                  return_lse=return_lse, out=out, schedule=schedule, rab_timestamps=rab_timestamps,
                  rab_time=rab_time, rab_pos=rab_pos)
        ws_ptr, ws_bytes = _workspace(lib, c, 1, workspace, q.device)
        _abi.check(lib.hstu_fwd(ctypes.byref(c.args), ws_ptr, ws_bytes, c.stream(stream)))
    return _result(c, return_lse)


def _on(stream):
    """Context in which a call's own allocations (output, LSE, workspace, counters) are
    made: the caller's stream when one is given, so that the caching allocator
    hands out and later reuses those blocks in that stream's order (the kernels
    run there); otherwise the current stream, where they run too."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _workspace(lib, c, num_splits, workspace, device):
    """(pointer, bytes) of the call's workspace, allocated (on the stream of the
    enclosing _on context) when not given and the call needs one."""
    need = int(lib.hstu_fwd_workspace_size(ctypes.byref(c.args), int(num_splits)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace is None:
        return None, 0
    c.keep_workspace = workspace
    return _ptr(workspace), workspace.numel() * workspace.element_size()


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
    with _on(stream):
        c = _Call(q, k, v, **d)
        ws_ptr, ws_bytes = _workspace(lib, c, num_splits, workspace, q.device)
        _abi.check(lib.hstu_fwd_splitkv(ctypes.byref(c.args), int(num_splits), ws_ptr, ws_bytes,
                                        c.stream(stream)))
    return _result(c, d["return_lse"])


def hstu_fwd_splitkv_noalloc(q, k, v, num_splits, *, out, lse_out=None, stream=None, **kw):
    """hstu_fwd_splitkv for callers that cannot allocate: the split-KV partials and
    the work queues go to the library's static scratch (HSTU_NOALLOC_SCRATCH_BYTES
    per GPU), and the caller passes the output (and, with return_lse, lse_out):
    nothing is allocated.  Calls that overlap in time on one GPU race (they share
    its scratch)."""
    lib = _abi.load()
    if out is None:
        raise ValueError("the allocation-free call needs out")
    d = _call_kw(kw)
    if d["return_lse"] and lse_out is None:
        raise ValueError("the allocation-free call needs lse_out with return_lse")
    d.update(out=out)
    c = _Call(q, k, v, lse_out=lse_out, **d)
    _abi.check(lib.hstu_fwd_splitkv_noalloc(ctypes.byref(c.args), int(num_splits), c.stream(stream)))
    return _result(c, d["return_lse"])


class PreparedCall:
    """One forward call with its argument block, output (and LSE) and workspace
    fixed once, for loops that launch the same call again and again (serving,
    benchmarking): each call() is one C call, hstu_fwd (num_splits == 1) or
    hstu_fwd_splitkv, on the given or current stream, with none of the argument
    checks and allocations of hstu_fwd.  Every call overwrites the same out (and
    lse) and reuses the workspace, so calls must not overlap in time; the tensors
    given to prepare() must stay alive and unchanged in shape while it is used."""

    def __init__(self, lib, c, num_splits, workspace, return_lse):
        self._lib, self._c, self._splits = lib, c, int(num_splits)
        self._args = ctypes.byref(c.args)
        self._ws = workspace
        self._ws_ptr = ctypes.c_void_p(_ptr(workspace)) if workspace is not None else None
        self._ws_bytes = workspace.numel() if workspace is not None else 0
        self.out, self.lse = c.out, c.lse
        self._return_lse = return_lse
        self._streams = {}

    def set_profiling_events(self, begin=None, end=None):
        """torch.cuda.Event objects (or None) that the following calls record right
        before and right after their main kernel (the argument block's profiling
        hooks); an event must have been recorded once, so that it exists."""
        self._c.args.prof_begin = begin.cuda_event if begin is not None else None
        self._c.args.prof_end = end.cuda_event if end is not None else None

    def __call__(self, stream=None):
        if stream is None:
            stream = torch.cuda.current_stream(self._c.device)
        sp = self._streams.get(stream.cuda_stream)
        if sp is None:
            sp = self._streams[stream.cuda_stream] = ctypes.c_void_p(stream.cuda_stream)
        if self._splits == 1:
            st = self._lib.hstu_fwd(self._args, self._ws_ptr, self._ws_bytes, sp)
        else:
            st = self._lib.hstu_fwd_splitkv(self._args, self._splits, self._ws_ptr, self._ws_bytes, sp)
        if st != _abi.HSTU_OK:
            _abi.check(st)
        return (self.out, self.lse) if self._return_lse else self.out


def prepare(q, k, v, num_splits=1, *, workspace=None, stream=None, **kw):
    """A PreparedCall of hstu_fwd (num_splits == 1) or hstu_fwd_splitkv with these
    arguments: checked once here (the library validates the argument block), its
    output, LSE and workspace allocated once (on the given or current stream)."""
    lib = _abi.load()
    d = _call_kw(kw)
    with _on(stream):
        c = _Call(q, k, v, **d)
        _abi.check(lib.hstu_validate_args(ctypes.byref(c.args)))
        need = int(lib.hstu_fwd_workspace_size(ctypes.byref(c.args), int(num_splits)))
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_cuda
                                      or workspace.numel() < need):
            raise ValueError(f"workspace must be a uint8 device tensor of at least {need} bytes")
    return PreparedCall(lib, c, num_splits, workspace, d["return_lse"])


def hstu_count_visible_pairs(q, k, v, *, stream=None, **kw) -> int:
    """Visible (b, h, i, j) pairs inside the key tiles the forward kernel schedules,
    counted on the device with the kernel's own predicate."""
    lib = _abi.load()
    with _on(stream):
        c = _Call(q, k, v, **_call_kw(kw))
        cnt = torch.zeros(1, dtype=torch.int64, device=q.device)
        _abi.check(lib.hstu_count_visible_pairs(ctypes.byref(c.args), ctypes.c_void_p(cnt.data_ptr()),
                                                c.stream(stream)))
        return int(cnt.item())


# ------------------------------------------------------------- the HSTU layer
# (include/hstu_layer.h: HSTU explainer, "The layer, line by line")

_ACT = {"none": _abi.HSTU_ACT_NONE, "silu": _abi.HSTU_ACT_SILU}


def _stream_ptr(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _rows2d(t: torch.Tensor, name: str):
    if not t.is_cuda or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D device tensor with contiguous rows")
    return t.stride(0)


def _f32vec(t: Optional[torch.Tensor], n: int, name: str):
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name} must be a contiguous float32 device tensor of {n} elements")
    return t.data_ptr()


def hstu_linear(x, w, bias=None, *, activation="none", residual=None, out=None, stream=None):
    """y = act(x w^T + bias) (+ residual): x [M, K] (rows may be strided), w [N, K]
    contiguous (a torch Linear weight), bias float32 [N], residual [M, N]."""
    lib = _abi.load()
    dt = _dtype_code(x)
    xs = _rows2d(x, "x")
    if w.dtype != x.dtype or not w.is_cuda or not w.is_contiguous() or w.dim() != 2:
        raise ValueError("w must be a contiguous 2-D device tensor of x's dtype")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError(f"w is [{N}, {w.shape[1]}], x has {K} features")
    rs = 0
    if residual is not None:
        if residual.dtype != x.dtype or tuple(residual.shape) != (M, N):
            raise ValueError(f"residual must be [{M}, {N}] of x's dtype")
        rs = _rows2d(residual, "residual")
    if out is None:
        with _on(stream):
            out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if out.dtype != x.dtype or tuple(out.shape) != (M, N):
        raise ValueError(f"out must be [{M}, {N}] of x's dtype")
    a = _abi.LinearArgsC(dtype=dt, rows=M, in_features=K, out_features=N, x=x.data_ptr(), x_stride=xs,
                         w=w.data_ptr(), bias=_f32vec(bias, N, "bias"), activation=_ACT[activation],
                         residual=_ptr(residual), residual_stride=rs, y=out.data_ptr(),
                         y_stride=_rows2d(out, "out"))
    _abi.check(lib.hstu_linear_fwd(ctypes.byref(a), _stream_ptr(x.device, stream)))
    return out


def hstu_norm_gate(a, u, gamma=None, beta=None, eps=1e-6, *, out=None, stream=None):
    """(LayerNorm(a) * gamma + beta) * u over the last dim of the 2-D tensors a, u
    (rows may be strided; out may be a)."""
    lib = _abi.load()
    dt = _dtype_code(a)
    if u.dtype != a.dtype or u.shape != a.shape:
        raise ValueError("u must match a's shape and dtype")
    M, W_ = a.shape
    if out is None:
        with _on(stream):
            out = torch.empty((M, W_), dtype=a.dtype, device=a.device)
    if out.dtype != a.dtype or out.shape != a.shape:
        raise ValueError("out must match a's shape and dtype")
    args = _abi.NormGateArgsC(dtype=dt, rows=M, width=W_, a=a.data_ptr(), a_stride=_rows2d(a, "a"),
                              u=u.data_ptr(), u_stride=_rows2d(u, "u"),
                              gamma=_f32vec(gamma, W_, "gamma"), beta=_f32vec(beta, W_, "beta"),
                              eps=float(eps), z=out.data_ptr(), z_stride=_rows2d(out, "out"))
    _abi.check(lib.hstu_norm_gate_fwd(ctypes.byref(args), _stream_ptr(a.device, stream)))
    return out


class _LayerCall:
    """The hstu_layer_args_t of one call plus the objects it points into."""

    def __init__(self, x, w1, b1, w2, b2, *, nhead, hdim_qk, hdim_v, ln_gamma, ln_beta, ln_eps,
                 seq_offsets, max_seqlen, batch, num_targets, causal, softmax, alpha, groups,
                 schedule, rab_timestamps, rab_time, rab_pos, out):
        dt = _dtype_code(x)
        if not x.is_cuda or x.dim() != 2 or not x.is_contiguous():
            raise ValueError("x must be a contiguous [tokens, d_model] device tensor")
        n, d_model = x.shape
        H, dqk, dv = int(nhead), int(hdim_qk), int(hdim_v)
        n1 = 2 * H * (dv + dqk)
        for t, shape, name in ((w1, (n1, d_model), "w1"), (w2, (d_model, H * dv), "w2")):
            if t.dtype != x.dtype or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != shape:
                raise ValueError(f"{name} must be a contiguous {list(shape)} device tensor of x's dtype")
        jagged = seq_offsets is not None
        if jagged:
            if seq_offsets.dtype != torch.int32 or not seq_offsets.is_cuda:
                raise ValueError("seq_offsets must be an int32 device tensor")
            if max_seqlen is None:
                raise ValueError("jagged mode needs max_seqlen (an upper bound of the lengths)")
            B, S = seq_offsets.numel() - 1, int(max_seqlen)
        else:
            if batch is None or n % int(batch):
                raise ValueError("batched mode needs batch dividing the token count")
            B, S = int(batch), n // int(batch)
        if num_targets is not None and (num_targets.dtype != torch.int32 or not num_targets.is_cuda):
            raise ValueError("num_targets must be an int32 device tensor")
        _check_rab(rab_timestamps, rab_time, rab_pos, H, n)
        if out is None:
            out = torch.empty_like(x)
        self.out = out
        self.groups = _groups_c(groups)
        self.keep = (x, w1, b1, w2, b2, ln_gamma, ln_beta, seq_offsets, num_targets, rab_timestamps,
                     rab_time, rab_pos)
        t = _abi.FwdArgsC()
        t.dtype, t.batch, t.nhead, t.hdim_qk, t.hdim_v = dt, B, H, dqk, dv
        t.jagged, t.cross = int(jagged), 0
        t.seqlen_q = t.seqlen_kv = S
        t.total_q = n
        t.seq_offsets_q = _ptr(seq_offsets)
        t.num_targets = _ptr(num_targets)
        t.causal, t.softmax, t.alpha = int(bool(causal)), int(bool(softmax)), float(alpha)
        t.num_groups = len(groups)
        t.groups = ctypes.cast(self.groups, ctypes.POINTER(_abi.MaskGroupC))
        t.schedule = int(schedule)
        t.rab_timestamps, t.rab_time, t.rab_pos = _ptr(rab_timestamps), _ptr(rab_time), _ptr(rab_pos)
        t.rab_pos_len = 0 if rab_pos is None else int(rab_pos.shape[-1])
        a = _abi.LayerArgsC()
        a.attn = t
        a.d_model = d_model
        a.x, a.w1, a.w2, a.out = x.data_ptr(), w1.data_ptr(), w2.data_ptr(), out.data_ptr()
        a.b1 = _f32vec(b1, n1, "b1")
        a.b2 = _f32vec(b2, d_model, "b2")
        a.ln_gamma = _f32vec(ln_gamma, H * dv, "ln_gamma")
        a.ln_beta = _f32vec(ln_beta, H * dv, "ln_beta")
        a.ln_eps = float(ln_eps)
        self.args = a
        self.device = x.device


def hstu_layer_workspace_size(x, w1, b1, w2, b2, **kw) -> int:
    lib = _abi.load()
    c = _LayerCall(x, w1, b1, w2, b2, **_layer_kw(kw))
    return int(lib.hstu_layer_workspace_size(ctypes.byref(c.args)))


def _layer_kw(kw):
    d = dict(ln_gamma=None, ln_beta=None, ln_eps=1e-6, seq_offsets=None, max_seqlen=None, batch=None,
             num_targets=None, causal=True, softmax=False, alpha=0.0, groups=(HstuGroup(),),
             schedule=0, rab_timestamps=None, rab_time=None, rab_pos=None, out=None)
    unknown = set(kw) - set(d) - {"nhead", "hdim_qk", "hdim_v"}
    if unknown:
        raise TypeError(f"unknown arguments {sorted(unknown)}")
    d.update(kw)
    return d


def hstu_layer(x, w1, b1, w2, b2, *, workspace=None, stream=None, **kw):
    """One HSTU layer: out = x + ((LayerNorm(A) * ln_gamma + ln_beta) * U) w2^T + b2 with
    [U | V | Q | K] = SiLU(x w1^T + b1) and A the attention on Q, K, V.  Keywords:
    nhead, hdim_qk, hdim_v (required); seq_offsets + max_seqlen (jagged) or batch;
    the attention's mask, groups and rab_* as for hstu_fwd; ln_gamma, ln_beta, ln_eps.
    The workspace (uint8 device tensor, hstu_layer_workspace_size bytes) is allocated
    when not given."""
    lib = _abi.load()
    with _on(stream):
        c = _LayerCall(x, w1, b1, w2, b2, **_layer_kw(kw))
        need = int(lib.hstu_layer_workspace_size(ctypes.byref(c.args)))
        if need == 0:
            # invalid arguments (the call reports which) or nothing to compute
            _abi.check(lib.hstu_layer_fwd(ctypes.byref(c.args), None, 0, _stream_ptr(x.device, stream)))
            return c.out
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        _abi.check(lib.hstu_layer_fwd(ctypes.byref(c.args), ctypes.c_void_p(workspace.data_ptr()),
                                      workspace.numel(), _stream_ptr(x.device, stream)))
    return c.out

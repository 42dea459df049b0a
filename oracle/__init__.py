"""CPU oracle of the HSTU attention forward operator (ctypes wrapper of hstu_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
cpu_baseline leg may use it; the product path (the HIP library and its Python
binding) never imports it.  The C source states, step by step, what is computed
and which passage of the pages each step follows.

Parity status (what pins each function, see tests/test_oracle_*.py):
  * mask rule     - pinned by brute-force enumeration (oracle/mask_enum.py), the
                    closed-form per-row interval counts, and the invariants the
                    pages state (targets excluded, context always visible,
                    lower-triangular when only causal).  Its agreement with CK's
                    own mask code cannot be checked here: the readings of the
                    open points are listed in the C source header.
  * SiLU forward  - pinned by the pages' worked mass example (HSTU explainer
                    section 3.4) and by the dense causal special case.
  * softmax + LSE - pinned by torch scaled_dot_product_attention in float64
                    (causal and full special cases) and the worked example.
  * relative attention bias - the time-gap buckets pinned by the explainer's
                    bucket table (tests/golden/rab_time_buckets.json); the bias
                    as a whole by SDPA with an additive float mask (softmax) and
                    the dense SiLU product with the bias added (SiLU).
  * HSTU layer (oracle/layer.py: f1 + SiLU + split, attention, norm * gate,
                    f2 + residual) - pinned by an independent torch float64
                    evaluation and the zero-gate / zero-f2 identities.

Precision: the default build evaluates in double precision; load_fp32() gives
the same C source built with ORACLE_FP32 (single precision throughout a row),
and tests/test_oracle_fp32.py bounds the difference between the two.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hstu_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_LIB32_PATH = os.path.join(_HERE, "liboracle32.so")
_lib = None
_lib32 = None

_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)

_PROBLEM = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64p, _i64p, _i32p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
            _i32p, _i32p, _i32p, _f64p]


def build(src: str = _SRC, out: str = _LIB_PATH, extra_flags=()) -> str:
    """Compile the oracle with gcc (plain C, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", *extra_flags, src, "-o",
           out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def build_fp32(out: str = _LIB32_PATH, extra_flags=()) -> str:
    """Compile the single-precision build of the oracle."""
    return build(out=out, extra_flags=["-DORACLE_FP32", *extra_flags])


def load_fp32():
    """The single-precision build (compiled first if missing or older than the source);
    pass it as lib= to any function below."""
    global _lib32
    if _lib32 is None:
        if not os.path.exists(_LIB32_PATH) or os.path.getmtime(_LIB32_PATH) < os.path.getmtime(_SRC):
            build_fp32()
        _lib32 = load(_LIB32_PATH)
    return _lib32


def load(path: Optional[str] = None):
    """Load the compiled oracle (compiling it first if it is not built)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p) or (path is None and os.path.getmtime(p) < os.path.getmtime(_SRC)):
        build(out=p)
    lib = ctypes.CDLL(p)
    lib.oracle_mask.argtypes = [ctypes.c_int] * 8 + [_u8p]
    lib.oracle_hstu_fwd.argtypes = _PROBLEM + [_f32p, _f32p, _f32p, _f64p, _f64p, _i64p,
                                               ctypes.c_int]
    lib.oracle_hstu_rows.argtypes = _PROBLEM + [_f32p, _f32p, _f32p, ctypes.c_int, _i32p, _i32p,
                                                _i32p, _f64p, _f64p, ctypes.c_int]
    lib.oracle_count_pairs.argtypes = _PROBLEM + [_i64p]
    lib.oracle_seq_info.argtypes = _PROBLEM + [_i32p, _f64p]
    lib.oracle_hstu_fwd_rab.argtypes = _PROBLEM + [_i32p, _f64p, _f64p, ctypes.c_int, _f32p, _f32p,
                                                   _f32p, _f64p, _f64p, _i64p, ctypes.c_int]
    lib.oracle_hstu_rows_rab.argtypes = _PROBLEM + [_i32p, _f64p, _f64p, ctypes.c_int, _f32p, _f32p,
                                                    _f32p, ctypes.c_int, _i32p, _i32p, _i32p, _f64p,
                                                    _f64p, ctypes.c_int]
    lib.oracle_rab_bucket.argtypes = [ctypes.c_int64]
    lib.oracle_rab_bucket.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    for f in ("oracle_mask", "oracle_hstu_fwd", "oracle_hstu_fwd_rab", "oracle_hstu_rows",
              "oracle_hstu_rows_rab",
              "oracle_count_pairs", "oracle_seq_info"):
        getattr(lib, f).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray], t):
    if a is None:
        return ctypes.cast(None, t)
    return a.ctypes.data_as(t)


class Problem:
    """Scalars and metadata of one call, in the oracle's own terms."""

    def __init__(self, *, batch, nhead, hdim_qk, hdim_v, q_offsets, kv_offsets, num_targets,
                 cross, causal, softmax, alpha, local_lens, context_lens, minfull_lens,
                 attn_scales):
        self.B, self.H, self.Dqk, self.Dv = int(batch), int(nhead), int(hdim_qk), int(hdim_v)
        self.q_off = np.ascontiguousarray(q_offsets, np.int64)
        self.kv_off = np.ascontiguousarray(kv_offsets, np.int64)
        self.tg = None if num_targets is None else np.ascontiguousarray(num_targets, np.int32)
        self.cross, self.causal, self.softmax = int(bool(cross)), int(bool(causal)), int(bool(softmax))
        self.alpha = float(alpha)
        self.gL = np.ascontiguousarray(local_lens, np.int32)
        self.gC = np.ascontiguousarray(context_lens, np.int32)
        self.gM = np.ascontiguousarray(minfull_lens, np.int32)
        self.ga = np.ascontiguousarray(attn_scales, np.float64)
        self.G = len(self.gL)

    def args(self):
        return (self.B, self.H, self.Dqk, self.Dv, _ptr(self.q_off, _i64p), _ptr(self.kv_off, _i64p),
                _ptr(self.tg, _i32p), self.cross, self.causal, self.softmax, self.alpha, self.G,
                _ptr(self.gL, _i32p), _ptr(self.gC, _i32p), _ptr(self.gM, _i32p),
                _ptr(self.ga, _f64p))

    @property
    def total_q(self):
        return int(self.q_off[-1])


def problem_of(w) -> Problem:
    """The oracle's view of a workloads.Workload."""
    return Problem(batch=w.batch, nhead=w.nhead, hdim_qk=w.hdim_qk, hdim_v=w.hdim_v,
                   q_offsets=w.q_offsets, kv_offsets=w.kv_offsets, num_targets=w.targets,
                   cross=w.cross, causal=w.causal, softmax=w.softmax, alpha=w.alpha,
                   local_lens=[g.local_len for g in w.groups],
                   context_lens=[g.context_len for g in w.groups],
                   minfull_lens=[g.minfull_len for g in w.groups],
                   attn_scales=[g.attn_scale for g in w.groups])


def _f32(a):
    return np.ascontiguousarray(a, np.float32)


def mask(S_q, S_kv, context_len, num_targets, cross, local_len, minfull_len, causal, lib=None):
    """Dense mask of one sequence, uint8 [S_q, S_kv] (1 = attended)."""
    lib = lib or load()
    m = np.zeros((S_q, S_kv), np.uint8)
    rc = lib.oracle_mask(S_q, S_kv, context_len, num_targets, int(cross), local_len, minfull_len,
                         int(causal), _ptr(m, _u8p))
    assert rc == 0
    return m


def forward(p: Problem, q, k, v, nthreads: int = 0, lib=None):
    """Whole forward. Returns (o [total_q,H,Dv] f64, lse [total_q,H] f64 or None, pairs)."""
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    o = np.zeros((p.total_q, p.H, p.Dv), np.float64)
    lse = np.zeros((p.total_q, p.H), np.float64) if p.softmax else None
    pairs = np.zeros(1, np.int64)
    rc = lib.oracle_hstu_fwd(*p.args(), _ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p),
                             _ptr(o, _f64p), _ptr(lse, _f64p), _ptr(pairs, _i64p), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_hstu_fwd rejected its arguments")
    return o, lse, int(pairs[0])


def forward_rab(p: Problem, q, k, v, timestamps=None, time_table=None, pos_table=None,
                nthreads: int = 0, lib=None):
    """Whole forward with the relative attention bias (self-attention only).
    timestamps: int32 [tokens] or None; time_table [H, 11]; pos_table [H, P] or None.
    Returns (o, lse, pairs) like forward()."""
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    ts = None if timestamps is None else np.ascontiguousarray(timestamps, np.int32)
    tt = None if time_table is None else np.ascontiguousarray(time_table, np.float64)
    pt = None if pos_table is None else np.ascontiguousarray(pos_table, np.float64)
    P = 0 if pt is None else int(pt.shape[1])
    o = np.zeros((p.total_q, p.H, p.Dv), np.float64)
    lse = np.zeros((p.total_q, p.H), np.float64) if p.softmax else None
    pairs = np.zeros(1, np.int64)
    rc = lib.oracle_hstu_fwd_rab(*p.args(), _ptr(ts, _i32p), _ptr(tt, _f64p), _ptr(pt, _f64p), P,
                                 _ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p), _ptr(o, _f64p),
                                 _ptr(lse, _f64p), _ptr(pairs, _i64p), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_hstu_fwd_rab rejected its arguments")
    return o, lse, int(pairs[0])


def rows_rab(p: Problem, q, k, v, rows_b, rows_h, rows_i, timestamps=None, time_table=None,
             pos_table=None, nthreads: int = 0, lib=None):
    """Selected rows with the relative attention bias (arguments as rows() and forward_rab())."""
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    ts = None if timestamps is None else np.ascontiguousarray(timestamps, np.int32)
    tt = None if time_table is None else np.ascontiguousarray(time_table, np.float64)
    pt = None if pos_table is None else np.ascontiguousarray(pos_table, np.float64)
    P = 0 if pt is None else int(pt.shape[1])
    rb = np.ascontiguousarray(rows_b, np.int32)
    rh = np.ascontiguousarray(rows_h, np.int32)
    ri = np.ascontiguousarray(rows_i, np.int32)
    n = len(rb)
    o = np.zeros((n, p.Dv), np.float64)
    lse = np.zeros(n, np.float64) if p.softmax else None
    rc = lib.oracle_hstu_rows_rab(*p.args(), _ptr(ts, _i32p), _ptr(tt, _f64p), _ptr(pt, _f64p), P,
                                  _ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p), n, _ptr(rb, _i32p),
                                  _ptr(rh, _i32p), _ptr(ri, _i32p), _ptr(o, _f64p), _ptr(lse, _f64p),
                                  int(nthreads))
    if rc != 0:
        raise ValueError("oracle_hstu_rows_rab rejected its arguments")
    return o, lse


def rab_bucket(d: int, lib=None) -> int:
    """Time-gap bucket (0..10) of a gap of d seconds."""
    return int((lib or load()).oracle_rab_bucket(int(d)))


def rows(p: Problem, q, k, v, rows_b, rows_h, rows_i, nthreads: int = 0, lib=None):
    """Selected rows (b, h, i-in-sequence). Returns (o [n,Dv] f64, lse [n] f64 or None)."""
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    rb = np.ascontiguousarray(rows_b, np.int32)
    rh = np.ascontiguousarray(rows_h, np.int32)
    ri = np.ascontiguousarray(rows_i, np.int32)
    n = len(rb)
    o = np.zeros((n, p.Dv), np.float64)
    lse = np.zeros(n, np.float64) if p.softmax else None
    rc = lib.oracle_hstu_rows(*p.args(), _ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p), n,
                              _ptr(rb, _i32p), _ptr(rh, _i32p), _ptr(ri, _i32p), _ptr(o, _f64p),
                              _ptr(lse, _f64p), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_hstu_rows rejected its arguments")
    return o, lse


def count_pairs(p: Problem, lib=None) -> np.ndarray:
    """Visible (i, j) pairs of each sequence, per head."""
    lib = lib or load()
    out = np.zeros(p.B, np.int64)
    rc = lib.oracle_count_pairs(*p.args(), _ptr(out, _i64p))
    if rc != 0:
        raise ValueError("oracle_count_pairs rejected its arguments")
    return out


def num_threads(lib=None) -> int:
    """OpenMP threads the oracle's parallel loops use by default."""
    return int((lib or load()).oracle_num_threads())


def seq_info(p: Problem, lib=None):
    """Per-sequence (Cq, Uq, Tq, Ck, Ukv, Tk) and resolved attn_scale."""
    lib = lib or load()
    info = np.zeros((p.B, 6), np.int32)
    scale = np.zeros(p.B, np.float64)
    rc = lib.oracle_seq_info(*p.args(), _ptr(info, _i32p), _ptr(scale, _f64p))
    if rc != 0:
        raise ValueError("oracle_seq_info rejected its arguments")
    return info, scale

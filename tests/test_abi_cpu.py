"""The C-ABI library without a GPU: it loads, exports every declared symbol, and
rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from recsys_attention_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_abi.LIB_PATH):
        from recsys_attention_amd import build
        build.build()
    return _abi.load()


def _declared_functions():
    out = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        out |= set(re.findall(r"\b(hstu_[a-z_]+)\s*\(", text))
    return out


def test_header_symbols_exported(lib):
    declared = _declared_functions()
    assert declared == set(_abi.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.hstu_abi_version() == _abi.HSTU_ABI_VERSION


def _args(**over):
    """A valid jagged bf16 hdim-128 argument block with fake (never dereferenced) pointers."""
    groups = (_abi.MaskGroupC * 1)()
    groups[0].local_len, groups[0].context_len, groups[0].minfull_len = 5, 6, 6
    groups[0].attn_scale, groups[0].max_uih_q = 0.0, 870
    a = _abi.FwdArgsC(dtype=_abi.HSTU_BF16, batch=10, nhead=4, hdim_qk=128, hdim_v=128,
                      jagged=1, cross=0, seqlen_q=881, seqlen_kv=881, total_q=8038,
                      q=0x10000, k=0x20000, v=0x30000, o=0x40000, seq_offsets_q=0x50000,
                      num_targets=0x60000, causal=1, softmax=0, alpha=0.0, num_groups=1,
                      schedule=0)
    a.groups = ctypes.cast(groups, ctypes.POINTER(_abi.MaskGroupC))
    a._keep = groups
    for k, v in over.items():
        if k == "group":
            for gk, gv in v.items():
                setattr(groups[0], gk, gv)
        else:
            setattr(a, k, v)
    return a


def test_valid_args_pass(lib):
    assert lib.hstu_validate_args(ctypes.byref(_args())) == _abi.HSTU_OK
    rab = dict(rab_timestamps=0xb0000, rab_time=0xc0000, rab_pos=0xa0000,
               rab_pos_len=_abi.HSTU_RAB_MAX_POS)
    assert lib.hstu_validate_args(ctypes.byref(_args(**rab))) == _abi.HSTU_OK
    assert lib.hstu_validate_args(ctypes.byref(_args(rab_pos=0xa0000, rab_pos_len=1))) == _abi.HSTU_OK


@pytest.mark.parametrize("over,status", [
    (dict(dtype=7), _abi.HSTU_ERR_INVALID_ARG),
    (dict(batch=-1), _abi.HSTU_ERR_INVALID_ARG),
    (dict(nhead=0), _abi.HSTU_ERR_INVALID_ARG),
    (dict(hdim_qk=96, hdim_v=128), _abi.HSTU_ERR_UNSUPPORTED),
    (dict(hdim_qk=80, hdim_v=80), _abi.HSTU_ERR_UNSUPPORTED),
    (dict(hdim_qk=32, hdim_v=32), _abi.HSTU_ERR_UNSUPPORTED),
    (dict(seq_offsets_q=None), _abi.HSTU_ERR_INVALID_ARG),
    (dict(cross=1), _abi.HSTU_ERR_INVALID_ARG),            # jagged cross without kv offsets
    (dict(q=None), _abi.HSTU_ERR_INVALID_ARG),
    (dict(o=0x40008), _abi.HSTU_ERR_INVALID_ARG),           # misaligned
    (dict(q_tok_stride=100), _abi.HSTU_ERR_INVALID_ARG),    # < nhead * hdim
    (dict(q_tok_stride=516), _abi.HSTU_ERR_INVALID_ARG),    # not a multiple of 8
    (dict(num_groups=3), _abi.HSTU_ERR_INVALID_ARG),        # 10 % 3 != 0
    (dict(num_groups=0), _abi.HSTU_ERR_INVALID_ARG),
    (dict(groups=None), _abi.HSTU_ERR_INVALID_ARG),
    (dict(group=dict(local_len=-1)), _abi.HSTU_ERR_INVALID_ARG),
    (dict(group=dict(max_uih_q=-1)), _abi.HSTU_ERR_INVALID_ARG),  # attn_scale 0 needs it
    (dict(alpha=float("nan")), _abi.HSTU_ERR_INVALID_ARG),
    (dict(lse=0x70000), _abi.HSTU_ERR_INVALID_ARG),         # lse without softmax
    (dict(causal=2), _abi.HSTU_ERR_INVALID_ARG),
    (dict(schedule=4), _abi.HSTU_ERR_INVALID_ARG),
    (dict(jagged=0, seqlen_kv=5), _abi.HSTU_ERR_INVALID_ARG),  # batched self needs equal lengths
    # relative attention bias
    (dict(cross=1, seq_offsets_kv=0x58000, rab_pos=0xa0000, rab_pos_len=8), _abi.HSTU_ERR_UNSUPPORTED),
    (dict(rab_timestamps=0xb0000), _abi.HSTU_ERR_INVALID_ARG),              # no time table
    (dict(rab_timestamps=0xb0002, rab_time=0xc0000), _abi.HSTU_ERR_INVALID_ARG),  # misaligned
    (dict(rab_pos=0xa0000, rab_pos_len=0), _abi.HSTU_ERR_INVALID_ARG),
    (dict(rab_pos=0xa0000, rab_pos_len=_abi.HSTU_RAB_MAX_POS + 1), _abi.HSTU_ERR_INVALID_ARG),
])
def test_invalid_args_rejected(lib, over, status):
    a = _args(**over)
    assert lib.hstu_validate_args(ctypes.byref(a)) == status
    assert lib.hstu_last_error()
    # the compute entry points reject the same block before touching the GPU
    assert lib.hstu_fwd(ctypes.byref(a), None, 0, None) == status
    assert lib.hstu_count_visible_pairs(ctypes.byref(a), ctypes.c_void_p(0x80000), None) == status


def test_null_args(lib):
    assert lib.hstu_validate_args(None) == _abi.HSTU_ERR_INVALID_ARG
    assert lib.hstu_fwd(None, None, 0, None) == _abi.HSTU_ERR_INVALID_ARG


def test_workspace_size_and_checks(lib):
    a = _args(softmax=1)
    # schedule left to the library: room for the persistent schedule's queues
    # (a 256-byte header and 8 bytes per possible item: 40 (b, h) pairs, 7 q-tiles
    # of 128 rows for 881 rows, times the splits); an unsplit call on a grid too
    # small for the persistent schedule also gets room for cutting each
    # sequence's last two q-tiles (3 chunks: 40 x (7 + 2 x 2) = 440 work-groups
    # fit the chip's 512, 4 would not; 128 rows each, 128 fp32 columns plus an
    # LSE) and the cut q-tiles' records (8 bytes each)
    queue = 256 + 8 * 40 * 7
    slots_rows = 40 * 2 * 3 * 128
    meta = (40 * 2 * 8 + 255) // 256 * 256
    heavy = slots_rows * 128 * 4 + slots_rows * 4 + meta
    assert lib.hstu_fwd_workspace_size(ctypes.byref(a), 1) == (queue + 255) // 256 * 256 + heavy
    silu = _args(softmax=0)
    assert lib.hstu_fwd_workspace_size(ctypes.byref(silu), 1) == \
        (queue + 255) // 256 * 256 + slots_rows * 128 * 4 + meta
    # no room for chunks where none is cut: sequences of at most 4 key tiles
    # (256 keys), a grid that would fill the chip (hdim 256: one work-group per
    # CU, 40 x (7 + 2) = 360 work-groups with the fewest chunk slots), or an
    # explicit schedule
    short = _args(seqlen_q=256, seqlen_kv=256, total_q=2560)
    assert lib.hstu_fwd_workspace_size(ctypes.byref(short), 1) == 256 + 8 * 40 * 2
    wide = _args(hdim_qk=256, hdim_v=256)
    assert lib.hstu_fwd_workspace_size(ctypes.byref(wide), 1) == 256 + 8 * 40 * 7
    assert lib.hstu_fwd_workspace_size(ctypes.byref(_args(schedule=2)), 1) == 0
    n = lib.hstu_fwd_workspace_size(ctypes.byref(a), 16)
    rows = 8038 * 4 * 16
    o_bytes = (rows * 128 * 4 + 255) // 256 * 256
    lse_bytes = (rows * 4 + 255) // 256 * 256
    assert n == o_bytes + lse_bytes + 256 + 8 * 40 * 7 * 16
    # a schedule without counters needs no workspace of its own
    a2 = _args(softmax=1, schedule=2)
    assert lib.hstu_fwd_workspace_size(ctypes.byref(a2), 1) == 0
    assert lib.hstu_fwd_workspace_size(ctypes.byref(a2), 16) == o_bytes + lse_bytes
    assert lib.hstu_fwd_workspace_size(ctypes.byref(a), 0) == 0
    assert lib.hstu_fwd_workspace_size(ctypes.byref(a), _abi.HSTU_MAX_SPLITS + 1) == 0
    # missing or short workspace is reported before any launch
    assert lib.hstu_fwd_splitkv(ctypes.byref(a), 16, None, 0, None) == _abi.HSTU_ERR_WORKSPACE
    assert lib.hstu_fwd_splitkv(ctypes.byref(a), 16, ctypes.c_void_p(0x90000), o_bytes + lse_bytes - 1,
                                None) == _abi.HSTU_ERR_WORKSPACE
    assert lib.hstu_fwd_splitkv(ctypes.byref(a), 0, None, 0, None) == _abi.HSTU_ERR_INVALID_ARG
    # the persistent schedule asked for explicitly needs its counters
    a3 = _args(softmax=1, schedule=3)
    assert lib.hstu_fwd(ctypes.byref(a3), None, 0, None) == _abi.HSTU_ERR_WORKSPACE
    q1 = 256 + 8 * 40 * 7
    assert lib.hstu_fwd(ctypes.byref(a3), ctypes.c_void_p(0x90000), q1 - 1, None) == _abi.HSTU_ERR_WORKSPACE
    assert lib.hstu_fwd(ctypes.byref(a3), ctypes.c_void_p(0x90008), q1, None) == _abi.HSTU_ERR_WORKSPACE
    assert lib.hstu_fwd_splitkv(ctypes.byref(a3), 16, ctypes.c_void_p(0x90000), n - 1,
                                None) == _abi.HSTU_ERR_WORKSPACE


def test_status_strings(lib):
    for s, name in [(0, "HSTU_OK"), (1, "HSTU_ERR_INVALID_ARG"), (2, "HSTU_ERR_UNSUPPORTED"),
                    (3, "HSTU_ERR_WORKSPACE"), (4, "HSTU_ERR_HIP")]:
        assert lib.hstu_status_string(s).decode() == name


def test_product_path_does_not_use_the_oracle():
    """The HIP library and its binding never import, link or call the oracle."""
    pkg = os.path.join(ROOT, "recsys_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f
                assert "workloads" not in text, f


def test_binding_raises_without_library(tmp_path):
    saved = _abi._lib
    _abi._lib = None
    try:
        with pytest.raises(RuntimeError):
            _abi.load(str(tmp_path / "missing.so"))
    finally:
        _abi._lib = saved


# ----------------------------------------------------------- the layer entry points

def _linear(**over):
    a = _abi.LinearArgsC(dtype=_abi.HSTU_BF16, rows=1000, in_features=512, out_features=2048,
                         x=0x100000, x_stride=0, w=0x200000, bias=0x300000,
                         activation=_abi.HSTU_ACT_SILU, residual=None, residual_stride=0,
                         y=0x400000, y_stride=0)
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,status", [
    (dict(dtype=5), _abi.HSTU_ERR_INVALID_ARG),
    (dict(rows=-1), _abi.HSTU_ERR_INVALID_ARG),
    (dict(in_features=96), _abi.HSTU_ERR_UNSUPPORTED),       # not a multiple of 64
    (dict(out_features=12), _abi.HSTU_ERR_UNSUPPORTED),      # not a multiple of 8
    (dict(activation=3), _abi.HSTU_ERR_INVALID_ARG),
    (dict(x=None), _abi.HSTU_ERR_INVALID_ARG),
    (dict(bias=0x300004), _abi.HSTU_ERR_INVALID_ARG),        # misaligned
    (dict(x_stride=500), _abi.HSTU_ERR_INVALID_ARG),         # shorter than a row
    (dict(x_stride=516), _abi.HSTU_ERR_INVALID_ARG),         # not a multiple of 8
    (dict(x_stride=(1 << 22) + 8), _abi.HSTU_ERR_UNSUPPORTED),  # beyond the 32-bit tile range
    (dict(residual=0x500000, residual_stride=100), _abi.HSTU_ERR_INVALID_ARG),
])
def test_linear_invalid_args_rejected(lib, over, status):
    assert lib.hstu_linear_fwd(ctypes.byref(_linear(**over)), None) == status
    assert lib.hstu_last_error()


def test_linear_empty_is_a_no_op(lib):
    assert lib.hstu_linear_fwd(ctypes.byref(_linear(rows=0)), None) == _abi.HSTU_OK


def _norm(**over):
    a = _abi.NormGateArgsC(dtype=_abi.HSTU_BF16, rows=10, width=512, a=0x100000, a_stride=0,
                           u=0x200000, u_stride=2048, gamma=None, beta=None, eps=1e-6, z=0x100000,
                           z_stride=0)
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,status", [
    (dict(width=4104), _abi.HSTU_ERR_UNSUPPORTED),
    (dict(width=12), _abi.HSTU_ERR_UNSUPPORTED),
    (dict(eps=0.0), _abi.HSTU_ERR_INVALID_ARG),
    (dict(eps=float("nan")), _abi.HSTU_ERR_INVALID_ARG),
    (dict(u=None), _abi.HSTU_ERR_INVALID_ARG),
    (dict(z_stride=1024), _abi.HSTU_ERR_INVALID_ARG),        # in place with another stride
    (dict(gamma=0x300008), _abi.HSTU_ERR_INVALID_ARG),
])
def test_norm_gate_invalid_args_rejected(lib, over, status):
    assert lib.hstu_norm_gate_fwd(ctypes.byref(_norm(**over)), None) == status


def _layer(attn, **over):
    """A valid layer block around the attention block attn (which the caller keeps
    alive: it owns the host group array the library reads)."""
    a = _abi.LayerArgsC()
    a.attn = attn  # jagged, 10 sequences, 4 heads of 128, 8038 tokens
    a.d_model, a.x, a.w1, a.b1, a.w2, a.b2, a.out = 512, 0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000
    a.ln_eps = 1e-6
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_layer_workspace_size(lib):
    attn = _args()
    a = _layer(attn)
    n, H, d = 8038, 4, 128
    proj = (n * 2 * H * (d + d) * 2 + 255) // 256 * 256
    att = (n * H * d * 2 + 255) // 256 * 256
    # the attention's workspace: its work queues, and (a grid too small for the
    # persistent schedule) the heavy q-tiles' chunk partials and records
    queue = (256 + 8 * 40 * 7 + 255) // 256 * 256 + 40 * 2 * 3 * 128 * 128 * 4 + (40 * 2 * 8 + 255) // 256 * 256
    assert lib.hstu_layer_workspace_size(ctypes.byref(a)) == proj + att + queue
    assert lib.hstu_layer_fwd(ctypes.byref(a), None, 0, None) == _abi.HSTU_ERR_WORKSPACE
    assert lib.hstu_layer_fwd(ctypes.byref(a), ctypes.c_void_p(0x700000), proj + att + queue - 1,
                              None) == _abi.HSTU_ERR_WORKSPACE
    assert lib.hstu_layer_fwd(ctypes.byref(a), ctypes.c_void_p(0x700010), proj + att + queue,
                              None) == _abi.HSTU_ERR_WORKSPACE  # not 256-byte aligned


@pytest.mark.parametrize("attn_over,over,status", [
    (dict(cross=1, seq_offsets_kv=0x58000), {}, _abi.HSTU_ERR_UNSUPPORTED),
    ({}, dict(d_model=100), _abi.HSTU_ERR_UNSUPPORTED),
    ({}, dict(w2=None), _abi.HSTU_ERR_INVALID_ARG),
    ({}, dict(ln_eps=-1.0), _abi.HSTU_ERR_INVALID_ARG),
    (dict(hdim_qk=80, hdim_v=80), {}, _abi.HSTU_ERR_UNSUPPORTED),
    ({}, dict(b2=0x500004), _abi.HSTU_ERR_INVALID_ARG),
])
def test_layer_invalid_args_rejected(lib, attn_over, over, status):
    attn = _args(**attn_over)
    a = _layer(attn, **over)
    assert lib.hstu_layer_workspace_size(ctypes.byref(a)) == 0
    assert lib.hstu_layer_fwd(ctypes.byref(a), ctypes.c_void_p(0x700000), 1 << 30, None) == status


def test_layer_checks_the_attention_on_its_strided_views(lib):
    """The layer's Q/K/V are views of the projection (token stride 2H(dqk+dv)), so a
    sequence length the attention accepts on dense tensors can exceed its 32-bit
    per-sequence range here; the layer must refuse before its first launch."""
    attn = _args(seqlen_q=1_100_000, seqlen_kv=1_100_000, total_q=1_100_000)
    dense = attn
    assert lib.hstu_validate_args(ctypes.byref(dense)) == _abi.HSTU_OK  # dense: 1.1 GB per sequence
    a = _layer(attn)
    assert lib.hstu_layer_workspace_size(ctypes.byref(a)) == 0
    assert lib.hstu_layer_fwd(ctypes.byref(a), ctypes.c_void_p(0x700000), 1 << 40,
                              None) == _abi.HSTU_ERR_UNSUPPORTED
    assert b"4 GiB" in lib.hstu_last_error()


def test_layer_rejects_f2_width_before_any_launch(lib):
    """One head of 96/96 makes H dv = 96, which f2 (input width a multiple of 64)
    does not take: the layer must say so before its first launch, not after f1,
    the attention and the norm-gate have run."""
    attn = _args(nhead=1, hdim_qk=96, hdim_v=96)
    a = _layer(attn)
    assert lib.hstu_layer_workspace_size(ctypes.byref(a)) == 0
    assert lib.hstu_layer_fwd(ctypes.byref(a), ctypes.c_void_p(0x700000), 1 << 30,
                              None) == _abi.HSTU_ERR_UNSUPPORTED
    assert b"in_features 96" in lib.hstu_last_error()
    # three heads of 96 (H dv = 288) are refused too; four (384) are taken
    assert lib.hstu_layer_workspace_size(ctypes.byref(_layer(_args(nhead=3, hdim_qk=96, hdim_v=96)))) == 0
    attn4 = _args(nhead=4, hdim_qk=96, hdim_v=96)
    assert lib.hstu_layer_workspace_size(ctypes.byref(_layer(attn4))) > 0


def test_layer_with_no_tokens_is_a_no_op(lib):
    """An empty problem (no sequences, no tokens) launches nothing and needs no
    workspace."""
    attn = _args(batch=0, total_q=0, seq_offsets_q=None, num_targets=None)
    a = _layer(attn)
    assert lib.hstu_layer_fwd(ctypes.byref(a), None, 0, None) == _abi.HSTU_OK


def test_noalloc_rejects_beyond_the_static_scratch(lib):
    """The allocation-free entry point refuses, before any HIP call, a problem whose
    workspace exceeds its static scratch (here 128 splits of 8038 rows x 4 heads x
    128 fp32 partial columns)."""
    a = _args()
    need = lib.hstu_fwd_workspace_size(ctypes.byref(a), 128)
    assert need > _abi.HSTU_NOALLOC_SCRATCH_BYTES
    assert lib.hstu_fwd_splitkv_noalloc(ctypes.byref(a), 128, None) == _abi.HSTU_ERR_WORKSPACE
    assert b"static scratch" in lib.hstu_last_error()
    assert lib.hstu_fwd_splitkv_noalloc(ctypes.byref(a), 0, None) == _abi.HSTU_ERR_INVALID_ARG
    assert lib.hstu_fwd_splitkv_noalloc(ctypes.byref(_args(dtype=9)), 1, None) == _abi.HSTU_ERR_INVALID_ARG

"""The ctypes mirror of the C argument blocks (recsys_attention_amd/_abi.py) against
the header: a host program built with gcc from include/hstu.h and
include/hstu_layer.h prints every field's offset and each struct's size, which
must equal what ctypes lays out."""
import ctypes
import os
import shutil
import subprocess

import pytest

from recsys_attention_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

STRUCTS = {
    "hstu_mask_group_t": _abi.MaskGroupC,
    "hstu_fwd_args_t": _abi.FwdArgsC,
    "hstu_linear_args_t": _abi.LinearArgsC,
    "hstu_norm_gate_args_t": _abi.NormGateArgsC,
    "hstu_layer_args_t": _abi.LayerArgsC,
}


def _program():
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "hstu.h"', '#include "hstu_layer.h"',
             'int main(void) {']
    for cname, cls in STRUCTS.items():
        lines.append(f'    printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'    printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ['    return 0;', '}']
    return "\n".join(lines) + "\n"


def test_ctypes_mirror_matches_the_header(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc needed")
    src = tmp_path / "layout.c"
    src.write_text(_program())
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I" + os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for ln in out:
        if ln:
            parts = ln.split()
            got[tuple(parts[:-1])] = int(parts[-1])
    for cname, cls in STRUCTS.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got[(cname, fname)] == getattr(cls, fname).offset, (cname, fname)

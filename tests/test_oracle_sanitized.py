"""The oracle's C code built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, OpenMP) and run in a child process over small problems covering every entry
point (dense mask, whole forward, selected rows, pair counts, sequence info, the
biased forward and rows, the bucket function), in both builds (double and
single precision): no sanitizer report, and the same results as the regular
build of the same precision within its rounding."""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys, numpy as np
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, workloads as W
lib = oracle.load({lib!r})
out = {{}}
for seed, kw in enumerate([dict(softmax=False, jagged=True), dict(softmax=True, jagged=False),
                           dict(softmax=True, jagged=True, cross=True),
                           dict(softmax=False, jagged=True, causal=False)]):
    w = W.random_workload(900 + seed, hdim_qk=64, batch=3, nhead=2, max_uih=40, **kw)
    p = oracle.problem_of(w)
    o, lse, pairs = oracle.forward(p, w.q, w.k, w.v, nthreads=2, lib=lib)
    out[f"o{{seed}}"] = o
    if lse is not None:
        out[f"lse{{seed}}"] = lse
    out[f"pairs{{seed}}"] = np.array([pairs])
    out[f"count{{seed}}"] = oracle.count_pairs(p, lib=lib)
    info, scale = oracle.seq_info(p, lib=lib)
    out[f"info{{seed}}"], out[f"scale{{seed}}"] = info, scale
    rb = [0, 1, 2, 2]; rh = [0, 1, 0, 1]; ri = [0, 1, 2, w.seqlen_q[2] - 1]
    r, rl = oracle.rows(p, w.q, w.k, w.v, rb, rh, ri, lib=lib)
    out[f"rows{{seed}}"] = r
    if not w.cross:
        rab = W.rab_inputs(w, 910 + seed, pos_len=17)
        o2, _, _ = oracle.forward_rab(p, w.q, w.k, w.v, timestamps=rab.timestamps,
                                      time_table=rab.time_table, pos_table=rab.pos_table,
                                      nthreads=2, lib=lib)
        out[f"rab{{seed}}"] = o2
        r2, _ = oracle.rows_rab(p, w.q, w.k, w.v, rb, rh, ri, timestamps=rab.timestamps,
                                time_table=rab.time_table, pos_table=rab.pos_table, lib=lib)
        out[f"rabrows{{seed}}"] = r2
out["mask"] = oracle.mask(23, 23, 3, 4, 0, 5, 6, 1, lib=lib)
out["xmask"] = oracle.mask(17, 30, 2, 3, 1, 4, 0, 1, lib=lib)
out["buckets"] = np.array([oracle.rab_bucket(d, lib=lib) for d in (0, 1, 4, 5, 2599999, 2600000, 2**40)])
np.savez({npz!r}, **out)
print("child ok", flush=True)
'''


def _libasan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _run_child(lib_path, npz, preload=None):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    if preload:
        env["LD_PRELOAD"] = preload
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib_path, npz=npz)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                          timeout=600)


@pytest.mark.parametrize("precision", ["fp64", "fp32"])
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path, precision):
    asan = _libasan()
    if shutil.which("gcc") is None or asan is None:
        pytest.skip("gcc with libasan needed")
    mode = ["-DORACLE_FP32"] if precision == "fp32" else []
    plain = oracle.build(out=str(tmp_path / "liboracle_plain.so"), extra_flags=mode)
    san = oracle.build(out=str(tmp_path / "liboracle_san.so"),
                       extra_flags=[*mode, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                    "-fno-omit-frame-pointer"])
    r_plain = _run_child(plain, str(tmp_path / "plain.npz"))
    assert r_plain.returncode == 0, r_plain.stderr[-3000:]
    r_san = _run_child(san, str(tmp_path / "san.npz"), preload=asan)
    assert r_san.returncode == 0 and "child ok" in r_san.stdout, r_san.stderr[-4000:]
    assert "runtime error" not in r_san.stderr and "AddressSanitizer" not in r_san.stderr, r_san.stderr[-4000:]
    a, b = np.load(tmp_path / "plain.npz"), np.load(tmp_path / "san.npz")
    assert sorted(a.files) == sorted(b.files)
    for k in a.files:
        x, y = a[k], b[k]
        if x.dtype.kind == "f":
            tol = dict(rtol=1e-12, atol=1e-15) if precision == "fp64" else dict(rtol=1e-6, atol=1e-9)
            assert np.allclose(x, y, equal_nan=True, **tol), k
        else:
            assert np.array_equal(x, y), k

"""The forward kernels' planner (recsys_attention_amd/csrc/hstu_plan.h) compiled for
the host with AddressSanitizer and UndefinedBehaviorSanitizer, checked against the
oracle's dense masks (tests/plan_check.cpp lists the checks): the interval form
equals the rule form, skipped key tiles hold no visible pair, EMPTY / FULL tiles
(per row and for the whole work-group) are right, split ranges partition the
tiles, and counting by tile classes gives the mask's pair count.

The pattern follows the OpenTau flash_attn_cuda page's module docstring: a compact
mask representation is checked to reproduce the dense mask."""
import itertools
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "plan_check.cpp")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _build(out, sanitize=True):
    cmd = ["g++", "-std=c++17", "-O1", "-g", *(SAN if sanitize else []),
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "recsys_attention_amd", "csrc"), SRC, "-o", out]
    subprocess.run(cmd, check=True)
    return out


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    return _build(str(tmp_path_factory.mktemp("plan") / "plan_check"))


def _case_text(S_q, S_kv, C, T, cross, L, M, causal, mask=None):
    if mask is None:
        mask = oracle.mask(S_q, S_kv, C, T, cross, L, M, causal)
    body = "".join(mask.reshape(-1).astype(np.uint8).astype(str)) if mask.size else "-"
    return f"{S_q} {S_kv} {C} {T} {int(cross)} {L} {M} {int(causal)}\n{body}\n"


def _run(checker, text):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([checker], input=text, capture_output=True, text=True, env=env,
                          timeout=600)


def _assert_ok(res, n):
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert res.stdout.strip().startswith(f"checked {n} cases"), res.stdout[-500:]


def test_planner_self_attention_exhaustive(checker):
    """Every C in 0..3, U in 0..12, T in 0..3, L in 0..4, M in 0..4, causal or not."""
    cases = []
    for C, U, T, L, M, causal in itertools.product(range(4), range(13), range(4), range(5), range(5),
                                                   (0, 1)):
        S = C + U + T
        cases.append(_case_text(S, S, C, T, 0, L, M, causal))
    _assert_ok(_run(checker, "".join(cases)), len(cases))


def test_planner_cross_attention_sweep(checker):
    """Cross-attention (keys without targets): U_q in 0..12, U_kv in 0..14."""
    cases = []
    for C, Uq, Ukv, T, L, M, causal in itertools.product(range(4), range(13), range(15), range(4),
                                                         (0, 2, 4), (0, 3), (0, 1)):
        cases.append(_case_text(C + Uq + T, C + Ukv, C, T, 1, L, M, causal))
    _assert_ok(_run(checker, "".join(cases)), len(cases))


def test_planner_mid_size_random(checker):
    """Sequences of a few hundred events: the kernels' own tiles (128 query rows; 32,
    64 and 128 keys) with ragged tails, every mask component."""
    rng = np.random.default_rng(4242)
    cases = []
    for _ in range(40):
        C, T = int(rng.integers(0, 12)), int(rng.integers(0, 40))
        Uq = int(rng.integers(0, 600))
        cross = bool(rng.integers(0, 4) == 0)
        Ukv = int(rng.integers(0, 700)) if cross else Uq
        L, M = int(rng.choice([0, 1, 5, 64, 200])), int(rng.choice([0, 6, 100]))
        causal = bool(rng.integers(0, 5))
        cases.append(_case_text(C + Uq + T, C + Ukv + (0 if cross else T), C, T, cross, L, M, causal))
    _assert_ok(_run(checker, "".join(cases)), len(cases))


def test_planner_check_is_sensitive(checker):
    """A mask with one pair flipped (a visible pair hidden, or a hidden one shown)
    must fail the check: the checker compares, it does not merely run."""
    m = oracle.mask(40, 40, 3, 4, 0, 5, 6, 1)
    for flip in [(20, 18), (20, 30), (39, 1), (0, 35)]:
        bad = m.copy()
        bad[flip] ^= 1
        res = _run(checker, _case_text(40, 40, 3, 4, 0, 5, 6, 1, mask=bad))
        assert res.returncode == 1 and "FAIL" in res.stdout, (flip, res.stdout)

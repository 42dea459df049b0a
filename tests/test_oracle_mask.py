"""Pins of the oracle's mask rule (CPU only).

The rule in oracle/hstu_oracle.c is checked against
  * a brute-force enumerator written separately (oracle/mask_enum.py),
  * per-row closed-form counts of the visible keys (interval lengths),
  * the invariants the pages state for each mask component (CK example README,
    "Masking" table), and
  * pair counts worked out by hand for the README's example workloads.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle import mask_enum


def _row_counts_closed_form(S_q, S_kv, C, T, cross, L, M, causal):
    """Visible keys per row from interval lengths (causal only)."""
    assert causal
    Cq = min(C, S_q)
    Tq = min(T, S_q - Cq)
    Uq = S_q - Cq - Tq
    Ck = min(C, S_kv)
    Tk = 0 if cross else min(T, S_kv - Ck)
    Ukv = S_kv - Ck - Tk
    counts = []
    for i in range(S_q):
        if i < Cq:
            counts.append(Ck)
            continue
        if i < Cq + Uq:
            u = i - Cq
            x = u + Ukv - Uq
            full = L == 0 or (M > 0 and u >= Uq - M)
        else:
            x = Ukv
            full = L == 0 or M > 0
        hi = min(x, Ukv - 1)
        lo = 0 if full else max(0, x - L)
        counts.append(Ck + max(0, hi - lo + 1))
    return counts


def test_mask_matches_enumerator_self_attention():
    lib = oracle.load()
    n = 0
    for C, U, T, L, M, causal in itertools.product(range(4), range(13), range(4), range(5),
                                                    range(5), (0, 1)):
        S = C + U + T
        m = oracle.mask(S, S, C, T, False, L, M, causal, lib=lib)
        ref = np.array(mask_enum.enumerate_mask(S, S, C, T, False, L, M, causal),
                       dtype=np.uint8).reshape(S, S)
        assert np.array_equal(m, ref), (C, U, T, L, M, causal)
        if causal:
            cf = _row_counts_closed_form(S, S, C, T, False, L, M, True)
            assert list(m.sum(axis=1)) == cf, (C, U, T, L, M)
        n += 1
    assert n == 4 * 13 * 4 * 5 * 5 * 2


def test_mask_matches_enumerator_cross_attention():
    lib = oracle.load()
    for C, Uq, T, Ukv, L, M, causal in itertools.product(range(3), range(9), range(3), range(13),
                                                          (0, 1, 3), (0, 2), (0, 1)):
        Sq, Skv = C + Uq + T, C + Ukv
        m = oracle.mask(Sq, Skv, C, T, True, L, M, causal, lib=lib)
        ref = np.array(mask_enum.enumerate_mask(Sq, Skv, C, T, True, L, M, causal),
                       dtype=np.uint8).reshape(Sq, Skv)
        assert np.array_equal(m, ref), (C, Uq, T, Ukv, L, M, causal)
        if causal:
            assert list(m.sum(axis=1)) == _row_counts_closed_form(Sq, Skv, C, T, True, L, M, True)


@pytest.mark.parametrize("C,U,T,L,M", [(0, 9, 0, 0, 0), (3, 7, 2, 2, 0), (2, 12, 3, 3, 4),
                                       (4, 20, 5, 6, 7), (1, 5, 0, 0, 3)])
def test_mask_invariants(C, U, T, L, M):
    S = C + U + T
    m = oracle.mask(S, S, C, T, False, L, M, True).astype(bool)
    # targets: no row sees a target key, including a target's own diagonal
    assert not m[:, C + U:].any()
    # contextual: every row sees every context key
    assert m[:, :C].all()
    # causal: no UIH row sees a later UIH key
    for i in range(C, C + U):
        assert not m[i, i + 1:C + U].any()
    # context rows see nothing but the context under causal masking
    assert not m[:C, C:].any()
    # local: with M = 0 every target row sees the C context keys plus the
    # min(L, U) most recent UIH keys
    if M == 0 and L > 0:
        for i in range(C + U, S):
            assert m[i].sum() == C + min(L, U)
            assert m[i, C + U - min(L, U):C + U].all()
    # min-full: the last M UIH rows see their whole causal history
    for u in range(max(0, U - M), U):
        assert m[C + u, C:C + u + 1].all()


def test_plain_causal_is_lower_triangular():
    """With only the causal component active the mask is the lower triangle with diagonal."""
    for S in (1, 2, 7, 33):
        m = oracle.mask(S, S, 0, 0, False, 0, 0, True)
        assert np.array_equal(m, np.tril(np.ones((S, S), np.uint8)))
        full = oracle.mask(S, S, 0, 0, False, 0, 0, False)
        assert full.all()


def test_local_window_shape():
    """Local window: the diagonal plus the L previous UIH keys (no context, no targets)."""
    S, L = 16, 3
    m = oracle.mask(S, S, 0, 0, False, L, 0, True)
    ref = np.tril(np.ones((S, S), np.uint8)) - np.tril(np.ones((S, S), np.uint8), -L - 1)
    assert np.array_equal(m, ref)
    # non-causal local: a symmetric band
    m2 = oracle.mask(S, S, 0, 0, False, L, 0, False)
    ref2 = np.triu(np.tril(np.ones((S, S), np.uint8), L), -L)
    assert np.array_equal(m2, ref2)


def test_pair_count_readme_batched_example():
    """B=2, H=2, U=64, T=4, C=2, L=5, M=6, causal: 1098 pairs per (sequence, head).

    By hand: 2 context rows x 2; UIH rows u<58 see 2 + min(u,5)+1; the 6
    min-full rows see 2 + u + 1; 4 target rows see 2 + 64.
    """
    hand = 2 * 2 + sum(2 + min(u, 5) + 1 for u in range(58)) + \
        sum(2 + u + 1 for u in range(58, 64)) + 4 * (2 + 64)
    assert hand == 1098
    m = oracle.mask(70, 70, 2, 4, False, 5, 6, True)
    assert int(m.sum()) == 1098


def test_pair_count_readme_jagged_example():
    """The README's jagged invocation (C=6, L=5, M=6): per-sequence counts by hand."""
    U = [750, 730, 733, 860, 870, 788, 760, 821, 833, 779]
    T = [5, 5, 6, 6, 5, 6, 5, 6, 4, 6]
    C, L, M = 6, 5, 6
    p = oracle.Problem(batch=10, nhead=4, hdim_qk=128, hdim_v=128,
                       q_offsets=np.concatenate([[0], np.cumsum([C + u + t for u, t in zip(U, T)])]),
                       kv_offsets=np.concatenate([[0], np.cumsum([C + u + t for u, t in zip(U, T)])]),
                       num_targets=T, cross=False, causal=True, softmax=False, alpha=0.0,
                       local_lens=[L], context_lens=[C], minfull_lens=[M], attn_scales=[0.0])
    per = oracle.count_pairs(p)
    for b in range(10):
        u_, t_ = U[b], T[b]
        hand = C * C  # context rows
        hand += sum(C + min(u, L) + 1 for u in range(u_ - M))
        hand += sum(C + u + 1 for u in range(u_ - M, u_))
        hand += t_ * (C + u_)
        assert per[b] == hand, b
    assert list(per) == [17250, 16790, 17598, 20646, 20010, 18918, 17480, 19710, 18320, 18702]
    assert int(per.sum()) * 4 == 741696


def test_pair_count_cross_example():
    """Cross attention U_q=64, T=8, U_kv=16384, C=6, causal, L=0: bottom-right aligned."""
    C, Uq, T, Ukv = 6, 64, 8, 16384
    hand = C * C + sum(C + (u + Ukv - Uq) + 1 for u in range(Uq)) + T * (C + Ukv)
    p = oracle.Problem(batch=1, nhead=1, hdim_qk=8, hdim_v=8, q_offsets=[0, C + Uq + T],
                       kv_offsets=[0, C + Ukv], num_targets=[T], cross=True, causal=True,
                       softmax=True, alpha=0.0, local_lens=[0], context_lens=[C],
                       minfull_lens=[0], attn_scales=[1.0])
    assert int(oracle.count_pairs(p)[0]) == hand == 1178100


def test_degenerate_lengths_are_clamped():
    """S < C + T: context takes what fits, then targets, and U = 0."""
    m = oracle.mask(3, 3, 5, 2, False, 0, 0, True)
    assert m.all()  # every key is context, visible to all
    m = oracle.mask(4, 4, 2, 5, False, 0, 0, True)
    assert np.array_equal(m[:, :2], np.ones((4, 2), np.uint8)) and not m[:, 2:].any()
    m = oracle.mask(0, 0, 2, 1, False, 0, 0, True)
    assert m.shape == (0, 0)

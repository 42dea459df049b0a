"""Brute-force enumerator of the HSTU functional mask (second, independent encoding).

TEST INFRASTRUCTURE ONLY.  Pure-Python loops for tiny sequences; it shares no
code with hstu_oracle.c (which encodes the same rule in C) nor with the HIP
library (which uses per-row key intervals).  The mask is built here as the
composite of the components of the CK example README's "Masking" table, each
evaluated on its own and then combined:

  targets      - target keys are excluded from attention
  contextual   - context keys are visible to every query
  causal       - on the UIH axis a query sees no later key; context queries
                 come before every UIH key
  local        - a query sees keys within local_len of its UIH position
                 (0 disables the component)
  min-full     - the last minfull_len UIH queries (and the target queries that
                 follow them) are exempt from the local component

Positions: query row i of a sequence ``[C | U_q | T]`` gets a UIH-axis
position: context rows -1, UIH row u -> u + (U_kv - U_q), target rows U_kv;
UIH key v has position v.
"""
from __future__ import annotations

from typing import List


def _split(S: int, C: int, T: int):
    c = min(C, S)
    t = min(max(T, 0), S - c)
    return c, S - c - t, t


def enumerate_mask(S_q: int, S_kv: int, context_len: int, num_targets: int, cross: bool,
                   local_len: int, minfull_len: int, causal: bool) -> List[List[bool]]:
    Cq, Uq, Tq = _split(S_q, context_len, num_targets)
    Ck, Ukv, Tk = _split(S_kv, context_len, 0 if cross else num_targets)
    q_kind = ["ctx"] * Cq + ["uih"] * Uq + ["tgt"] * Tq
    k_kind = ["ctx"] * Ck + ["uih"] * Ukv + ["tgt"] * Tk
    q_pos = [-1] * Cq + [u + (Ukv - Uq) for u in range(Uq)] + [Ukv] * Tq
    k_pos = [None] * Ck + list(range(Ukv)) + [None] * Tk
    tail_start = Cq + Uq - minfull_len  # first row of the min-full tail

    out = []
    for i in range(S_q):
        row = []
        for j in range(S_kv):
            if k_kind[j] == "tgt":
                row.append(False)          # targets component
                continue
            if k_kind[j] == "ctx":
                row.append(True)           # contextual component
                continue
            if causal:
                causal_ok = q_kind[i] != "ctx" and q_pos[i] >= k_pos[j]
            else:
                causal_ok = True
            exempt = minfull_len > 0 and (q_kind[i] == "tgt" or
                                          (q_kind[i] == "uih" and i >= tail_start))
            local_ok = local_len == 0 or exempt or abs(q_pos[i] - k_pos[j]) <= local_len
            row.append(causal_ok and local_ok)
        out.append(row)
    return out


def count(mask) -> int:
    return sum(sum(1 for x in row if x) for row in mask)

"""Exact size of the selected sets, sum_i |M(i)| (test infrastructure only).

The algorithmic attention work of a head is 4 d sum_i |M(i)| FLOP (QK^T and PV,
two FLOP per multiply-add), counted here from the index sets themselves.
"""
import numpy as np


def selected_count_dense(nq, q_offset=0):
    p = np.arange(nq, dtype=np.int64) + q_offset
    return int((p + 1).sum())


def selected_count_vs(nq, nk, V, S, q_offset=0):
    """sum_i |{j <= p_i : j in V} u {p_i - o : o in S, o <= p_i}|."""
    V = np.sort(np.asarray(V, dtype=np.int64))
    S = np.sort(np.asarray(S, dtype=np.int64))
    p = np.arange(nq, dtype=np.int64) + q_offset
    cols = np.searchsorted(V, p, side="right").sum()
    diags = np.searchsorted(S, p, side="right").sum()
    # pairs (j, o) with j + o = p for a valid query position count twice above
    lo, hi = q_offset, q_offset + nq - 1
    both = 0
    for start in range(0, V.size, 256):
        pos = V[start:start + 256, None] + S[None, :]
        both += int(((pos >= lo) & (pos <= hi)).sum())
    return int(cols + diags - both)


def selected_count_block(nq, nk, sel, block, q_offset=0):
    total = 0
    nqb = -(-(nq + q_offset) // block)
    for I in range(q_offset // block, nqb):
        r0 = max(I * block, q_offset)
        r1 = min((I + 1) * block, q_offset + nq)   # rows r0..r1-1 (positions)
        if r1 <= r0:
            continue
        p = np.arange(r0, r1, dtype=np.int64)
        for J in sel[I]:
            lo = J * block
            hi = np.minimum(np.minimum(lo + block, p + 1), nk)
            total += int(np.maximum(hi - lo, 0).sum())
    return total

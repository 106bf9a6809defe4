"""Masked causal softmax attention in float64 (test infrastructure only).

[MInf] section "how it works" and the authors' abstract: attention is computed
only at the positions the head's pattern and indices select.  This is the
plain definition the sparse kernel must reproduce:

    z_ij  = q_i . k_j / sqrt(d)               for j in M(i)
    O_i   = sum_j exp(z_ij - m_i) v_j / sum_j exp(z_ij - m_i)
    LSE_i = m_i + ln sum_j exp(z_ij - m_i)

M(i) is a set, so an entry chosen by two rules counts once.  An empty M(i)
gives O_i = 0 and LSE_i = -inf (reading; the pages never speak of empty rows).
"""
import numpy as np


def masked_attention(q, k, v, mask, scale=None):
    """q [Nq, d], k and v [Nk, d], mask [Nq, Nk] bool -> (O [Nq, d], LSE [Nq])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    z = (q @ k.T) * scale
    z = np.where(mask, z, -np.inf)
    m = z.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.where(mask, np.exp(z - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = (e @ v) / np.where(empty, 1.0, l)[:, None]
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    o[empty] = 0.0
    return o, lse


def attention_rows(q, k, v, rows, row_sets, scale=None):
    """The same definition for selected query rows only.

    rows: query row indices; row_sets: the index array M(i) of each row.
    Returns (O [len(rows), d], LSE [len(rows)]).
    """
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    O = np.zeros((len(rows), v.shape[1]))
    L = np.full(len(rows), -np.inf)
    for n, (i, idx) in enumerate(zip(rows, row_sets)):
        idx = np.unique(np.asarray(idx, dtype=np.int64))
        if idx.size == 0:
            continue
        kk = np.asarray(k[idx], dtype=np.float64)
        vv = np.asarray(v[idx], dtype=np.float64)
        z = (kk @ q[i]) * scale
        m = z.max()
        e = np.exp(z - m)
        O[n] = (e @ vv) / e.sum()
        L[n] = m + np.log(e.sum())
    return O, L

"""Indexer token top-k and its routed variant, in float64.

TEST INFRASTRUCTURE ONLY (see the package header).

[MISA] section "the big problem": the DeepSeek-style sparse attention indexer
scores every key with 64 lightweight heads and keeps the best tokens; the main
attention then reads only those.  Section "how MISA works, step by step": a
router that looks at the keys in large blocks picks 8 of the 64 heads for each
query, and only those heads score tokens.

Readings (the explainer gives no formulas):
  * score_ij = sum_{h in H(i)} w_ih * max(0, q_ih . k_j) for causal j <= p_i,
    one indexer key per token shared by all heads, no 1/sqrt(d) scale.
  * Router (parity unpinned beyond brute force): kbar_J is the bf16-rounded
    mean of 64 indexer keys, over complete causal blocks (64 J + 63 <= p_i);
    r_ih = w_ih * max(0, max_J q_ih . kbar_J); H(i) = the `route_heads` heads of
    largest r_ih, ties to the lower head.
"""
import numpy as np

from .rules import block_means, topk_rule


def indexer_row(q_i, k_idx, w_i, p, heads=None):
    """Scores of one query (q_i [Hi, di], w_i [Hi]) against keys 0..p."""
    q_i = np.asarray(q_i, dtype=np.float64)
    w_i = np.asarray(w_i, dtype=np.float64)
    kk = np.asarray(k_idx[:p + 1], dtype=np.float64)
    hs = np.arange(q_i.shape[0]) if heads is None else np.asarray(heads, dtype=np.int64)
    dots = kk @ q_i[hs].T                          # [p+1, |H|]
    return np.maximum(dots, 0.0) @ w_i[hs]


def indexer_scores(q_idx, k_idx, w, q_offset, heads=None):
    """[Nq, Nk] scores, -inf where j > p_i.  heads: None or [Nq, r] indices."""
    nq = q_idx.shape[0]
    nk = k_idx.shape[0]
    out = np.full((nq, nk), -np.inf)
    for i in range(nq):
        p = i + q_offset
        out[i, :p + 1] = indexer_row(q_idx[i], k_idx, w[i], p, None if heads is None else heads[i])
    return out


def router_heads(q_idx, k_idx, w, q_offset, route_heads=8, block=64, rows=None):
    """Routed head set H(i) (ascending head indices) for each query row."""
    q_idx = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    kbar = block_means(k_idx, block)
    rows = range(q_idx.shape[0]) if rows is None else rows
    out = []
    for i in rows:
        p = i + q_offset
        ncomplete = (p + 1) // block                 # blocks J with 64J + 63 <= p
        if ncomplete == 0:
            r = np.zeros(q_idx.shape[1])
        else:
            best = (kbar[:ncomplete] @ q_idx[i].T).max(axis=0)   # [Hi]
            r = w[i] * np.maximum(best, 0.0)
        out.append(topk_rule(r, np.arange(q_idx.shape[1]), route_heads))
    return np.array(out, dtype=np.int64)


def token_topk(scores_row, p, k):
    """Top-k keys of one query among j <= p, ascending."""
    return topk_rule(scores_row, np.arange(p + 1), k)


def hierarchical_tokens(q_idx, k_idx, w, q_offset, route_heads, cand, k, block=64, rows=None):
    """Two-stage token selection of MISA's hierarchical variant, per query row.

    [MISA] section "how MISA works", the hierarchical option: first the
    router's few heads score the keys and keep a larger candidate list; then
    all of the indexer heads score only those candidates, and the best of
    them are kept.  Readings (the explainer gives no sizes or formulas):
      * stage 1: H(i) = router_heads(...); candidates C(i) = top-`cand` keys
        j <= p_i by the routed score (ties to the lower index);
      * stage 2: the dense score (all heads) of each candidate; the result is
        the top-`k` of C(i) by that score (ties to the lower index), ascending,
        min(k, |C(i)|) keys.
    Parity unpinned beyond brute force and the special cases that reduce it
    to the dense or the routed indexer (cand >= p_i + 1; route_heads = all
    heads; cand = k).
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    rows = range(q_idx.shape[0]) if rows is None else rows
    rows = list(rows)
    heads = router_heads(q_idx, k_idx, w, q_offset, route_heads, block, rows=rows)
    out = []
    for n, i in enumerate(rows):
        p = i + q_offset
        routed = indexer_row(q_idx[i], k_idx, w[i], p, heads[n])
        c_set = topk_rule(routed, np.arange(p + 1), cand)
        full = np.full(p + 1, -np.inf)
        full[c_set] = indexer_row(q_idx[i], np.asarray(k_idx)[c_set], w[i], len(c_set) - 1)
        out.append(topk_rule(full, c_set, k))
    return out

"""Vertical and slash discovery from pooled block scores, in float64.

TEST INFRASTRUCTURE ONLY (see the package header).

[FP] section 2.1 says that one fast search over blocks, with keys represented
by their block means, finds the three sparse shapes of an attention map at
once: vertical (a key that matters wherever it appears), slash (a run of
diagonals) and block.  The page gives no rule that turns block scores into
columns or diagonals.  Reading (O-22), the plainest one the rest of the pages
support:

  1. pooled scores S[I, J] = qbar_I . kbar_J / sqrt(d), J <= I, as the block
     rule computes them (block_means + block_scores);
  2. the block-level attention of each query block: P[I, :] = softmax over
     J <= I of S[I, J] (the Vertical-Slash rule of [MInf] works on attention
     weights too, of the last queries);
  3. the vertical mass of key block J, vbar[J] = sum over I >= J of P[I, J],
     and the slash mass of block offset D, sbar[D] = sum over I >= D of
     P[I, I - D];
  4. the top `nv_blocks` key blocks by vbar and the top `ns_blocks` offsets by
     sbar (ties to the lower index);
  5. expansion to token sets: the columns are every key of a kept block,
     cols = union of [J B, min((J + 1) B, N)); the diagonals are every token
     offset i - j of a pair (i, j) whose blocks lie D apart, which is
     [max(0, D B - (B - 1)), min(N - 1, D B + (B - 1))] for each kept D.

The result is a Vertical-Slash index set, so the attention takes it like any
other.  Parity unpinned as to the choice of rule (the page states none); the
functions are pinned by brute force, by the row-sum invariant, by a closed form
(equal scores give harmonic sums), and by the reduction to the Vertical-Slash
scores of every row when blocks are single tokens.
"""
import numpy as np

from .rules import topk_rule


def pooled_vs_scores(S, q_block0=0):
    """vbar [nkb] and sbar [nkb] from a block score matrix S (-inf beyond the
    causal bound): the column and block-diagonal sums of the row-softmax of S.

    Row r of S is absolute query block I = q_block0 + r (block_scores of a
    prefill chunk): its softmax runs over J <= I and its slash terms are the
    offsets D = I - J, so sbar has one entry per key block offset."""
    S = np.asarray(S, dtype=np.float64)
    nq, nk = S.shape
    vbar = np.zeros(nk)
    sbar = np.zeros(nk)
    for r in range(nq):
        I = q_block0 + r
        row = S[r, :I + 1]
        e = np.exp(row - row.max())
        p = e / e.sum()
        vbar[:I + 1] += p
        # offset D = I - J: J = I .. 0 gives D = 0 .. I
        sbar[:I + 1] += p[::-1]
    return vbar, sbar


def pooled_vs_blocks(vbar, sbar, nv_blocks, ns_blocks):
    """Kept key blocks and block offsets (ascending, ties to the lower index)."""
    return (topk_rule(vbar, np.arange(len(vbar)), nv_blocks),
            topk_rule(sbar, np.arange(len(sbar)), ns_blocks))


def expand_blocks(Vb, Sb, block, nk):
    """Token columns and token diagonals of kept key blocks and block offsets."""
    cols = np.zeros(nk, dtype=bool)
    for J in np.asarray(Vb, dtype=np.int64):
        cols[J * block:min((J + 1) * block, nk)] = True
    diags = np.zeros(nk, dtype=bool)
    for D in np.asarray(Sb, dtype=np.int64):
        lo, hi = max(0, D * block - (block - 1)), min(nk - 1, D * block + (block - 1))
        if lo <= hi:
            diags[lo:hi + 1] = True
    return np.flatnonzero(cols).astype(np.int64), np.flatnonzero(diags).astype(np.int64)


def pooled_vs_sets(q, k, block, nv_blocks, ns_blocks, q_offset=0):
    """The whole rule for one head: q [Nq, d], k [Nk, d] (bf16 values in
    float64; a prefill chunk whose first query sits at q_offset, a multiple of
    the block, Nq = Nk - q_offset).  Returns (cols, diags, vbar, sbar, Vb, Sb)."""
    from .rules import block_means, block_scores
    assert q_offset % block == 0
    qb0 = q_offset // block
    S = block_scores(block_means(q, block), block_means(k, block), q_block0=qb0)
    vbar, sbar = pooled_vs_scores(S, q_block0=qb0)
    Vb, Sb = pooled_vs_blocks(vbar, sbar, nv_blocks, ns_blocks)
    cols, diags = expand_blocks(Vb, Sb, block, np.asarray(k).shape[0])
    return cols, diags, vbar, sbar, Vb, Sb

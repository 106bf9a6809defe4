"""Index rules of dynamic sparse prefill attention, in float64.

TEST INFRASTRUCTURE ONLY (see the package header).

Conventions.  One head at a time: ``q`` is [Nq, d], ``k`` is [Nk, d], both
float64 arrays holding bf16 values.  Query row i sits at absolute position
p_i = i + q_offset (a prefill chunk ends at the last key, so Nq = Nk - q_offset).
Every selection orders candidates by (score descending, index ascending), so
ties go to the lower index, and returns indices in ascending order.
"""
import numpy as np

from .bf16 import round_bf16


# ---------------------------------------------------------------------------
# Block rule: mean-pooled blocks, block-level scores, top-k or threshold.
# [MInf] section "inference-time dynamic masks" (Block-Sparse heads pool Q and K
# per block and score blocks); [FP] section 2.1 (mean-pooled keys as block
# representatives) and section 2.2 (max-based threshold); [MoBA] section
# FlashMoBA (top-k over key-block centroids).
# ---------------------------------------------------------------------------
def block_means(x, block):
    """Mean of each run of `block` rows of x [N, d], rounded to bf16.

    The pages leave the precision of the pooled vectors open.  Reading: the
    exact mean (the float64 sum of at most a few hundred bf16 values is exact,
    and dividing by a power of two is exact) rounded once to bf16, the form a
    matrix-core scoring step consumes.  A partial last block is averaged over
    its real rows (that division rounds once in float64, correctly).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    nb = -(-n // block)
    out = np.empty((nb, x.shape[1]), dtype=np.float64)
    for b in range(nb):
        rows = x[b * block:min(n, (b + 1) * block)]
        out[b] = rows.sum(axis=0) / rows.shape[0]
    return round_bf16(out)


def block_scores(qbar, kbar, scale=None, q_block0=0):
    """S[I, J] = qbar_I . kbar_J * scale for J <= q_block0 + I, -inf beyond.

    Row I of qbar is absolute query block q_block0 + I: a prefill chunk whose
    first query sits at q_offset = q_block0 * block pools its own rows, and its
    block I sees the key blocks up to and including its own absolute block.
    The pages do not fix the scale; reading: 1/sqrt(d), as in attention.
    """
    qbar = np.asarray(qbar, dtype=np.float64)
    kbar = np.asarray(kbar, dtype=np.float64)
    d = qbar.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    s = (qbar @ kbar.T) * scale
    nq, nk = s.shape
    causal = np.arange(nk)[None, :] <= np.arange(nq)[:, None] + q_block0
    return np.where(causal, s, -np.inf)


def topk_rule(scores, candidates, k):
    """The first min(k, |candidates|) candidates by (score desc, index asc).

    `candidates` is an integer index array into `scores`.  Returned ascending.
    """
    cand = np.asarray(candidates, dtype=np.int64)
    if cand.size == 0 or k <= 0:
        return np.zeros(0, dtype=np.int64)
    sc = np.asarray(scores, dtype=np.float64)[cand]
    order = np.lexsort((cand, -sc))      # primary key last: -score, then index
    return np.sort(cand[order[:k]])


def threshold_rule(scores, candidates, log_alpha):
    """Candidates J with S_J >= max_J' S_J' + ln(alpha).

    [FP] section 2.2 writes the threshold as alpha times the row maximum of the
    score.  For signed logits that product changes meaning when the maximum is
    negative; reading: the probability form, softmax weight >= alpha x the
    largest weight, which is the log form used here (inclusive).  The argmax
    always survives.
    """
    cand = np.asarray(candidates, dtype=np.int64)
    if cand.size == 0:
        return cand
    sc = np.asarray(scores, dtype=np.float64)[cand]
    keep = sc >= sc.max() + log_alpha
    return np.sort(cand[keep])


def select_blocks(S, mode, k=0, log_alpha=-np.log(20.0), force_first=False, force_diag=False, q_block0=0):
    """Selected key blocks Sel(I) for every absolute query block I.

    Row r of S is absolute query block I = q_block0 + r (block_scores of a
    prefill chunk).  Candidates are the block-causal J <= I.  Forced blocks
    (first block 0 and the diagonal block I) are added outside the budget:
    top-k runs over the other candidates, the threshold over all of J <= I.
    Reading for the forced blocks under the threshold rule: parity unpinned
    beyond brute force (the pages only pair forced blocks with top-k).
    The result is indexed by absolute query block; the q_block0 blocks before
    the chunk hold empty lists.
    """
    out = [np.zeros(0, dtype=np.int64) for _ in range(q_block0)]
    for r in range(S.shape[0]):
        I = q_block0 + r
        forced = set()
        if force_first:
            forced.add(0)
        if force_diag:
            forced.add(I)
        if mode == "topk":
            cand = [J for J in range(I + 1) if J not in forced]
            sel = set(topk_rule(S[r], cand, k).tolist())
        elif mode == "thresh":
            sel = set(threshold_rule(S[r], np.arange(I + 1), log_alpha).tolist())
        else:
            raise ValueError(mode)
        out.append(np.array(sorted(sel | forced), dtype=np.int64))
    return out


# ---------------------------------------------------------------------------
# Vertical-Slash rule.  [MInf] sections "three sparse patterns / Vertical-Slash"
# and "inference-time dynamic masks": the last `last_q` queries are scored
# against every key ("rough attention"), and important columns (vertical) and
# diagonals (slash) are kept.
# ---------------------------------------------------------------------------
def vs_scores(q_last, k, scale=None):
    """Column sums v[j] and diagonal sums s[o] of the causal softmax of the last
    rows.

    Row r of ``q_last`` [L, d] sits at position p_r = Nk - L + r.  Readings: the
    "rough attention" is the causal softmax over j <= p_r with scale 1/sqrt(d);
    v[j] = sum_r p[r, j]; s[o] = sum_r p[r, p_r - o] over rows with p_r - o >= 0
    (offset o = i - j; offsets seen by fewer rows keep their smaller sums).
    """
    q_last = np.asarray(q_last, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    L, d = q_last.shape
    nk = k.shape[0]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    z = (q_last @ k.T) * scale                       # [L, Nk]
    v = np.zeros(nk)
    s = np.zeros(nk)
    for r in range(L):
        pr = nk - L + r
        zr = z[r, :pr + 1]
        e = np.exp(zr - zr.max())
        p = e / e.sum()
        v[:pr + 1] += p
        # key j = pr - o  <=>  o = pr - j; j runs 0..pr so o runs pr..0
        s[:pr + 1] += p[::-1]
    return v, s


def vs_select(v, s, nv, ns):
    """Top-nv columns of v and top-ns offsets of s, each over [0, Nk)."""
    n = len(v)
    return topk_rule(v, np.arange(n), nv), topk_rule(s, np.arange(n), ns)


def ashape_sets(nk, sink, local):
    """A-shape as Vertical-Slash sets: columns [0, sink), offsets [0, local).

    [MInf] section "three sparse patterns / A-shape": sink tokens at the start
    plus a local window; a static mask.  Readings: token-exact edges, the
    window counts the query itself (i - j < local).
    """
    return np.arange(min(sink, nk), dtype=np.int64), np.arange(min(local, nk), dtype=np.int64)


# ---------------------------------------------------------------------------
# Masks M(i) as dense boolean matrices (small sizes) or per-row index sets.
# ---------------------------------------------------------------------------
def _positions(nq, nk, q_offset):
    return np.arange(nq)[:, None] + q_offset, np.arange(nk)[None, :]


def mask_dense(nq, nk, q_offset=0):
    p, j = _positions(nq, nk, q_offset)
    return j <= p


def mask_vs(nq, nk, V, S, q_offset=0):
    """M(i) = {j <= p_i : j in V or p_i - j in S}."""
    p, j = _positions(nq, nk, q_offset)
    inV = np.zeros(nk, dtype=bool)
    inV[np.asarray(V, dtype=np.int64)] = True
    inS = np.zeros(nk, dtype=bool)
    inS[np.asarray(S, dtype=np.int64)] = True
    off = p - j
    causal = off >= 0
    return causal & (inV[np.broadcast_to(j, off.shape)] | inS[np.clip(off, 0, nk - 1)])


def mask_block(nq, nk, sel, block, q_offset=0):
    """M(i) = {j <= p_i : floor(j / block) in Sel(floor(p_i / block))}."""
    p, j = _positions(nq, nk, q_offset)
    m = np.zeros((nq, nk), dtype=bool)
    for i in range(nq):
        pi = i + q_offset
        keyblocks = np.zeros(-(-nk // block), dtype=bool)
        keyblocks[sel[pi // block]] = True
        m[i] = keyblocks[np.arange(nk) // block]
    return m & (j <= p)


def mask_tokens(nq, nk, tok):
    m = np.zeros((nq, nk), dtype=bool)
    for i in range(nq):
        m[i, np.asarray(tok[i], dtype=np.int64)] = True
    return m


def row_set_dense(p):
    return np.arange(p + 1, dtype=np.int64)


def row_set_vs(p, V, S):
    V = np.asarray(V, dtype=np.int64)
    S = np.asarray(S, dtype=np.int64)
    cols = V[V <= p]
    diag = p - S[S <= p]
    return np.union1d(cols, diag)


def row_set_block(p, sel, block, nk):
    parts = [np.arange(J * block, min((J + 1) * block, p + 1, nk)) for J in sel[p // block]]
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(parts).astype(np.int64)

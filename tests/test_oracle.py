"""Pins of the fp64 oracle against brute force, closed forms and library routines.

Each test checks a rule of the oracle against something other than itself, so
that a dropped term, a wrong sign or index, or a transposed operand fails.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def bf16_array(shape, scale=1.0, rng=RNG):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * scale)
    return x.to(torch.bfloat16).to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------
def test_round_bf16_matches_torch_rne():
    x = (RNG.standard_normal(200000) * np.exp2(RNG.integers(-40, 40, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even one (1).
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: goes to 1 + 2^-6.
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -40])
    assert O.round_bf16(x).tolist() == [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7]


def _fraction_bf16(fr):
    """Round an exact rational to bf16 with integer arithmetic only."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    # a in [2^e, 2^(e+1)); keep 8 significant bits: grid 2^(e-7)
    scaled = a / (Fraction(2) ** (e - 7))
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n * Fraction(2) ** (e - 7))


# ---------------------------------------------------------------------------
# Block rule
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("block,n", [(4, 16), (4, 14), (8, 24)])
def test_block_means_exact_then_rne(block, n):
    x = bf16_array((n, 6), scale=3.0)
    got = O.block_means(x, block)
    for b in range(got.shape[0]):
        rows = x[b * block:(b + 1) * block]
        for c in range(x.shape[1]):
            exact = sum(Fraction(float(t)) for t in rows[:, c]) / rows.shape[0]
            assert got[b, c] == _fraction_bf16(exact)


def test_pool_bilinear_and_geometric_mean():
    # With unrounded means, qbar . kbar equals the mean of the B x B logit block,
    # and exp of it is the geometric mean of the block's exp(z).
    B, d = 8, 16
    q = bf16_array((B, d))
    k = bf16_array((B, d))
    z = q @ k.T / math.sqrt(d)
    qb, kb = q.mean(0), k.mean(0)
    s = qb @ kb / math.sqrt(d)
    assert abs(s - z.mean()) < 1e-12
    geo = math.exp(np.log(np.exp(z)).mean())
    assert abs(math.exp(s) - geo) < 1e-12 * geo


def test_block_scores_causal_and_scale():
    qb = bf16_array((5, 8))
    kb = bf16_array((5, 8))
    S = O.block_scores(qb, kb)
    for I in range(5):
        for J in range(5):
            if J > I:
                assert S[I, J] == -np.inf
            else:
                ref = sum(qb[I, c] * kb[J, c] for c in range(8)) / math.sqrt(8)
                assert abs(S[I, J] - ref) < 1e-12


def _brute_topk(scores, cand, k):
    cand = list(cand)
    k = min(k, len(cand))
    best = None
    for sub in itertools.combinations(sorted(cand), k):
        tot = sum(scores[j] for j in sub)
        key = (-tot, sub)
        if best is None or key < best:
            best = key
    return list(best[1]) if best else []


@pytest.mark.parametrize("trial", range(40))
def test_topk_matches_brute_force_with_ties(trial):
    rng = np.random.default_rng(trial)
    n = int(rng.integers(1, 9))
    scores = rng.integers(-2, 3, n).astype(np.float64)     # many exact ties
    cand = sorted(rng.choice(n, int(rng.integers(0, n + 1)), replace=False).tolist())
    k = int(rng.integers(0, n + 2))
    got = O.topk_rule(scores, cand, k).tolist()
    assert got == _brute_topk(scores, cand, k)
    # equals a full stable sort by (-score, index)
    srt = sorted(cand, key=lambda j: (-scores[j], j))[:k]
    assert got == sorted(srt)


@pytest.mark.parametrize("trial", range(30))
def test_threshold_probability_and_log_forms(trial):
    rng = np.random.default_rng(100 + trial)
    n = int(rng.integers(1, 12))
    s = rng.standard_normal(n) * 3
    alpha = 0.05
    got = O.threshold_rule(s, np.arange(n), math.log(alpha)).tolist()
    p = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    ref = [j for j in range(n) if p[j] >= alpha * p.max() * (1 - 1e-12)]
    assert got == ref
    assert int(np.argmax(s)) in got


def test_select_blocks_forced_topk_brute():
    rng = np.random.default_rng(7)
    S = O.block_scores(bf16_array((9, 8), rng=rng), bf16_array((9, 8), rng=rng))
    sel = O.select_blocks(S, "topk", k=3, force_first=True, force_diag=True)
    for I in range(9):
        assert len(sel[I]) == min(I + 1, 5)
        assert 0 in sel[I] and I in sel[I]
        rest = [J for J in range(1, I)]
        top = _brute_topk(S[I], rest, 3)
        assert sorted(set(top) | {0, I}) == sel[I].tolist()


def test_select_blocks_threshold_unforced():
    rng = np.random.default_rng(8)
    S = O.block_scores(bf16_array((7, 8), 4.0, rng), bf16_array((7, 8), 4.0, rng))
    sel = O.select_blocks(S, "thresh", log_alpha=-math.log(20))
    for I in range(7):
        row = S[I, :I + 1]
        ref = [J for J in range(I + 1) if row[J] >= row.max() - math.log(20)]
        assert sel[I].tolist() == ref


@pytest.mark.parametrize("mode", ["topk", "thresh"])
def test_block_rule_chunk_equals_full_prompt_rows(mode):
    # A prefill chunk whose first query sits at q_offset = q_block0 * block pools
    # the same rows as the whole prompt's query blocks q_block0.., so its scores,
    # selection, mask and attention equal the whole prompt's from there on.
    rng = np.random.default_rng(21)
    n, d, block, qb0 = 100, 16, 8, 5          # ragged last block
    q, k, v = bf16_array((n, d), 2.0, rng), bf16_array((n, d), 2.0, rng), bf16_array((n, d), rng=rng)
    off = qb0 * block
    kb = O.block_means(k, block)
    S_full = O.block_scores(O.block_means(q, block), kb)
    S_chunk = O.block_scores(O.block_means(q[off:], block), kb, q_block0=qb0)
    assert np.array_equal(S_chunk, S_full[qb0:])
    kw = dict(k=3, log_alpha=-math.log(20), force_first=True, force_diag=True)
    sel_full = O.select_blocks(S_full, mode, **kw)
    sel_chunk = O.select_blocks(S_chunk, mode, q_block0=qb0, **kw)
    assert len(sel_chunk) == len(sel_full)
    for I in range(len(sel_full)):
        assert sel_chunk[I].tolist() == (sel_full[I].tolist() if I >= qb0 else [])
    m_full = O.mask_block(n, n, sel_full, block)
    m_chunk = O.mask_block(n - off, n, sel_chunk, block, q_offset=off)
    assert np.array_equal(m_chunk, m_full[off:])
    o_f, l_f = O.masked_attention(q, k, v, m_full)
    o_c, l_c = O.masked_attention(q[off:], k, v, m_chunk)
    assert np.allclose(o_c, o_f[off:], atol=1e-13) and np.allclose(l_c, l_f[off:], atol=1e-13)
    # the forced diagonal is the absolute block, and every list stays causal
    for I in range(qb0, len(sel_chunk)):
        assert I in sel_chunk[I] and sel_chunk[I].max() <= I


# ---------------------------------------------------------------------------
# Vertical-Slash rule
# ---------------------------------------------------------------------------
def _vs_brute(q_last, k):
    L, d = q_last.shape
    n = k.shape[0]
    v = [0.0] * n
    s = [0.0] * n
    for r in range(L):
        pr = n - L + r
        z = [sum(q_last[r, c] * k[j, c] for c in range(d)) / math.sqrt(d) for j in range(pr + 1)]
        m = max(z)
        den = sum(math.exp(t - m) for t in z)
        for j in range(pr + 1):
            pj = math.exp(z[j] - m) / den
            v[j] += pj
            s[pr - j] += pj
    return np.array(v), np.array(s)


@pytest.mark.parametrize("n,L", [(12, 4), (9, 9), (20, 3)])
def test_vs_scores_brute_force(n, L):
    q = bf16_array((L, 8))
    k = bf16_array((n, 8))
    v, s = O.vs_scores(q, k)
    vb, sb = _vs_brute(q, k)
    assert np.allclose(v, vb, rtol=0, atol=1e-13)
    assert np.allclose(s, sb, rtol=0, atol=1e-13)


def test_vs_sums_invariant():
    L, n = 16, 300
    q = bf16_array((L, 32), 2.0)
    k = bf16_array((n, 32))
    v, s = O.vs_scores(q, k)
    assert abs(v.sum() - L) < 1e-12 and abs(s.sum() - L) < 1e-12
    assert v.min() >= 0 and s.min() >= 0 and v.max() <= L and s.max() <= L
    # the slash sum at offset 0 collects the diagonal of every row
    z = q @ k.T / math.sqrt(32)
    diag = 0.0
    for r in range(L):
        pr = n - L + r
        e = np.exp(z[r, :pr + 1] - z[r, :pr + 1].max())
        diag += e[pr] / e.sum()
    assert abs(s[0] - diag) < 1e-13


def test_vs_select_and_planted_columns():
    w = synth.vs_single(seed=11, N=512, nv=16, ns=16)
    q = O.to_f64(w.q[0, 0])
    k = O.to_f64(w.k[0, 0])
    v, s = O.vs_scores(q[-64:], k)
    V, S = O.vs_select(v, s, 16, 16)
    assert len(V) == 16 and len(S) == 16
    # planted keys (4x the last queries' mean direction) are among the top columns
    assert set(w.extra["planted_cols"].tolist()) <= set(V.tolist())


def test_ashape_equals_sink_plus_window():
    nq, nk, sink, local = 40, 40, 3, 7
    V, S = O.ashape_sets(nk, sink, local)
    m = O.mask_vs(nq, nk, V, S)
    for i in range(nq):
        for j in range(nk):
            assert m[i, j] == (j <= i and (j < sink or i - j < local))


# ---------------------------------------------------------------------------
# Masked attention
# ---------------------------------------------------------------------------
def _attn_brute(q, k, v, mask):
    nq, d = q.shape
    O_ = np.zeros((nq, v.shape[1]))
    L = np.full(nq, -np.inf)
    for i in range(nq):
        js = [j for j in range(k.shape[0]) if mask[i, j]]
        if not js:
            continue
        z = [sum(q[i, c] * k[j, c] for c in range(d)) / math.sqrt(d) for j in js]
        m = max(z)
        w = [math.exp(t - m) for t in z]
        den = sum(w)
        for c in range(v.shape[1]):
            O_[i, c] = sum(wj * v[j, c] for wj, j in zip(w, js)) / den
        L[i] = m + math.log(den)
    return O_, L


def _sdpa_causal(q, k, v):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)[0, 0].numpy()


def test_all_selected_masks_are_dense_attention():
    n, d = 24, 8
    q, k, v = bf16_array((n, d)), bf16_array((n, d)), bf16_array((n, d))
    dense = O.mask_dense(n, n)
    Vall, Sall = O.ashape_sets(n, 0, n)          # local >= N
    sel_all = O.select_blocks(O.block_scores(O.block_means(q, 4), O.block_means(k, 4)), "topk", k=99)
    tok = [np.arange(i + 1) for i in range(n)]
    for m in (O.mask_vs(n, n, Vall, Sall), O.mask_vs(n, n, np.arange(n), []),
              O.mask_block(n, n, sel_all, 4), O.mask_tokens(n, n, tok)):
        assert np.array_equal(m, dense)
    o, lse = O.masked_attention(q, k, v, dense)
    ob, lb = _attn_brute(q, k, v, dense)
    assert np.allclose(o, ob, atol=1e-13) and np.allclose(lse, lb, atol=1e-13)
    assert np.allclose(o, _sdpa_causal(q, k, v), atol=1e-12)


def test_random_masks_match_brute_force():
    n, d = 20, 8
    q, k, v = bf16_array((n, d)), bf16_array((n, d)), bf16_array((n, d))
    m = (RNG.random((n, n)) < 0.3) & O.mask_dense(n, n)
    o, lse = O.masked_attention(q, k, v, m)
    ob, lb = _attn_brute(q, k, v, m)
    assert np.allclose(o, ob, atol=1e-13)
    assert np.array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    assert np.allclose(lse[fin], lb[fin], atol=1e-13)


def test_empty_rows_give_zero_and_minus_inf():
    n, d = 12, 8
    q, k, v = bf16_array((n, d)), bf16_array((n, d)), bf16_array((n, d))
    m = O.mask_vs(n, n, [5], [])
    o, lse = O.masked_attention(q, k, v, m)
    assert np.all(o[:5] == 0) and np.all(np.isneginf(lse[:5]))
    assert np.allclose(o[5:], v[5][None, :], atol=0)
    assert not np.isnan(o).any()


def test_closed_forms():
    n, d = 16, 8
    k, v = bf16_array((n, d)), bf16_array((n, d))
    m = (RNG.random((n, n)) < 0.5) & O.mask_dense(n, n)
    m[np.arange(n), np.arange(n)] = True
    # Q = 0: uniform weights, O = mean of V over M(i)
    o, _ = O.masked_attention(np.zeros((n, d)), k, v, m)
    for i in range(n):
        assert np.allclose(o[i], v[m[i]].mean(0), atol=1e-14)
    # constant V column stays constant
    v2 = v.copy()
    v2[:, 3] = 1.25
    q = bf16_array((n, d))
    o2, _ = O.masked_attention(q, k, v2, m)
    assert np.allclose(o2[:, 3], 1.25, atol=1e-14)
    # a single selected key returns its value row
    single = np.zeros((n, n), dtype=bool)
    single[np.arange(n), RNG.integers(0, n, n) % (np.arange(n) + 1)] = True
    o3, lse3 = O.masked_attention(q, k, v, single)
    js = single.argmax(1)
    assert np.array_equal(o3, v[js])
    assert np.allclose(lse3, (q * k[js]).sum(1) / math.sqrt(d), atol=1e-14)
    # permuting keys (and the mask with them) changes nothing
    perm = RNG.permutation(n)
    o4, _ = O.masked_attention(q, k[perm], v[perm], m[:, perm])
    o5, _ = O.masked_attention(q, k, v, m)
    assert np.allclose(o4, o5, atol=1e-13)


def test_attention_rows_matches_mask_form():
    n, d = 64, 16
    q, k, v = bf16_array((n, d)), bf16_array((n, d)), bf16_array((n, d))
    V, S = np.array([0, 3, 17, 40]), np.array([0, 1, 9, 30])
    m = O.mask_vs(n, n, V, S)
    o, lse = O.masked_attention(q, k, v, m)
    rows = [0, 5, 31, 63]
    o_r, l_r = O.attention_rows(q, k, v, rows, [O.row_set_vs(i, V, S) for i in rows])
    assert np.allclose(o_r, o[rows], atol=1e-13) and np.allclose(l_r, lse[rows], atol=1e-13)
    sel = O.select_blocks(O.block_scores(O.block_means(q, 8), O.block_means(k, 8)), "topk", k=2)
    mb = O.mask_block(n, n, sel, 8)
    ob, lb = O.masked_attention(q, k, v, mb)
    o_r, l_r = O.attention_rows(q, k, v, rows, [O.row_set_block(i, sel, 8, n) for i in rows])
    assert np.allclose(o_r, ob[rows], atol=1e-13)


def test_gqa_mapping_equals_repeat_kv():
    # Q head h reads KV head h // (H / Hkv): identical to repeating each KV head.
    H, Hkv, n, d = 4, 2, 16, 8
    q = bf16_array((H, n, d))
    k = bf16_array((Hkv, n, d))
    v = bf16_array((Hkv, n, d))
    krep = np.repeat(k, H // Hkv, axis=0)
    vrep = np.repeat(v, H // Hkv, axis=0)
    m = O.mask_dense(n, n)
    for h in range(H):
        a, _ = O.masked_attention(q[h], k[h // (H // Hkv)], v[h // (H // Hkv)], m)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[h])[None, None], torch.from_numpy(krep[h])[None, None],
            torch.from_numpy(vrep[h])[None, None], is_causal=True)[0, 0].numpy()
        assert np.allclose(a, ref, atol=1e-12)


def test_selected_counts():
    n = 70
    V, S = np.array([0, 3, 17, 40, 69]), np.array([0, 2, 9, 30, 66])
    for qo in (0, 10):
        m = O.mask_vs(n - qo, n, V, S, q_offset=qo)
        assert O.selected_count_vs(n - qo, n, V, S, q_offset=qo) == int(m.sum())
        assert O.selected_count_dense(n - qo, qo) == int(O.mask_dense(n - qo, n, qo).sum())
    q, k = bf16_array((n, 8)), bf16_array((n, 8))
    sel = O.select_blocks(O.block_scores(O.block_means(q, 16), O.block_means(k, 16)), "topk", k=2)
    assert O.selected_count_block(n, n, sel, 16) == int(O.mask_block(n, n, sel, 16).sum())


# ---------------------------------------------------------------------------
# Indexer and router
# ---------------------------------------------------------------------------
def test_indexer_brute_force():
    nq, nk, Hi, di, qo = 3, 10, 4, 8, 7
    q = bf16_array((nq, Hi, di))
    k = bf16_array((nk, di))
    w = RNG.random((nq, Hi))
    sc = O.indexer_scores(q, k, w, qo)
    for i in range(nq):
        for j in range(nk):
            if j > i + qo:
                assert sc[i, j] == -np.inf
                continue
            ref = sum(w[i, h] * max(0.0, sum(q[i, h, c] * k[j, c] for c in range(di))) for h in range(Hi))
            assert abs(sc[i, j] - ref) < 1e-12


def test_indexer_special_cases():
    nq, nk, di, qo = 4, 40, 8, 36
    q = bf16_array((nq, 1, di))
    k = bf16_array((nk, di))
    sc = O.indexer_scores(q, k, np.ones((nq, 1)), qo)
    for i in range(nq):
        p = i + qo
        relu = np.maximum(k[:p + 1] @ q[i, 0], 0)
        assert np.allclose(sc[i, :p + 1], relu, atol=1e-13)
        tk = O.token_topk(sc[i], p, 5)
        assert tk.tolist() == sorted(sorted(range(p + 1), key=lambda j: (-relu[j], j))[:5])
        assert O.token_topk(sc[i], p, nk).tolist() == list(range(p + 1))   # k = N: all causal keys
    # routing every head equals the dense indexer
    qh = bf16_array((nq, 6, di))
    w = RNG.random((nq, 6))
    route = O.router_heads(qh, k, w, qo, route_heads=6, block=8)
    assert np.array_equal(route, np.tile(np.arange(6), (nq, 1)))
    assert np.allclose(O.indexer_scores(qh, k, w, qo, heads=route), O.indexer_scores(qh, k, w, qo))


def test_router_brute_force():
    nq, nk, Hi, di, blk, qo = 3, 40, 6, 8, 8, 20
    q = bf16_array((nq, Hi, di))
    k = bf16_array((nk, di))
    w = RNG.random((nq, Hi))
    route = O.router_heads(q, k, w, qo, route_heads=2, block=blk)
    for i in range(nq):
        p = i + qo
        nc = (p + 1) // blk
        kbar = [O.round_bf16(k[J * blk:(J + 1) * blk].sum(0) / blk) for J in range(nc)]
        r = [w[i, h] * max(0.0, max(float(q[i, h] @ kb) for kb in kbar)) for h in range(Hi)]
        ref = sorted(sorted(range(Hi), key=lambda h: (-r[h], h))[:2])
        assert route[i].tolist() == ref


def test_router_invariances():
    """Properties any implementation of the router reading keeps, each failing
    under a plausible slip: a per-row positive scale of w (ranking by w plus a
    score), a block replaced by copies of its bf16 mean (raw keys instead of
    block means), keys after the last complete block (partial blocks counted),
    and scores all below zero (no ReLU: the heads would not tie at 0)."""
    rng = np.random.default_rng(21)
    nq, nk, Hi, di, blk, qo, rh = 5, 61, 7, 16, 8, 50, 3
    q = bf16_array((nq, Hi, di), rng=rng)
    k = bf16_array((nk, di), rng=rng)
    w = rng.random((nq, Hi))
    base = O.router_heads(q, k, w, qo, route_heads=rh, block=blk)
    c = rng.uniform(0.1, 10.0, size=(nq, 1))
    assert np.array_equal(O.router_heads(q, k, w * c, qo, route_heads=rh, block=blk), base)
    k2 = k.copy()
    for J in range(nk // blk):
        k2[J * blk:(J + 1) * blk] = O.round_bf16(k[J * blk:(J + 1) * blk].sum(0) / blk)
    assert np.array_equal(O.router_heads(q, k2, w, qo, route_heads=rh, block=blk), base)
    # rows i see positions p = i + qo; the complete blocks end at 8 * ((p + 1) // 8)
    k3 = k.copy()
    pmin = qo
    k3[8 * ((pmin + 1) // 8):] = 100.0
    i0 = [i for i in range(nq) if (i + qo + 1) // blk == (pmin + 1) // blk]
    got = O.router_heads(q, k3, w, qo, route_heads=rh, block=blk)
    assert np.array_equal(got[i0], base[i0])
    qn = -np.abs(q)
    kp = np.abs(k)
    assert np.array_equal(O.router_heads(qn, kp, w, qo, route_heads=rh, block=blk),
                          np.tile(np.arange(rh), (nq, 1)))


def test_select_blocks_threshold_forced_is_union():
    """Under the threshold rule the forced blocks join the unforced set and the
    row maximum stays the one over every causal candidate (a maximum taken
    without the forced blocks would move the cutoff); with alpha -> 0 every
    causal block is kept."""
    rng = np.random.default_rng(9)
    S = O.block_scores(bf16_array((9, 8), 4.0, rng), bf16_array((9, 8), 4.0, rng))
    free = O.select_blocks(S, "thresh", log_alpha=-math.log(20))
    forced = O.select_blocks(S, "thresh", log_alpha=-math.log(20), force_first=True, force_diag=True)
    for I in range(9):
        assert forced[I].tolist() == sorted(set(free[I].tolist()) | {0, I})
    # a diagonal block far above the rest: the cutoff follows it, forced or not
    S2 = S.copy()
    for I in range(9):
        S2[I, I] = S[I, :I + 1].max() + 10.0
    f2 = O.select_blocks(S2, "thresh", log_alpha=-math.log(20), force_diag=True)
    for I in range(9):
        assert f2[I].tolist() == [I]
    allk = O.select_blocks(S, "thresh", log_alpha=-1e9, force_first=True)
    for I in range(9):
        assert allk[I].tolist() == list(range(I + 1))


def test_hierarchical_brute_force():
    """Both stages written out with plain loops and sorts on a tiny chunk."""
    nq, nk, Hi, di, blk, qo = 4, 48, 6, 8, 8, 40
    q = bf16_array((nq, Hi, di))
    k = bf16_array((nk, di))
    w = RNG.random((nq, Hi))
    r, cand, kk = 2, 12, 5
    got = O.hierarchical_tokens(q, k, w, qo, r, cand, kk, block=blk)
    for i in range(nq):
        p = i + qo
        nc = (p + 1) // blk
        kbar = [O.round_bf16(k[J * blk:(J + 1) * blk].sum(0) / blk) for J in range(nc)]
        rr = [w[i, h] * max(0.0, max(float(q[i, h] @ kb) for kb in kbar)) for h in range(Hi)]
        heads = sorted(range(Hi), key=lambda h: (-rr[h], h))[:r]
        routed = [sum(w[i, h] * max(0.0, float(q[i, h] @ k[j])) for h in heads) for j in range(p + 1)]
        c_set = sorted(range(p + 1), key=lambda j: (-routed[j], j))[:cand]
        full = {j: sum(w[i, h] * max(0.0, float(q[i, h] @ k[j])) for h in range(Hi)) for j in c_set}
        ref = sorted(sorted(c_set, key=lambda j: (-full[j], j))[:kk])
        assert got[i].tolist() == ref


def test_hierarchical_special_cases():
    nq, nk, Hi, di, blk, qo = 5, 64, 6, 8, 8, 59
    q = bf16_array((nq, Hi, di))
    k = bf16_array((nk, di))
    w = RNG.random((nq, Hi))
    dense = O.indexer_scores(q, k, w, qo)
    for kk in (1, 7, 30):
        dense_sets = [O.token_topk(dense[i], i + qo, kk) for i in range(nq)]
        # every causal key a candidate: the dense indexer
        for a, b in zip(O.hierarchical_tokens(q, k, w, qo, 2, nk, kk, block=blk), dense_sets):
            assert np.array_equal(a, b)
        # every head routed: stage 1 ranks by the dense score, so any cand >= k gives the dense top-k
        for a, b in zip(O.hierarchical_tokens(q, k, w, qo, Hi, kk + 3, kk, block=blk), dense_sets):
            assert np.array_equal(a, b)
        # cand = k: the routed indexer's own top-k
        route = O.router_heads(q, k, w, qo, 2, blk)
        routed = O.indexer_scores(q, k, w, qo, heads=route)
        for i, a in enumerate(O.hierarchical_tokens(q, k, w, qo, 2, kk, kk, block=blk)):
            assert np.array_equal(a, O.token_topk(routed[i], i + qo, kk))
    # the result is a subset of the candidates, of size min(k, cand, p + 1)
    route = O.router_heads(q, k, w, qo, 2, blk)
    routed = O.indexer_scores(q, k, w, qo, heads=route)
    for i, a in enumerate(O.hierarchical_tokens(q, k, w, qo, 2, 20, 9, block=blk)):
        c_set = O.token_topk(routed[i], i + qo, 20)
        assert set(a.tolist()) <= set(c_set.tolist()) and len(a) == 9


# ---------------------------------------------------------------------------
# Hand-written closed-form fixtures
# ---------------------------------------------------------------------------
# ---------------------------------------------------------------------------
# Vertical and slash discovery from pooled block scores (reading O-22)
# ---------------------------------------------------------------------------
def _pooled_brute(S, qb0=0):
    """Row softmax and its column / block-diagonal sums with explicit loops;
    row r is absolute query block qb0 + r."""
    nq, nk = S.shape
    v = [0.0] * nk
    s = [0.0] * nk
    for r in range(nq):
        I = qb0 + r
        m = max(S[r][J] for J in range(I + 1))
        den = sum(math.exp(S[r][J] - m) for J in range(I + 1))
        for J in range(I + 1):
            p = math.exp(S[r][J] - m) / den
            v[J] += p
            s[I - J] += p
    return np.array(v), np.array(s)


@pytest.mark.parametrize("nq", [1, 2, 7, 33])
def test_pooled_vs_scores_brute_force(nq):
    S = RNG.standard_normal((nq, nq)) * 3.0
    S = np.where(np.tril(np.ones((nq, nq), dtype=bool)), S, -np.inf)
    v, s = O.pooled_vs_scores(S)
    vb, sb = _pooled_brute(S)
    assert np.allclose(v, vb, rtol=1e-12, atol=1e-14) and np.allclose(s, sb, rtol=1e-12, atol=1e-14)
    # every row's weights sum to one: both masses total the number of query blocks
    assert abs(v.sum() - nq) < 1e-12 and abs(s.sum() - nq) < 1e-12
    assert np.all(v >= 0) and np.all(s >= 0) and v.max() <= nq and s.max() <= nq


@pytest.mark.parametrize("qb0", [1, 5, 16])
def test_pooled_vs_scores_chunk_adds_up_to_whole_prompt(qb0):
    """Each query block adds its own softmax at its absolute block, so the
    masses of a prefill chunk (query blocks qb0..) plus those of the earlier
    query blocks are the whole prompt's; the chunk alone also matches the loops
    at absolute positions."""
    n = 17
    S = RNG.standard_normal((n, n)) * 3.0
    S = np.where(np.tril(np.ones((n, n), dtype=bool)), S, -np.inf)
    v, s = O.pooled_vs_scores(S)
    v1, s1 = O.pooled_vs_scores(S[:qb0])
    v2, s2 = O.pooled_vs_scores(S[qb0:], q_block0=qb0)
    assert len(s1) == len(s2) == n
    assert np.allclose(v1 + v2, v, rtol=1e-12, atol=1e-14) and np.allclose(s1 + s2, s, rtol=1e-12, atol=1e-14)
    vb, sb = _pooled_brute(S[qb0:], qb0)
    assert np.allclose(v2, vb, rtol=1e-12, atol=1e-14) and np.allclose(s2, sb, rtol=1e-12, atol=1e-14)
    assert abs(v2.sum() - (n - qb0)) < 1e-12 and abs(s2.sum() - (n - qb0)) < 1e-12


def test_pooled_vs_scores_equal_scores_harmonic():
    """Equal scores give P[I, J] = 1 / (I + 1), so vbar[J] = H(n) - H(J) and
    sbar[D] = H(n) - H(D) with H the harmonic numbers (exact fractions)."""
    n = 12
    S = np.where(np.tril(np.ones((n, n), dtype=bool)), 0.0, -np.inf)
    v, s = O.pooled_vs_scores(S)
    H = [sum((Fraction(1, m) for m in range(1, t + 1)), Fraction(0)) for t in range(n + 1)]
    want = np.array([float(H[n] - H[j]) for j in range(n)])
    assert np.allclose(v, want, rtol=1e-13) and np.allclose(s, want, rtol=1e-13)
    # strictly decreasing: the top-k are the first k indices
    Vb, Sb = O.pooled_vs_blocks(v, s, 3, 5)
    assert Vb.tolist() == [0, 1, 2] and Sb.tolist() == [0, 1, 2, 3, 4]


def test_pooled_vs_single_token_blocks_are_vertical_slash_of_every_row():
    """With blocks of one token the pooled vectors are the rows themselves, and
    vbar / sbar are the Vertical-Slash column and diagonal sums taken over every
    query row (last_q = N)."""
    N, d = 40, 8
    q, k = bf16_array((N, d)), bf16_array((N, d))
    S = O.block_scores(O.block_means(q, 1), O.block_means(k, 1))
    v, s = O.pooled_vs_scores(S)
    v2, s2 = O.vs_scores(q, k)
    assert np.allclose(v, v2, rtol=1e-12, atol=1e-15) and np.allclose(s, s2, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("N,block", [(37, 4), (64, 8), (50, 16), (9, 1)])
def test_expand_blocks_brute_force(N, block):
    """Token columns and diagonals of kept blocks against enumeration of every
    pair j <= i < N."""
    nb = -(-N // block)
    rng = np.random.default_rng(N + block)
    Vb = np.sort(rng.choice(nb, min(nb, 3), replace=False))
    Sb = np.sort(rng.choice(nb, min(nb, 3), replace=False))
    cols, diags = O.expand_blocks(Vb, Sb, block, N)
    assert cols.tolist() == [j for j in range(N) if j // block in set(Vb.tolist())]
    want = sorted({i - j for i in range(N) for j in range(i + 1) if (i // block - j // block) in set(Sb.tolist())})
    assert diags.tolist() == want


def test_pooled_vs_sets_find_planted_structure():
    """A key block made to match every query is the top vertical block; query
    and key blocks that share a direction whenever they lie 3 blocks apart make
    block offset 3 the top slash offset, expanded to token offsets 3B - (B - 1)
    .. 3B + (B - 1)."""
    N, d, B = 512, 16, 32
    nb = N // B
    rng = np.random.default_rng(9)
    u = rng.standard_normal(d)
    dirs = rng.standard_normal((4, d)) * 2.0
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    for I in range(nb):
        q[I * B:(I + 1) * B] += u + dirs[I % 4]
        k[I * B:(I + 1) * B] += dirs[(I + 3) % 4]
    k[5 * B:6 * B] += 4.0 * u
    q, k = O.round_bf16(q), O.round_bf16(k)
    cols, diags, v, s, Vb, Sb = O.pooled_vs_sets(q, k, B, 1, 1)
    assert Vb.tolist() == [5] and cols.tolist() == list(range(5 * B, 6 * B))
    assert Sb.tolist() == [3] and diags.tolist() == list(range(3 * B - (B - 1), 3 * B + B))


def test_golden_closed_forms():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        if c["kind"] == "attention":
            q = np.array(c["q"], dtype=np.float64)
            k = np.array(c["k"], dtype=np.float64)
            v = np.array(c["v"], dtype=np.float64)
            m = np.array(c["mask"], dtype=bool)
            o, lse = O.masked_attention(q, k, v, m, scale=c.get("scale"))
            assert np.allclose(o, np.array(c["o"]), atol=1e-15), c["name"]
            exp_lse = np.array([(-np.inf if x is None else x) for x in c["lse"]])
            assert np.allclose(lse, exp_lse, atol=1e-15), c["name"]
        elif c["kind"] == "threshold":
            got = O.threshold_rule(np.array(c["scores"]), np.arange(len(c["scores"])), math.log(c["alpha"]))
            assert got.tolist() == c["keep"], c["name"]
        elif c["kind"] == "topk":
            got = O.topk_rule(np.array(c["scores"]), np.arange(len(c["scores"])), c["k"])
            assert got.tolist() == c["keep"], c["name"]
        elif c["kind"] == "vs":
            v, s = O.vs_scores(np.array(c["q_last"]), np.array(c["k"]), scale=c["scale"])
            assert np.allclose(v, c["v"], atol=1e-15) and np.allclose(s, c["s"], atol=1e-15), c["name"]
        else:
            raise AssertionError(c["kind"])


# ---------------------------------------------------------------------------
# Generators: seeded and shaped as stated
# ---------------------------------------------------------------------------
def test_generators_are_seeded():
    a = synth.block_planted(seed=3, H=2, N=512)
    b = synth.block_planted(seed=3, H=2, N=512)
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    c = synth.mixed_layer(seed=3, N=1024, period=256, nv=16, ns=32, local=128, sink=16, topk=4)
    assert c.q.shape == (1, 32, 1024, 128) and c.k.shape == (1, 8, 1024, 128)
    assert c.q.dtype == torch.bfloat16

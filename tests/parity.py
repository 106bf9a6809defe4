"""Shared helpers of the GPU parity tests: oracle index sets, the cutoff band
rule for comparing selections, and oracle attention on given index sets."""
import itertools
import math

import numpy as np
import torch

import oracle as O
import dynamic_sparse_attention_mean_amd as dsa

# Acceptance bar for attention outputs computed from the oracle's indices.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def f64(t):
    return O.to_f64(t)


# ---------------------------------------------------------------------------
# Selections compared with the cutoff band
# ---------------------------------------------------------------------------
def band_topk(scores, cand, k, rel_only=False):
    """Oracle top-k set and the exemption band around its cutoff.

    Returns (selected set, cutoff or None, tolerance).  Items whose oracle
    score lies within the band may be in or out of the GPU's set."""
    sel = O.topk_rule(scores, cand, k)
    cand = np.asarray(cand, dtype=np.int64)
    if len(sel) >= len(cand) or len(sel) == 0:
        return set(sel.tolist()), None, 0.0
    c = float(np.min(np.asarray(scores)[sel]))
    tol = 1e-3 * c if rel_only else 1e-3 * max(1.0, abs(c))
    return set(sel.tolist()), c, tol


def assert_set_matches(gpu, scores, oracle_sel, cutoff, tol, expect_count=None, what=""):
    gpu = [int(x) for x in gpu]
    assert gpu == sorted(gpu), f"{what}: not ascending"
    assert len(set(gpu)) == len(gpu), f"{what}: duplicates"
    if expect_count is not None:
        assert len(gpu) == expect_count, f"{what}: count {len(gpu)} != {expect_count}"
    g = set(gpu)
    diff = g ^ oracle_sel
    if cutoff is None:
        assert not diff, f"{what}: differs at {sorted(diff)[:10]}"
        return
    scores = np.asarray(scores)
    bad = [j for j in diff if abs(scores[j] - cutoff) > tol]
    assert not bad, f"{what}: {len(bad)} non-exempt differences, e.g. {sorted(bad)[:10]} (cutoff {cutoff})"


def check_block_selection(gpu_idx, gpu_cnt, S, plan_mode, topk, log_alpha, ff, fd, what="", qb0=0):
    """Compare the GPU block lists of one head with the oracle rule on S.

    Row I of S and of the GPU lists is the chunk's query block I, absolute
    block qb0 + I (qb0 = q_offset / block)."""
    nqb = S.shape[0]
    for I in range(nqb):
        Ia = qb0 + I
        g = gpu_idx[I, :gpu_cnt[I]].tolist()
        forced = set()
        if ff:
            forced.add(0)
        if fd:
            forced.add(Ia)
        if plan_mode == "topk":
            cand = [J for J in range(Ia + 1) if J not in forced]
            sel, c, tol = band_topk(S[I], cand, topk)
            expect = len(sel) + len(forced)
            g_rest = [j for j in g if j not in forced]
            assert forced <= set(g), f"{what} I={I}: forced blocks missing"
            assert_set_matches(g_rest, S[I], sel, c, tol, expect_count=len(sel), what=f"{what} I={I}")
            assert len(g) == expect
        else:
            row = S[I, :Ia + 1]
            cut = row.max() + log_alpha
            sel = set(O.threshold_rule(S[I], np.arange(Ia + 1), log_alpha).tolist())
            tol = 1e-3 * max(1.0, abs(cut))
            assert forced <= set(g), f"{what} I={I}: forced blocks missing"
            assert_set_matches(g, S[I], sel | forced, cut, tol, what=f"{what} I={I}")


# ---------------------------------------------------------------------------
# Oracle index sets of a workload (per head)
# ---------------------------------------------------------------------------
def oracle_head_sets(w, b, h):
    """The oracle's index set for head h of batch b: ('vs', V, S, v, s) or
    ('block', sel, S) or ('dense',)."""
    p = w.heads[h]
    B, H, Hkv, Nq, Nk, d = w.shape
    kvh = h // (H // Hkv)
    if p.kind == dsa.VS and getattr(p, "ashape", False):
        V, S = O.ashape_sets(Nk, p.sink, p.local)
        return ("vs", V, S, None, None)
    if p.kind == dsa.VS and getattr(p, "pooled", False):
        cols, diags, vbar, sbar, Vb, Sb = O.pooled_vs_sets(f64(w.q[b, h]), f64(w.k[b, kvh]), p.block, p.nv_blocks,
                                                           p.ns_blocks, q_offset=w.q_offset)
        return ("vs", cols, diags, vbar, sbar)
    if p.kind == dsa.VS:
        q = f64(w.q[b, h, Nq - p.last_q:])
        k = f64(w.k[b, kvh])
        v, s = O.vs_scores(q, k)
        V, S = O.vs_select(v, s, p.nv, p.ns)
        return ("vs", V, S, v, s)
    if p.kind == dsa.BLOCK:
        # a chunk's query blocks start at absolute block q_offset / block
        qb0 = w.q_offset // p.block
        qb = O.block_means(f64(w.q[b, h]), p.block)
        kb = O.block_means(f64(w.k[b, kvh]), p.block)
        S = O.block_scores(qb, kb, q_block0=qb0)
        sel = O.select_blocks(S, p.mode, k=p.topk, log_alpha=p.log_alpha, force_first=p.force_first,
                              force_diag=p.force_diag, q_block0=qb0)
        return ("block", sel, S, qb, kb)
    return ("dense",)


def upload_sets(w, sets, device):
    """Oracle sets -> (head_kind list, VSIndex, BlockIndex) on the device."""
    B, H, Hkv, Nq, Nk, d = w.shape
    kinds = [int(p.kind) for p in w.heads]
    vs_cap_c = max([len(s[1]) for s in sets.values() if s[0] == "vs"] + [1])
    vs_cap_d = max([len(s[2]) for s in sets.values() if s[0] == "vs"] + [1])
    vsi = dsa.VSIndex.empty(B, H, vs_cap_c, vs_cap_d, device) if "vs" in [s[0] for s in sets.values()] else None
    blocks = {w.heads[h].block for (b, h), s in sets.items() if s[0] == "block"}
    bi = None
    if blocks:
        block = blocks.pop()
        nqb = -(-Nq // block)
        cap = max(len(x) for s in sets.values() if s[0] == "block" for x in s[1])
        bi = dsa.BlockIndex.empty(B, H, nqb, cap, block, device)
    cols = vsi.cols.cpu() if vsi else None
    if vsi:
        cc, dg, dc = vsi.cols_count.cpu(), vsi.diags.cpu(), vsi.diags_count.cpu()
    if bi:
        bidx, bcnt = bi.idx.cpu(), bi.count.cpu()
    for (b, h), s in sets.items():
        if s[0] == "vs":
            V, S = s[1], s[2]
            cols[b, h, :len(V)] = torch.from_numpy(np.asarray(V, dtype=np.int32))
            cc[b, h] = len(V)
            dg[b, h, :len(S)] = torch.from_numpy(np.asarray(S, dtype=np.int32))
            dc[b, h] = len(S)
        elif s[0] == "block":
            # the oracle's lists are indexed by absolute query block; the
            # device's by the chunk's query blocks
            qb0 = w.q_offset // w.heads[h].block
            for I, lst in enumerate(s[1][qb0:]):
                bidx[b, h, I, :len(lst)] = torch.from_numpy(np.asarray(lst, dtype=np.int32))
                bcnt[b, h, I] = len(lst)
    if vsi:
        vsi.cols.copy_(cols); vsi.cols_count.copy_(cc); vsi.diags.copy_(dg); vsi.diags_count.copy_(dc)
    if bi:
        bi.idx.copy_(bidx); bi.count.copy_(bcnt)
    return kinds, vsi, bi


def row_set(w, s, b, h, i):
    """M(i) of head h for query row i from an oracle set."""
    B, H, Hkv, Nq, Nk, d = w.shape
    p_i = i + w.q_offset
    if s[0] == "vs":
        return O.row_set_vs(p_i, s[1], s[2])
    if s[0] == "block":
        return O.row_set_block(p_i, s[1], w.heads[h].block, Nk)
    return O.row_set_dense(p_i)


def oracle_attention_rows(w, sets, b, h, rows):
    B, H, Hkv, Nq, Nk, d = w.shape
    kvh = h // (H // Hkv)
    q = f64(w.q[b, h])
    k = w.k[b, kvh]
    v = w.v[b, kvh]
    row_sets = [row_set(w, sets[(b, h)], b, h, i) for i in rows]
    need = np.unique(np.concatenate([r for r in row_sets if len(r)] + [np.zeros(1, dtype=np.int64)]))
    kk = np.zeros((Nk, d))
    vv = np.zeros((Nk, d))
    kk[need] = f64(k[torch.from_numpy(need)])
    vv[need] = f64(v[torch.from_numpy(need)])
    return O.attention_rows(q, kk, vv, rows, row_sets)


def assert_attention_close(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    err = np.abs(o_gpu - o_ref)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite outputs"
    assert err.max() <= MAX_ABS, f"{what}: max abs err {err.max():.3g}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean abs err {err.mean():.3g}"
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse_gpu), fin), f"{what}: LSE finiteness differs"
        assert np.all(np.isneginf(lse_gpu[~fin])), f"{what}: empty rows must have LSE = -inf"
        if fin.any():
            assert np.abs(lse_gpu[fin] - lse_ref[fin]).max() <= MAX_ABS, f"{what}: LSE error"
    return float(err.max()), float(err.mean())


def check_hier_row(qf_i, kf, wf_i, p, route, cand, topk, kbar, g_route, g_cands, g_tok, what="", rb=64):
    """One query of the hierarchical indexer against the oracle's own stages.

    The GPU's routing, candidates and final tokens are compared with the
    oracle's, each within its cutoff band; no GPU result feeds the oracle.
    Returns False when the GPU's routing or candidate choice fell inside a band
    (the later stages then legitimately differ and are not compared).  kbar:
    the oracle's means of the indexer keys over router blocks of rb keys."""
    Hi = qf_i.shape[0]
    nc = (p + 1) // rb
    best = (kbar[:nc] @ qf_i.T).max(axis=0) if nc else np.zeros(Hi)
    r = wf_i * np.maximum(best, 0.0)
    sel, c, tol = band_topk(r, np.arange(Hi), route)
    assert_set_matches(g_route, r, sel, c, tol, expect_count=route, what=f"{what} route")
    if set(int(x) for x in g_route) != sel:
        return False
    heads = np.array(sorted(sel))
    routed = O.indexer_row(qf_i, kf, wf_i, p, heads)
    sel1, c1, tol1 = band_topk(routed, np.arange(p + 1), cand)
    assert_set_matches(g_cands, routed, sel1, c1, tol1, expect_count=min(cand, p + 1), what=f"{what} candidates")
    if set(int(x) for x in g_cands) != sel1:
        return False
    members = np.array(sorted(sel1))
    dense = np.full(p + 1, -np.inf)
    dense[members] = O.indexer_row(qf_i, kf[members], wf_i, len(members) - 1)
    sel2, c2, tol2 = band_topk(dense, members, topk)
    assert_set_matches(g_tok, dense, sel2, c2, tol2, expect_count=min(topk, len(members)), what=f"{what} tokens")
    return True


def check_pooled_sets(g_cols, g_diags, vbar, sbar, block, nvb, nsb, N, what=""):
    """The GPU's Vertical-Slash set of a head with pooled discovery against the
    oracle's masses vbar / sbar: the key blocks behind the columns match the
    oracle's top-nv_blocks within the relative cutoff band and the columns are
    exactly their keys; the diagonals are exactly the expansion of a top-ns_blocks
    offset set that differs from the oracle's only inside the band."""
    g_cols = np.asarray(g_cols, dtype=np.int64)
    g_diags = np.asarray(g_diags, dtype=np.int64)
    gb = np.unique(g_cols // block)
    sel, c, tol = band_topk(vbar, np.arange(len(vbar)), nvb, rel_only=True)
    assert_set_matches(gb, vbar, sel, c, tol, expect_count=min(nvb, len(vbar)), what=f"{what} key blocks")
    assert np.array_equal(g_cols, O.expand_blocks(gb, [], block, N)[0]), f"{what}: columns are not whole blocks"
    sel, c, tol = band_topk(sbar, np.arange(len(sbar)), nsb, rel_only=True)
    if c is None:
        cands = [sorted(sel)]
    else:
        band = [j for j in range(len(sbar)) if abs(sbar[j] - c) <= tol]
        fixed = [j for j in sel if j not in band]
        need = min(nsb, len(sbar)) - len(fixed)
        assert len(band) <= 12, f"{what}: {len(band)} offsets inside the band"
        cands = [sorted(fixed + list(x)) for x in itertools.combinations(band, need)]
    ok = any(np.array_equal(g_diags, O.expand_blocks([], cs, block, N)[1]) for cs in cands)
    assert ok, f"{what}: diagonals are not the expansion of the top block offsets"

"""GPU parity: every step of the HIP path against the fp64 oracle on seeded
inputs, at sizes that span several tiles and a ragged tail."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
import dynamic_sparse_attention_mean_amd as dsa
from dynamic_sparse_attention_mean_amd.pipeline import SparsePrefillLayer

from parity import (assert_attention_close, assert_set_matches, band_topk, check_block_selection, check_pooled_sets,
                    f64, oracle_attention_rows, oracle_head_sets, upload_sets)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def dev(w):
    return w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)


def all_rows_check(w, sets, o, lse, what):
    B, H, Hkv, Nq, Nk, d = w.shape
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy() if lse is not None else None
    for (b, h) in sets:
        rows = list(range(Nq))
        ref_o, ref_l = oracle_attention_rows(w, sets, b, h, rows)
        assert_attention_close(o[b, h], None if lse is None else lse[b, h], ref_o, ref_l, f"{what} head {h}")


# ---------------------------------------------------------------------------
# Block rule: pooling (bit-exact), scores, selection
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,block,mode,force", [(1000, 64, "topk", True), (2048, 64, "topk", False),
                                                (1100, 128, "thresh", False), (777, 64, "thresh", True),
                                                (1000, 32, "topk", True), (700, 16, "thresh", False),
                                                (513, 16, "topk", False), (8192, 64, "topk", True),
                                                (4100, 32, "thresh", True)])
def test_block_index_parity(N, block, mode, force):
    w = synth.block_planted(seed=20 + N, H=3, Hkv=1, N=N, block=block, n_plant=3, mode=mode, topk=4, force=force)
    q, k, _ = dev(w)
    B, H, Hkv, Nq, Nk, d = w.shape
    nqb = -(-N // block)
    cap = nqb if mode == "thresh" else min(nqb, 4 + 2 * force)
    out = dsa.BlockIndex.empty(B, H, nqb, cap, block, DEV)
    qbar = torch.zeros(B, H, nqb, 128, dtype=torch.bfloat16, device=DEV)
    kbar = torch.zeros(B, Hkv, nqb, 128, dtype=torch.bfloat16, device=DEV)
    scores = torch.zeros(B, H, nqb, nqb, dtype=torch.float32, device=DEV)
    dsa.build_index_block(q, k, list(range(H)), block, dsa.TOPK if mode == "topk" else dsa.THRESHOLD, 4, out,
                          force_first=force, force_diag=force, qbar=qbar, kbar=kbar, scores=scores)
    torch.cuda.synchronize()
    for h in range(H):
        s = oracle_head_sets(w, 0, h)
        _, sel, S, qb, kb = s
        assert np.array_equal(f64(qbar[0, h].cpu()), qb), "pooled Q must be bit-exact"
        assert np.array_equal(f64(kbar[0, 0].cpu()), kb), "pooled K must be bit-exact"
        g = scores[0, h].cpu().double().numpy()
        tri = np.tril(np.ones_like(S, dtype=bool))
        assert np.all(np.isneginf(g[~tri]))
        assert np.abs(g[tri] - S[tri]).max() <= 1e-5 * max(1.0, np.abs(S[tri]).max())
        check_block_selection(out.idx[0, h].cpu().numpy(), out.count[0, h].cpu().numpy(), S, mode, 4,
                              -math.log(20.0), force, force, what=f"head {h}")


# ---------------------------------------------------------------------------
# Vertical-Slash: scores and sets
# ---------------------------------------------------------------------------
def assert_vs_scores_close(got, ref, last_q, what):
    """Column / diagonal sums within 1e-5 of each value, relative, with an
    absolute floor of 1e-7 of the mean value (last_q / N): sums far below the
    mean sit far below any cutoff.  The fp32 scoring path carries ~1e-6
    relative error (logits accumulated in fp32, exp2 to about an ulp)."""
    tol = 1e-5 * np.abs(ref) + 1e-7 * last_q / len(ref)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} values off, worst rel "
                           f"{(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300)).max():.3g}")


def check_vs_sets(out, b, h, v, s, nv, ns, what):
    N = len(v)
    for name, sc, kk, g, cnt in (("cols", v, nv, out.cols, out.cols_count), ("diags", s, ns, out.diags, out.diags_count)):
        sel, c, tol = band_topk(sc, np.arange(N), kk, rel_only=True)
        n = int(cnt[b, h].item())
        assert_set_matches(g[b, h, :n].cpu().numpy(), sc, sel, c, tol, expect_count=min(kk, N), what=f"{what} {name}")


@pytest.mark.parametrize("B,H,Hkv,Nk,Nq,heads,last_q", [(2, 4, 2, 1000, 1000, [3, 0, 2], 64),
                                                        (1, 4, 2, 1280, 320, [1, 2, 3], 64),
                                                        (2, 2, 1, 900, 333, [1, 0], 33),
                                                        (1, 2, 1, 700, 1, [0, 1], 1)])
def test_vs_index_batch_and_chunk(B, H, Hkv, Nk, Nq, heads, last_q):
    """build_index_vs with batch 2, heads listed out of order, and chunks that
    end at the last key (q_offset = Nk - Nq > 0): the v / s rows (listed order)
    and the index sets of every (batch, listed head) against the oracle."""
    w = synth.vs_multi(seed=70 + Nk + Nq, B=B, H=H, Hkv=Hkv, Nk=Nk, Nq=Nq, last_q=last_q)
    q, k, _ = dev(w)
    nv, ns = 40, 90
    out = dsa.VSIndex.empty(B, H, nv, ns, DEV)
    vsc = torch.zeros(B, len(heads), Nk, device=DEV)
    ssc = torch.zeros(B, len(heads), Nk, device=DEV)
    dsa.build_index_vs(q, k, heads, last_q, nv, ns, out, v_scores=vsc, s_scores=ssc)
    torch.cuda.synchronize()
    listed = set(heads)
    for b in range(B):
        for t, h in enumerate(heads):
            v, s = O.vs_scores(f64(w.q[b, h, Nq - last_q:]), f64(w.k[b, h // (H // Hkv)]))
            assert_vs_scores_close(vsc[b, t].cpu().double().numpy(), v, last_q, f"b{b} h{h} v")
            assert_vs_scores_close(ssc[b, t].cpu().double().numpy(), s, last_q, f"b{b} h{h} s")
            check_vs_sets(out, b, h, v, s, nv, ns, f"b{b} h{h}")
        for h in range(H):
            if h not in listed:
                assert int(out.cols_count[b, h]) == 0 and int(out.diags_count[b, h]) == 0, "unlisted head written"


def test_vs_index_many_groups():
    """build_index_vs over every head of a GQA layer (batch 2, 32 Q / 8 KV
    heads, heads listed in a scrambled order, a ragged key count): 64 groups
    of heads, so the scoring passes take chunks of another size than the
    smaller cases; v / s rows and sets of every (batch, head) against the oracle."""
    B, H, Hkv, Nk, Nq, last_q = 2, 32, 8, 8192 + 37, 8192 + 37, 64
    w = synth.vs_multi(seed=77, B=B, H=H, Hkv=Hkv, Nk=Nk, Nq=Nq, last_q=last_q)
    q, k, _ = dev(w)
    heads = [int(x) for x in np.random.default_rng(5).permutation(H)]
    nv, ns = 100, 300
    out = dsa.VSIndex.empty(B, H, nv, ns, DEV)
    vsc = torch.zeros(B, H, Nk, device=DEV)
    ssc = torch.zeros(B, H, Nk, device=DEV)
    dsa.build_index_vs(q, k, heads, last_q, nv, ns, out, v_scores=vsc, s_scores=ssc)
    torch.cuda.synchronize()
    for b in range(B):
        for t, h in enumerate(heads):
            v, s = O.vs_scores(f64(w.q[b, h, Nq - last_q:]), f64(w.k[b, h // (H // Hkv)]))
            assert_vs_scores_close(vsc[b, t].cpu().double().numpy(), v, last_q, f"b{b} h{h} v")
            assert_vs_scores_close(ssc[b, t].cpu().double().numpy(), s, last_q, f"b{b} h{h} s")
            check_vs_sets(out, b, h, v, s, nv, ns, f"b{b} h{h}")


@pytest.mark.parametrize("block,mode", [(64, "topk"), (32, "thresh"), (128, "topk")])
def test_block_index_batch2(block, mode):
    """build_index_block with batch 2, GQA 4/2 and heads listed out of order:
    pooled vectors bit-exact, scores and selections of every (batch, listed head)."""
    N, B, H, Hkv = 1500, 2, 4, 2
    w = synth.block_planted(seed=90 + block, B=B, H=H, Hkv=Hkv, N=N, block=block, n_plant=3, mode=mode, topk=4,
                            force=mode == "topk")
    q, k, _ = dev(w)
    heads = [2, 0, 3]
    nqb = -(-N // block)
    cap = nqb if mode == "thresh" else min(nqb, 6)
    out = dsa.BlockIndex.empty(B, H, nqb, cap, block, DEV)
    qbar = torch.zeros(B, H, nqb, 128, dtype=torch.bfloat16, device=DEV)
    kbar = torch.zeros(B, Hkv, nqb, 128, dtype=torch.bfloat16, device=DEV)
    scores = torch.zeros(B, len(heads), nqb, nqb, dtype=torch.float32, device=DEV)
    force = mode == "topk"
    dsa.build_index_block(q, k, heads, block, dsa.TOPK if mode == "topk" else dsa.THRESHOLD, 4, out,
                          force_first=force, force_diag=force, qbar=qbar, kbar=kbar, scores=scores)
    torch.cuda.synchronize()
    for b in range(B):
        for t, h in enumerate(heads):
            _, sel, S, qb, kb = oracle_head_sets(w, b, h)
            assert np.array_equal(f64(qbar[b, h].cpu()), qb), "pooled Q must be bit-exact"
            assert np.array_equal(f64(kbar[b, h // 2].cpu()), kb), "pooled K must be bit-exact"
            g = scores[b, t].cpu().double().numpy()
            tri = np.tril(np.ones_like(S, dtype=bool))
            assert np.all(np.isneginf(g[~tri]))
            assert np.abs(g[tri] - S[tri]).max() <= 1e-5 * max(1.0, np.abs(S[tri]).max())
            check_block_selection(out.idx[b, h].cpu().numpy(), out.count[b, h].cpu().numpy(), S, mode, 4,
                                  -math.log(20.0), force, force, what=f"b{b} head {h}")
        assert int(out.count[b, 1].sum()) == 0, "unlisted head written"
@pytest.mark.parametrize("N,off,block,mode,force", [(1500, 640, 64, "topk", True), (1500, 512, 128, "thresh", False),
                                                    (1000, 608, 32, "thresh", True), (777, 400, 16, "topk", False),
                                                    (2085, 1984, 64, "thresh", True), (1025, 1024, 64, "topk", True),
                                                    (2049, 2048, 128, "thresh", False)])
def test_block_index_chunk(N, off, block, mode, force):
    """build_index_block on a prefill chunk (q_offset > 0, a multiple of the
    block; batch 2, GQA 3/1): the chunk's pooled queries bit-exact, the scores
    of its query block I against key blocks J <= q_offset / block + I, and the
    selections over those candidates, forced diagonal the absolute block."""
    full = synth.block_planted(seed=60 + N, B=2, H=3, Hkv=1, N=N, block=block, n_plant=3, mode=mode, topk=4,
                               force=force)
    w = synth.Workload("block_chunk", full.q[:, :, off:].contiguous(), full.k, full.v, full.heads, q_offset=off)
    q, k, _ = dev(w)
    B, H, Hkv, Nq, Nk, d = w.shape
    nqb, nkb, qb0 = -(-Nq // block), -(-Nk // block), off // block
    cap = qb0 + nqb if mode == "thresh" else min(qb0 + nqb, 4 + 2 * force)
    out = dsa.BlockIndex.empty(B, H, nqb, cap, block, DEV)
    qbar = torch.zeros(B, H, nqb, 128, dtype=torch.bfloat16, device=DEV)
    kbar = torch.zeros(B, Hkv, nkb, 128, dtype=torch.bfloat16, device=DEV)
    scores = torch.zeros(B, H, nqb, nkb, dtype=torch.float32, device=DEV)
    dsa.build_index_block(q, k, list(range(H)), block, dsa.TOPK if mode == "topk" else dsa.THRESHOLD, 4, out,
                          force_first=force, force_diag=force, qbar=qbar, kbar=kbar, scores=scores)
    torch.cuda.synchronize()
    causal = np.arange(nkb)[None, :] <= np.arange(nqb)[:, None] + qb0
    for b in range(B):
        for h in range(H):
            _, sel, S, qb, kb = oracle_head_sets(w, b, h)
            assert S.shape == (nqb, nkb)
            assert np.array_equal(f64(qbar[b, h].cpu()), qb), "pooled Q must be bit-exact"
            assert np.array_equal(f64(kbar[b, 0].cpu()), kb), "pooled K must be bit-exact"
            g = scores[b, h].cpu().double().numpy()
            assert np.all(np.isneginf(g[~causal])) and np.all(np.isneginf(S[~causal]))
            assert np.abs(g[causal] - S[causal]).max() <= 1e-5 * max(1.0, np.abs(S[causal]).max())
            check_block_selection(out.idx[b, h].cpu().numpy(), out.count[b, h].cpu().numpy(), S, mode, 4,
                                  -math.log(20.0), force, force, what=f"chunk b{b} head {h}", qb0=qb0)


@pytest.mark.parametrize("N,last_q,nv,ns", [(1000, 64, 64, 64), (2048, 17, 100, 300), (130, 64, 8, 8)])
def test_vs_index_parity(N, last_q, nv, ns):
    w = synth.vs_single(seed=30 + N, N=N, last_q=last_q, nv=nv, ns=ns, n_plant=4)
    q, k, _ = dev(w)
    out = dsa.VSIndex.empty(1, 1, nv, ns, DEV)
    vsc = torch.zeros(1, 1, N, device=DEV)
    ssc = torch.zeros(1, 1, N, device=DEV)
    dsa.build_index_vs(q, k, [0], last_q, nv, ns, out, v_scores=vsc, s_scores=ssc)
    torch.cuda.synchronize()
    v, s = O.vs_scores(f64(w.q[0, 0, N - last_q:]), f64(w.k[0, 0]))
    gv = vsc[0, 0].cpu().double().numpy()
    gs = ssc[0, 0].cpu().double().numpy()
    assert_vs_scores_close(gv, v, last_q, "v")
    assert_vs_scores_close(gs, s, last_q, "s")
    assert abs(gv.sum() - last_q) < 1e-3 and abs(gs.sum() - last_q) < 1e-3
    for name, sc, kk, g, cnt in (("cols", v, nv, out.cols, out.cols_count), ("diags", s, ns, out.diags, out.diags_count)):
        sel, c, tol = band_topk(sc, np.arange(N), kk, rel_only=True)
        n = int(cnt[0, 0].item())
        assert_set_matches(g[0, 0, :n].cpu().numpy(), sc, sel, c, tol, expect_count=min(kk, N), what=name)


@pytest.mark.parametrize("B,H,Hkv,N,block,nvb,nsb,heads", [(1, 2, 1, 1000, 64, 3, 4, [0, 1]),
                                                        (2, 4, 2, 2048 + 37, 32, 8, 10, [3, 0, 2]),
                                                        (1, 2, 2, 4100, 16, 20, 30, [1]),
                                                        (1, 1, 1, 1500, 128, 2, 5, [0]),
                                                        (1, 2, 1, 700, 64, 11, 11, [1, 0])])
def test_vs_pooled_parity(B, H, Hkv, N, block, nvb, nsb, heads):
    """Vertical-Slash sets from pooled block scores: the vertical and slash
    masses (listed order) against the oracle's, the key blocks and block
    offsets within the band, the token columns and diagonals exactly their
    expansion; ragged N, batch 2, heads out of order, budgets above the
    number of blocks (every block kept)."""
    w = synth.vs_multi(seed=80 + N + block, B=B, H=H, Hkv=Hkv, Nk=N, n_plant=6)
    q, k, _ = dev(w)
    nb = -(-N // block)
    out = dsa.VSIndex.empty(B, H, min(N, nvb * block), min(N, nsb * (2 * block - 1)), DEV)
    vsc = torch.zeros(B, len(heads), nb, device=DEV)
    ssc = torch.zeros(B, len(heads), nb, device=DEV)
    dsa.build_index_vs_pooled(q, k, heads, block, nvb, nsb, out, v_scores=vsc, s_scores=ssc)
    torch.cuda.synchronize()
    for b in range(B):
        for t, h in enumerate(heads):
            cols, diags, vbar, sbar, Vb, Sb = O.pooled_vs_sets(f64(w.q[b, h]), f64(w.k[b, h // (H // Hkv)]), block,
                                                               nvb, nsb)
            for name, got, ref in (("vbar", vsc[b, t], vbar), ("sbar", ssc[b, t], sbar)):
                g = got.cpu().double().numpy()
                tol = 1e-5 * np.abs(ref) + 1e-7 * ref.sum() / len(ref)
                assert np.all(np.abs(g - ref) <= tol), f"b{b} h{h} {name}: {np.abs(g - ref).max():.3g}"
            assert abs(vsc[b, t].sum().item() - nb) < 1e-3 * nb and abs(ssc[b, t].sum().item() - nb) < 1e-3 * nb
            check_pooled_sets(out.cols[b, h, :int(out.cols_count[b, h])].cpu().numpy(),
                              out.diags[b, h, :int(out.diags_count[b, h])].cpu().numpy(), vbar, sbar, block, nvb,
                              nsb, N, what=f"b{b} h{h}")


@pytest.mark.parametrize("B,H,Hkv,N,off,block,nvb,nsb,heads", [(1, 2, 1, 1500, 640, 64, 3, 4, [0, 1]),
                                                            (2, 4, 2, 2085, 1024, 32, 8, 10, [3, 0, 2]),
                                                            (1, 1, 1, 1000, 896, 128, 2, 5, [0]),
                                                            (1, 2, 1, 1025, 1024, 64, 4, 4, [1])])
def test_vs_pooled_chunk(B, H, Hkv, N, off, block, nvb, nsb, heads):
    """Pooled discovery in a prefill chunk (q_offset a multiple of the block):
    query block I of the chunk is absolute block q_offset / block + I, so the
    slash masses have one entry per key block offset; masses, kept blocks and
    offsets, and the token sets against the oracle's."""
    full = synth.vs_multi(seed=90 + N + block, B=B, H=H, Hkv=Hkv, Nk=N, n_plant=6)
    w = synth.Workload("pooled_chunk", full.q[:, :, off:].contiguous(), full.k, full.v, full.heads, q_offset=off)
    q, k, _ = dev(w)
    nqb, nkb = -(-(N - off) // block), -(-N // block)
    out = dsa.VSIndex.empty(B, H, min(N, nvb * block), min(N, nsb * (2 * block - 1)), DEV)
    vsc = torch.zeros(B, len(heads), nkb, device=DEV)
    ssc = torch.zeros(B, len(heads), nkb, device=DEV)
    dsa.build_index_vs_pooled(q, k, heads, block, nvb, nsb, out, v_scores=vsc, s_scores=ssc)
    torch.cuda.synchronize()
    for b in range(B):
        for t, h in enumerate(heads):
            cols, diags, vbar, sbar, Vb, Sb = O.pooled_vs_sets(f64(w.q[b, h]), f64(w.k[b, h // (H // Hkv)]), block,
                                                               nvb, nsb, q_offset=off)
            assert len(vbar) == len(sbar) == nkb
            for name, got, ref in (("vbar", vsc[b, t], vbar), ("sbar", ssc[b, t], sbar)):
                g = got.cpu().double().numpy()
                tol = 1e-5 * np.abs(ref) + 1e-7 * ref.sum() / len(ref)
                assert np.all(np.abs(g - ref) <= tol), f"b{b} h{h} {name}: {np.abs(g - ref).max():.3g}"
            assert abs(vsc[b, t].sum().item() - nqb) < 1e-3 * nqb and abs(ssc[b, t].sum().item() - nqb) < 1e-3 * nqb
            check_pooled_sets(out.cols[b, h, :int(out.cols_count[b, h])].cpu().numpy(),
                              out.diags[b, h, :int(out.diags_count[b, h])].cpu().numpy(), vbar, sbar, block, nvb,
                              nsb, N, what=f"chunk b{b} h{h}")


def test_ashape_sets():
    w = synth.random_qkv(1, 1, 3, 1, 500)
    q, k, v = (t.to(DEV) for t in w)
    out = dsa.VSIndex.empty(1, 3, 128, 1024, DEV)
    dsa.build_index_ashape(q, k, [0, 2], 100, 1000, out)
    torch.cuda.synchronize()
    for h in (0, 2):
        assert out.cols_count[0, h].item() == 100 and out.diags_count[0, h].item() == 500
        assert out.cols[0, h, :100].tolist() == list(range(100))
        assert out.diags[0, h, :500].tolist() == list(range(500))
    assert out.cols_count[0, 1].item() == 0


# ---------------------------------------------------------------------------
# Attention on the oracle's indices
# ---------------------------------------------------------------------------
def mixed_small(N, seed=3):
    return synth.mixed_layer(seed=seed, N=N, H=8, Hkv=2, period=256, n_vert=8, last_q=64, sink=32, local=200,
                             nv=40, ns=160, block=64, topk=6, n_ashape=3, n_vs=3)


@pytest.mark.parametrize("N", [1000, 2048 + 37])
def test_attention_mixed_on_oracle_indices(N):
    w = mixed_small(N)
    q, k, v = dev(w)
    sets = {(0, h): oracle_head_sets(w, 0, h) for h in range(w.shape[1])}
    kinds, vsi, bi = upload_sets(w, sets, DEV)
    o, lse = dsa.sparse_prefill_attn(q, k, v, kinds, vs=vsi, blk=bi, out_dtype=dsa.OUT_F32)
    torch.cuda.synchronize()
    all_rows_check(w, sets, o, lse, f"mixed N={N}")


@pytest.mark.parametrize("block,N,mode", [(64, 1500, "thresh"), (128, 1500, "thresh"), (128, 2048, "thresh"),
                                         (32, 1500, "thresh"), (32, 2048, "topk"), (16, 1000, "thresh"),
                                         (16, 777, "topk")])
def test_attention_block_on_oracle_indices(block, N, mode):
    """Block heads on the oracle's block sets; blocks of 16 and 32 exercise the
    per-pair merged tile lists (query blocks smaller than a wave's rows)."""
    w = synth.block_planted(seed=40 + block, H=2, Hkv=1, N=N, block=block, n_plant=3, mode=mode, topk=5,
                            force=mode == "topk")
    q, k, v = dev(w)
    sets = {(0, h): oracle_head_sets(w, 0, h) for h in range(2)}
    kinds, vsi, bi = upload_sets(w, sets, DEV)
    o, lse = dsa.sparse_prefill_attn(q, k, v, kinds, vs=vsi, blk=bi)
    torch.cuda.synchronize()
    all_rows_check(w, sets, o, lse, f"block {block}")


@pytest.mark.parametrize("Nq,Nk", [(300, 300), (200, 456), (1, 129), (64, 64)])
def test_attention_dense_causal(Nq, Nk):
    q, k, v = synth.random_qkv(7, 1, 4, 2, Nk, Nq=Nq)
    o, lse = dsa.sparse_prefill_attn(q.to(DEV), k.to(DEV), v.to(DEV), [dsa.DENSE] * 4)
    torch.cuda.synchronize()
    for h in range(4):
        m = O.mask_dense(Nq, Nk, Nk - Nq)
        ref_o, ref_l = O.masked_attention(f64(q[0, h]), f64(k[0, h // 2]), f64(v[0, h // 2]), m)
        assert_attention_close(o[0, h].cpu().numpy(), lse[0, h].cpu().numpy(), ref_o, ref_l, f"dense head {h}")
    # the library routine agrees too
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.double(), k.double().repeat_interleave(2, 1), v.double().repeat_interleave(2, 1),
        attn_mask=torch.from_numpy(O.mask_dense(Nq, Nk, Nk - Nq)))
    assert (o.cpu().double() - ref).abs().max() <= 1e-2


def test_attention_empty_rows():
    N = 300
    q, k, v = synth.random_qkv(8, 1, 1, 1, N)
    vsi = dsa.VSIndex.empty(1, 1, 4, 4, DEV)
    vsi.cols[0, 0, 0] = 5
    vsi.cols_count[0, 0] = 1
    o, lse = dsa.sparse_prefill_attn(q.to(DEV), k.to(DEV), v.to(DEV), [dsa.VS], vs=vsi)
    torch.cuda.synchronize()
    o = o.cpu()
    assert torch.all(o[0, 0, :5] == 0) and torch.all(torch.isneginf(lse[0, 0, :5].cpu()))
    assert not torch.isnan(o).any()
    assert torch.allclose(o[0, 0, 5:].double(), v[0, 0, 5].double().expand(N - 5, 128), atol=1e-6)


def test_attention_bf16_output_and_determinism():
    w = mixed_small(1500, seed=5)
    q, k, v = dev(w)
    sets = {(0, h): oracle_head_sets(w, 0, h) for h in range(w.shape[1])}
    kinds, vsi, bi = upload_sets(w, sets, DEV)
    o32, l32 = dsa.sparse_prefill_attn(q, k, v, kinds, vs=vsi, blk=bi, out_dtype=dsa.OUT_F32)
    o32b, l32b = dsa.sparse_prefill_attn(q, k, v, kinds, vs=vsi, blk=bi, out_dtype=dsa.OUT_F32)
    o16, _ = dsa.sparse_prefill_attn(q, k, v, kinds, vs=vsi, blk=bi, out_dtype=dsa.OUT_BF16)
    torch.cuda.synchronize()
    assert torch.equal(o32, o32b) and torch.equal(l32, l32b), "two runs must be bit-identical"
    # the bf16 store is the fp32 result rounded to nearest even
    assert torch.equal(o16, o32.to(torch.bfloat16))


# ---------------------------------------------------------------------------
# The layer pipeline: GPU-built indices match the oracle's, attention on them too
# ---------------------------------------------------------------------------
def test_layer_pipeline_small():
    w = mixed_small(2048 + 64)
    q, k, v = dev(w)
    B, H, Hkv, Nq, Nk, d = w.shape
    layer = SparsePrefillLayer(w.heads, B, H, Hkv, Nk, DEV)
    o, lse = layer(q, k, v)
    torch.cuda.synchronize()
    vsi = layer.vs_index
    for h in range(H):
        s = oracle_head_sets(w, 0, h)
        p = w.heads[h]
        if s[0] == "vs" and p.ashape:
            assert vsi.cols[0, h, :vsi.cols_count[0, h]].tolist() == s[1].tolist()
            assert vsi.diags[0, h, :vsi.diags_count[0, h]].tolist() == s[2].tolist()
        elif s[0] == "vs":
            for name, sc, kk, g, cnt in (("cols", s[3], p.nv, vsi.cols, vsi.cols_count),
                                         ("diags", s[4], p.ns, vsi.diags, vsi.diags_count)):
                sel, c, tol = band_topk(sc, np.arange(Nk), kk, rel_only=True)
                n = int(cnt[0, h].item())
                assert_set_matches(g[0, h, :n].cpu().numpy(), sc, sel, c, tol, expect_count=kk, what=f"h{h} {name}")
        elif s[0] == "block":
            check_block_selection(layer.blk_index.idx[0, h].cpu().numpy(), layer.blk_index.count[0, h].cpu().numpy(),
                                  s[2], p.mode, p.topk, p.log_alpha, p.force_first, p.force_diag, what=f"h{h}")
    # attention on the GPU's own indices equals the oracle's attention on those same indices
    sets = {}
    for h in range(H):
        p = w.heads[h]
        if p.kind == dsa.VS:
            V = vsi.cols[0, h, :vsi.cols_count[0, h]].cpu().numpy()
            S = vsi.diags[0, h, :vsi.diags_count[0, h]].cpu().numpy()
            sets[(0, h)] = ("vs", V, S, None, None)
        else:
            bi = layer.blk_index
            sel = [bi.idx[0, h, I, :bi.count[0, h, I]].cpu().numpy() for I in range(bi.idx.shape[2])]
            sets[(0, h)] = ("block", sel, None)
    all_rows_check(w, sets, o, lse, "pipeline")

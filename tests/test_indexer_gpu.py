"""GPU parity of the indexer token top-k (dense and routed) and of attention
over per-query token lists, against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import dynamic_sparse_attention_mean_amd as dsa

from parity import assert_attention_close, assert_set_matches, band_topk, check_hier_row, f64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def small_chunk(seed, N, Nq, Hi, topk, H=4):
    return synth.indexer_chunk(seed=seed, N=N, Nq=Nq, Hi=Hi, H=H, topk=topk)


def check_token_rows(qi, ki, wt, idx, count, gr, N, Nq, topk, route, what="", rb=64):
    """One sequence's token lists (and routing, when route > 0) against the
    oracle outside the cutoff band; rows routed inside the band are skipped and
    must be rare.  rb: keys per router block."""
    qo = N - Nq
    qf, kf, wf = f64(qi), f64(ki), wt.double().numpy()
    heads = O.router_heads(qf, kf, wf, qo, route_heads=route, block=rb) if route else None
    skipped = 0
    if route:
        # the GPU's routing decision, checked against the oracle router within the band
        kbar = O.block_means(kf, rb)
        for i in range(Nq):
            p = i + qo
            nc = (p + 1) // rb
            best = (kbar[:nc] @ qf[i].T).max(axis=0) if nc else np.zeros(qf.shape[1])
            r = wf[i] * np.maximum(best, 0.0)
            sel, c, tol = band_topk(r, np.arange(qf.shape[1]), route)
            assert_set_matches(gr[i], r, sel, c, tol, expect_count=route, what=f"{what} route q{i}")
    for i in range(Nq):
        p = i + qo
        if route and set(gr[i].tolist()) != set(heads[i].tolist()):
            skipped += 1            # a routing choice inside the band: the token scores differ by design
            continue
        sc = O.indexer_row(qf[i], kf, wf[i], p, None if heads is None else heads[i])
        full = np.full(N, -np.inf)
        full[:p + 1] = sc
        sel, c, tol = band_topk(full, np.arange(p + 1), topk)
        n = int(count[i])
        assert_set_matches(idx[i, :n], full, sel, c, tol, expect_count=min(topk, p + 1), what=f"{what} tokens q{i}")
    assert skipped <= max(2, Nq // 20), f"{what}: {skipped} of {Nq} queries routed inside the band"


@pytest.mark.parametrize("N,Nq,Hi,topk,route", [(1000, 70, 64, 50, 0), (777, 33, 16, 700, 0),
                                                (1500, 90, 64, 64, 8), (640, 64, 12, 100, 3)])
def test_indexer_token_sets(N, Nq, Hi, topk, route):
    w = small_chunk(11 + N, N, Nq, Hi, topk)
    qi, ki, wt = w.extra["q_idx"], w.extra["k_idx"], w.extra["w"]
    out = dsa.TokenIndex.empty(1, Nq, topk, DEV)
    rt = torch.full((Nq, max(route, 1)), -1, dtype=torch.int32, device=DEV)
    dsa.build_index_tokens(qi.to(DEV), ki.to(DEV), wt.to(DEV), topk, out, route_heads=route,
                           route=rt if route else None)
    torch.cuda.synchronize()
    check_token_rows(qi, ki, wt, out.idx[0].cpu().numpy(), out.count[0].cpu().numpy(), rt.cpu().numpy(), N, Nq, topk,
                     route)


@pytest.mark.parametrize("route", [0, 8])
def test_indexer_batch2(route):
    """build_index_tokens over a batch of two chunks ([B, Nq, Hi, d] indexer
    queries, [B, Nk, d] keys, [B, Nq, Hi] weights): every sequence against the
    oracle, and equal to a call on that sequence alone."""
    N, Nq, Hi, topk = 900, 48, 64, 80
    ws = [small_chunk(31 + b, N, Nq, Hi, topk) for b in range(2)]
    qi, ki, wt = (torch.stack([w.extra[x] for w in ws]) for x in ("q_idx", "k_idx", "w"))
    out = dsa.TokenIndex.empty(2, Nq, topk, DEV)
    rt = torch.full((2, Nq, max(route, 1)), -1, dtype=torch.int32, device=DEV)
    dsa.build_index_tokens(qi.to(DEV), ki.to(DEV), wt.to(DEV), topk, out, route_heads=route,
                           route=rt if route else None)
    torch.cuda.synchronize()
    for b in range(2):
        check_token_rows(qi[b], ki[b], wt[b], out.idx[b].cpu().numpy(), out.count[b].cpu().numpy(),
                         rt[b].cpu().numpy(), N, Nq, topk, route, what=f"b{b}")
        one = dsa.TokenIndex.empty(1, Nq, topk, DEV)
        r1 = torch.full((Nq, max(route, 1)), -1, dtype=torch.int32, device=DEV)
        dsa.build_index_tokens(qi[b].to(DEV), ki[b].to(DEV), wt[b].to(DEV), topk, one, route_heads=route,
                               route=r1 if route else None)
        torch.cuda.synchronize()
        assert torch.equal(one.count[0], out.count[b]) and torch.equal(r1, rt[b])
        for i in range(Nq):
            n = int(one.count[0, i])
            assert torch.equal(one.idx[0, i, :n], out.idx[b, i, :n]), f"b{b} q{i}"


@pytest.mark.parametrize("N,Nq,k", [(1000, 70, 50), (300, 300, 40), (513, 17, 600)])
def test_token_attention_on_oracle_sets(N, Nq, k):
    H = 4
    g = np.random.default_rng(N)
    q, kk, v = synth.random_qkv(N + 1, 1, H, H, N, Nq=Nq)
    qo = N - Nq
    tok = [np.sort(g.choice(i + qo + 1, min(k, i + qo + 1), replace=False)) for i in range(Nq)]
    ti = dsa.TokenIndex.empty(1, Nq, k, DEV)
    idx = ti.idx.cpu()
    for i, t in enumerate(tok):
        idx[0, i, :len(t)] = torch.from_numpy(t.astype(np.int32))
    ti.idx.copy_(idx)
    ti.count.copy_(torch.tensor([[len(t) for t in tok]], dtype=torch.int32))
    o, lse = dsa.sparse_prefill_attn(q.to(DEV), kk.to(DEV), v.to(DEV), [dsa.TOKEN] * H, tok=ti)
    torch.cuda.synchronize()
    for h in range(H):
        ref_o, ref_l = O.attention_rows(f64(q[0, h]), f64(kk[0, h]), f64(v[0, h]), list(range(Nq)), tok)
        assert_attention_close(o[0, h].cpu().numpy(), lse[0, h].cpu().numpy(), ref_o, ref_l, f"token head {h}")


def test_indexer_pipeline_end_to_end():
    # GPU-built token sets feed the token attention; where they equal the
    # oracle's sets (every row outside the cutoff band), the outputs match the
    # oracle's attention over the oracle's sets
    N, Nq, Hi, topk, H = 1200, 80, 64, 96, 4
    w = small_chunk(5, N, Nq, Hi, topk, H=H)
    out = dsa.TokenIndex.empty(1, Nq, topk, DEV)
    dsa.build_index_tokens(w.extra["q_idx"].to(DEV), w.extra["k_idx"].to(DEV), w.extra["w"].to(DEV), topk, out)
    o, lse = dsa.sparse_prefill_attn(w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), [dsa.TOKEN] * H, tok=out)
    torch.cuda.synchronize()
    qo = N - Nq
    sc = O.indexer_scores(f64(w.extra["q_idx"]), f64(w.extra["k_idx"]), w.extra["w"].double().numpy(), qo)
    want = [O.token_topk(sc[i], i + qo, topk) for i in range(Nq)]
    got = [out.idx[0, i, :out.count[0, i]].cpu().numpy() for i in range(Nq)]
    rows = [i for i in range(Nq) if np.array_equal(got[i], want[i])]
    assert len(rows) >= Nq - 4, f"only {len(rows)} of {Nq} rows select the oracle's set"
    for h in range(H):
        ref_o, ref_l = O.attention_rows(f64(w.q[0, h]), f64(w.k[0, h]), f64(w.v[0, h]), rows, [want[i] for i in rows])
        assert_attention_close(o[0, h].cpu().numpy()[rows], lse[0, h].cpu().numpy()[rows], ref_o, ref_l,
                               f"pipeline head {h}")


@pytest.mark.parametrize("N,Nq,topk,kind", [(12000, 6, 500, "binary"), (12000, 4, 700, "zero"),
                                            (9000, 5, 2048, "binary")])
def test_token_select_exact_ties(N, Nq, topk, kind):
    """Integer-valued scores (one indexer head, w = 1, inputs in {0, 1}) are exact
    in fp32 on both sides, so the GPU's token sets must equal the oracle's top-k
    exactly, ties to the lower index included.  "zero" makes every score equal:
    the answer is the first `topk` keys, and the GPU selection takes its
    fallback path (one bin holds more candidates than it keeps on chip)."""
    g = torch.Generator().manual_seed(N + topk)
    if kind == "zero":
        qi = torch.zeros(Nq, 1, 128)
    else:
        qi = (torch.rand(Nq, 1, 128, generator=g) < 0.5).float()
    ki = (torch.rand(N, 128, generator=g) < 0.5).float()
    wt = torch.ones(Nq, 1)
    qi, ki = qi.to(torch.bfloat16), ki.to(torch.bfloat16)
    out = dsa.TokenIndex.empty(1, Nq, topk, DEV)
    dsa.build_index_tokens(qi.to(DEV), ki.to(DEV), wt.to(DEV), topk, out)
    torch.cuda.synchronize()
    qo = N - Nq
    qf, kf = f64(qi), f64(ki)
    for i in range(Nq):
        p = i + qo
        sc = O.indexer_row(qf[i], kf, wt[i].double().numpy(), p)
        want = O.token_topk(sc, p, topk)
        n = int(out.count[0, i])
        got = out.idx[0, i, :n].cpu().numpy()
        assert np.array_equal(got, want), f"query {i}: {np.setdiff1d(got, want)[:5]} / {np.setdiff1d(want, got)[:5]}"


@pytest.mark.parametrize("N,Nq,Hi,route,cand,topk", [(1500, 90, 64, 8, 300, 64), (900, 40, 16, 3, 200, 200),
                                                     (700, 64, 64, 8, 2000, 50), (2100, 33, 64, 8, 1024, 700)])
def test_hierarchical_token_sets(N, Nq, Hi, route, cand, topk):
    """Hierarchical indexer: routing, candidate list and final list, each
    against the oracle's own stage (no GPU result feeds the oracle).  Rows whose
    routing or candidate choice falls inside the cutoff band are counted and
    must be rare; every other row must match the oracle outside the band."""
    w = small_chunk(21 + N, N, Nq, Hi, topk)
    qi, ki, wt = w.extra["q_idx"], w.extra["k_idx"], w.extra["w"]
    out = dsa.TokenIndex.empty(1, Nq, topk, DEV)
    cands = dsa.TokenIndex.empty(1, Nq, cand, DEV)
    rt = torch.full((Nq, route), -1, dtype=torch.int32, device=DEV)
    dsa.build_index_tokens_hier(qi.to(DEV), ki.to(DEV), wt.to(DEV), cand, topk, out, route_heads=route, cands=cands,
                                route=rt)
    torch.cuda.synchronize()
    qo = N - Nq
    qf, kf, wf = f64(qi), f64(ki), wt.double().numpy()
    kbar = O.block_means(kf, 64)
    gr = rt.cpu().numpy()
    band_rows = 0
    for i in range(Nq):
        ok = check_hier_row(qf[i], kf, wf[i], i + qo, route, cand, topk, kbar, gr[i],
                            cands.idx[0, i, :cands.count[0, i]].cpu().numpy(),
                            out.idx[0, i, :out.count[0, i]].cpu().numpy(), what=f"q{i}")
        band_rows += not ok
    # the checker accepts the oracle's own stages (a check of the test helper)
    final = O.hierarchical_tokens(qf[:4], kf, wf[:4], qo, route, cand, topk)
    for i in range(4):
        p = i + qo
        h_o = O.router_heads(qf[i:i + 1], kf, wf[i:i + 1], p, route)[0]
        c_o = O.token_topk(O.indexer_row(qf[i], kf, wf[i], p, h_o), p, cand)
        assert check_hier_row(qf[i], kf, wf[i], p, route, cand, topk, kbar, h_o, c_o, final[i], what=f"self q{i}")
    assert band_rows <= max(2, Nq // 20), f"{band_rows} of {Nq} rows chose inside a band"


@pytest.mark.parametrize("rb", [16, 32, 128])
def test_indexer_route_block(rb):
    """Router blocks of 16, 32 and 128 keys (the route_block argument): the
    routing and the token lists against the oracle router of that block size,
    plain and hierarchical."""
    N, Nq, Hi, topk, route, cand = 1100, 60, 64, 90, 8, 300
    w = small_chunk(51 + rb, N, Nq, Hi, topk)
    qi, ki, wt = w.extra["q_idx"], w.extra["k_idx"], w.extra["w"]
    out = dsa.TokenIndex.empty(1, Nq, topk, DEV)
    rt = torch.full((Nq, route), -1, dtype=torch.int32, device=DEV)
    dsa.build_index_tokens(qi.to(DEV), ki.to(DEV), wt.to(DEV), topk, out, route_heads=route, route=rt, route_block=rb)
    torch.cuda.synchronize()
    check_token_rows(qi, ki, wt, out.idx[0].cpu().numpy(), out.count[0].cpu().numpy(), rt.cpu().numpy(), N, Nq, topk,
                     route, what=f"rb{rb}", rb=rb)
    hout = dsa.TokenIndex.empty(1, Nq, topk, DEV)
    cands = dsa.TokenIndex.empty(1, Nq, cand, DEV)
    hrt = torch.full((Nq, route), -1, dtype=torch.int32, device=DEV)
    dsa.build_index_tokens_hier(qi.to(DEV), ki.to(DEV), wt.to(DEV), cand, topk, hout, route_heads=route, cands=cands,
                                route=hrt, route_block=rb)
    torch.cuda.synchronize()
    qf, kf, wf = f64(qi), f64(ki), wt.double().numpy()
    kbar = O.block_means(kf, rb)
    band_rows = 0
    for i in range(Nq):
        ok = check_hier_row(qf[i], kf, wf[i], i + N - Nq, route, cand, topk, kbar, hrt[i].cpu().numpy(),
                            cands.idx[0, i, :cands.count[0, i]].cpu().numpy(),
                            hout.idx[0, i, :hout.count[0, i]].cpu().numpy(), what=f"hier rb{rb} q{i}", rb=rb)
        band_rows += not ok
    assert band_rows <= max(2, Nq // 20), f"{band_rows} of {Nq} rows chose inside a band"


def test_hierarchical_batch2():
    """build_index_tokens_hier over a batch of two chunks, candidate lists
    [B, Nq, cap] and routing [B, Nq, r]: every row of both sequences against the
    oracle's own stages, as for one sequence."""
    N, Nq, Hi, route, cand, topk = 800, 40, 64, 8, 256, 60
    ws = [small_chunk(41 + b, N, Nq, Hi, topk) for b in range(2)]
    qi, ki, wt = (torch.stack([w.extra[x] for w in ws]) for x in ("q_idx", "k_idx", "w"))
    out = dsa.TokenIndex.empty(2, Nq, topk, DEV)
    cands = dsa.TokenIndex.empty(2, Nq, cand, DEV)
    rt = torch.full((2, Nq, route), -1, dtype=torch.int32, device=DEV)
    dsa.build_index_tokens_hier(qi.to(DEV), ki.to(DEV), wt.to(DEV), cand, topk, out, route_heads=route, cands=cands,
                                route=rt)
    torch.cuda.synchronize()
    qo = N - Nq
    band_rows = 0
    for b in range(2):
        qf, kf, wf = f64(qi[b]), f64(ki[b]), wt[b].double().numpy()
        kbar = O.block_means(kf, 64)
        gr = rt[b].cpu().numpy()
        for i in range(Nq):
            ok = check_hier_row(qf[i], kf, wf[i], i + qo, route, cand, topk, kbar, gr[i],
                                cands.idx[b, i, :cands.count[b, i]].cpu().numpy(),
                                out.idx[b, i, :out.count[b, i]].cpu().numpy(), what=f"b{b} q{i}")
            band_rows += not ok
    assert band_rows <= max(2, Nq // 10), f"{band_rows} of {2 * Nq} rows chose inside a band"


@pytest.mark.parametrize("H,Hkv,N,Nq,k,kinds", [
    (16, 1, 1000, 70, 300, "token"),      # MQA: one group of 16 heads
    (16, 2, 700, 50, 90, "token"),        # 8 heads per KV head
    (24, 1, 600, 40, 64, "token"),        # groups of 16 and 8
    (16, 1, 513, 33, 600, "mixed"),       # token heads between dense heads: groups of one head
])
def test_token_attention_shared_kv(H, Hkv, N, Nq, k, kinds):
    """Token attention where 8 or more heads share a KV head (the grouped
    MFMA kernel), on oracle token sets with ragged counts, empty lists and a
    last chunk shorter than 32 tokens, against the fp64 oracle."""
    g = np.random.default_rng(H * N + Hkv)
    q, kk, v = synth.random_qkv(N + H, 1, H, Hkv, N, Nq=Nq)
    qo = N - Nq
    tok = []
    for i in range(Nq):
        m = 0 if i % 13 == 7 else int(g.integers(1, min(k, i + qo + 1) + 1))
        tok.append(np.sort(g.choice(i + qo + 1, m, replace=False)))
    ti = dsa.TokenIndex.empty(1, Nq, k, DEV)
    idx = ti.idx.cpu()
    for i, t in enumerate(tok):
        idx[0, i, :len(t)] = torch.from_numpy(t.astype(np.int32))
    ti.idx.copy_(idx)
    ti.count.copy_(torch.tensor([[len(t) for t in tok]], dtype=torch.int32))
    hk = [dsa.TOKEN if (kinds == "token" or h % 2 == 0) else dsa.DENSE for h in range(H)]
    o, lse = dsa.sparse_prefill_attn(q.to(DEV), kk.to(DEV), v.to(DEV), hk, tok=ti)
    torch.cuda.synchronize()
    rep = H // Hkv
    for h in range(H):
        kh = h // rep
        if hk[h] == dsa.TOKEN:
            ref_o, ref_l = O.attention_rows(f64(q[0, h]), f64(kk[0, kh]), f64(v[0, kh]), list(range(Nq)), tok)
        else:
            m = O.mask_dense(Nq, N, qo)
            ref_o, ref_l = O.masked_attention(f64(q[0, h]), f64(kk[0, kh]), f64(v[0, kh]), m)
        assert_attention_close(o[0, h].cpu().numpy(), lse[0, h].cpu().numpy(), ref_o, ref_l, f"head {h}")


@pytest.mark.parametrize("H,Hkv", [(4, 4), (16, 1)])
def test_token_attention_batch2(H, Hkv):
    """Token lists per (batch, query) with B = 2, for the per-head gather
    kernel (one head per KV head) and the grouped kernel (16 heads sharing one
    K/V): each batch's rows attend over their own lists and their own K/V."""
    B, N, Nq, k = 2, 600, 48, 120
    g = np.random.default_rng(100 + H)
    q, kk, v = synth.random_qkv(200 + H, B, H, Hkv, N, Nq=Nq)
    qo = N - Nq
    tok = [[np.sort(g.choice(i + qo + 1, int(g.integers(1, k + 1)), replace=False)) for i in range(Nq)]
           for _ in range(B)]
    ti = dsa.TokenIndex.empty(B, Nq, k, DEV)
    idx = ti.idx.cpu()
    cnt = torch.zeros(B, Nq, dtype=torch.int32)
    for b in range(B):
        for i, t in enumerate(tok[b]):
            idx[b, i, :len(t)] = torch.from_numpy(t.astype(np.int32))
            cnt[b, i] = len(t)
    ti.idx.copy_(idx)
    ti.count.copy_(cnt)
    o, lse = dsa.sparse_prefill_attn(q.to(DEV), kk.to(DEV), v.to(DEV), [dsa.TOKEN] * H, tok=ti)
    torch.cuda.synchronize()
    rep = H // Hkv
    for b in range(B):
        for h in range(H):
            ref_o, ref_l = O.attention_rows(f64(q[b, h]), f64(kk[b, h // rep]), f64(v[b, h // rep]), list(range(Nq)),
                                            tok[b])
            assert_attention_close(o[b, h].cpu().numpy(), lse[b, h].cpu().numpy(), ref_o, ref_l, f"b={b} head {h}")


def test_hierarchical_candidate_capacity_above_cand():
    """A caller candidate list wider than `cand` (cap = cand + 64): the results
    equal those of cap == cand, and nothing is written past the workspace the
    library asked for (a guard region after it keeps its fill pattern)."""
    N, Nq, Hi, route, cand, topk = 1500, 90, 64, 8, 300, 64
    w = small_chunk(21 + N, N, Nq, Hi, topk)
    qi, ki, wt = (w.extra[x].to(DEV) for x in ("q_idx", "k_idx", "w"))
    shape = dsa.Shape(1, 1, 1, Nq, N, 128, N - Nq)
    need = dsa.workspace_size(dsa.OP_TOKENS_HIER, shape, [Hi, route, cand, topk])
    guard = 1 << 20
    results = []
    for cap in (cand, cand + 64):
        buf = torch.full((need + guard,), 0xA5, dtype=torch.uint8, device=DEV)
        out = dsa.TokenIndex.empty(1, Nq, topk, DEV)
        cands = dsa.TokenIndex.empty(1, Nq, cap, DEV)
        dsa.build_index_tokens_hier(qi, ki, wt, cand, topk, out, route_heads=route, cands=cands, ws=buf[:need])
        torch.cuda.synchronize()
        assert torch.all(buf[need:] == 0xA5), f"cap {cap}: workspace overrun"
        results.append((out.idx.cpu(), out.count.cpu(), cands.idx[..., :cand].cpu(), cands.count.cpu()))
    for a, b in zip(*results):
        assert torch.equal(a, b)


def test_token_attention_ignores_noncausal_entries():
    """Token lists that also hold keys after the query's position (and a
    negative entry): those entries are not part of M(i), so the output equals
    the oracle over the causal entries only (per-head and grouped kernels)."""
    N, Nq, k = 700, 60, 80
    for H, Hkv in ((4, 4), (16, 1)):
        g = np.random.default_rng(300 + H)
        q, kk, v = synth.random_qkv(310 + H, 1, H, Hkv, N, Nq=Nq)
        qo = N - Nq
        causal, lists = [], []
        for i in range(Nq):
            p = i + qo
            c = np.sort(g.choice(p + 1, int(g.integers(1, k // 2)), replace=False))
            extra = np.array([p + 1 + x for x in range(min(5, N - 1 - p))] + [-3], dtype=np.int64)
            causal.append(c)
            lists.append(np.sort(np.concatenate([c, extra])))
        ti = dsa.TokenIndex.empty(1, Nq, k, DEV)
        idx = torch.zeros(1, Nq, k, dtype=torch.int32)
        cnt = torch.zeros(1, Nq, dtype=torch.int32)
        for i, L in enumerate(lists):
            idx[0, i, :len(L)] = torch.from_numpy(L.astype(np.int32))
            cnt[0, i] = len(L)
        ti.idx.copy_(idx)
        ti.count.copy_(cnt)
        o, lse = dsa.sparse_prefill_attn(q.to(DEV), kk.to(DEV), v.to(DEV), [dsa.TOKEN] * H, tok=ti)
        torch.cuda.synchronize()
        rep = H // Hkv
        for h in range(H):
            ref_o, ref_l = O.attention_rows(f64(q[0, h]), f64(kk[0, h // rep]), f64(v[0, h // rep]), list(range(Nq)),
                                            causal)
            assert_attention_close(o[0, h].cpu().numpy(), lse[0, h].cpu().numpy(), ref_o, ref_l,
                                   f"H={H} head {h}")

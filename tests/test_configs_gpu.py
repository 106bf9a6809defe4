"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (SparsePrefillLayer, bf16 output, LSE on): the GPU's index
sets against the oracle's (cutoff band), and attention on sampled rows against
the oracle over the same index sets.

Output precision.  The acceptance bar (max-abs 1e-2, mean-abs 1e-3) is checked
on the fp32-output path: the same attention launch with fp32 stores.  The
bf16-output path the benchmark times must equal that fp32 result rounded to
nearest even, bit for bit, over the whole output; each of its sampled values
must lie within max(1e-2, half a bf16 ulp of the exact value) of the oracle,
and its mean error within 1e-3 plus the mean error that storing the exact
values in bf16 makes by itself."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
import dynamic_sparse_attention_mean_amd as dsa
from dynamic_sparse_attention_mean_amd.pipeline import SparsePrefillLayer

from parity import (MAX_ABS, MEAN_ABS, assert_set_matches, band_topk, check_block_selection, check_hier_row,
                    check_pooled_sets, f64, oracle_head_sets, row_set)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def sample_rows(n, k=40, seed=0):
    """Edge rows (first, tile boundaries, middle, last) plus k random rows spread over [0, n)."""
    g = np.random.default_rng(seed)
    base = {0, 1, 63, 64, 127, 128, n // 2, n - 65, n - 64, n - 2, n - 1}
    base |= set(g.choice(n, min(k, n), replace=False).tolist())
    return sorted(x for x in base if 0 <= x < n)


def half_ulp_bf16(ref):
    """Half a bf16 ulp of |ref| (bf16 keeps 8 significant bits)."""
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def round_bf16_np(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def check_outputs(got32, got16, ref_o, ref_l, lse, what):
    """fp32 path at the acceptance bar.  The bf16 path (the fp32 output rounded
    to nearest even, checked bit for bit by run_layer) per element within
    max(1e-2, half an ulp of the stored value plus the fp32 error), which is
    what storing an fp32 result within the bar can cost, and on average within
    1e-3 plus the storage rounding of the exact values."""
    err = np.abs(got32 - ref_o)
    assert np.isfinite(got32).all(), f"{what}: non-finite outputs"
    assert err.max() <= MAX_ABS, f"{what}: fp32 max abs err {err.max():.3g}"
    assert err.mean() <= MEAN_ABS, f"{what}: fp32 mean abs err {err.mean():.3g}"
    e16 = np.abs(got16 - ref_o)
    bound16 = np.maximum(MAX_ABS, half_ulp_bf16(got32) + err)
    assert np.all(e16 <= bound16 * (1 + 1e-12)), f"{what}: bf16 max abs err {e16.max():.3g}"
    storage = np.abs(round_bf16_np(ref_o) - ref_o).mean()
    assert e16.mean() <= MEAN_ABS + storage, f"{what}: bf16 mean abs err {e16.mean():.3g} (storage {storage:.3g})"
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: LSE finiteness differs"
    if fin.any():
        assert np.abs(lse[fin] - ref_l[fin]).max() <= MAX_ABS, f"{what}: LSE error"
    return float(err.max()), float(err.mean())


def gpu_sets(layer, h):
    """The GPU's index lists of head h, read back once (compared with the oracle's, never fed to it)."""
    if layer.kinds[h] == dsa.VS:
        vsi = layer.vs_index
        return ("vs", vsi.cols[0, h, :int(vsi.cols_count[0, h])].cpu().numpy(),
                vsi.diags[0, h, :int(vsi.diags_count[0, h])].cpu().numpy())
    if layer.kinds[h] == dsa.BLOCK:
        idx, cnt = layer.blk_index.idx[0, h].cpu().numpy(), layer.blk_index.count[0, h].cpu().numpy()
        return ("block", [idx[I, :cnt[I]] for I in range(idx.shape[0])])
    return ("dense",)


def gpu_row(w, g, h, i):
    """Keys of query row i under the GPU's lists (plain numpy, for the comparison)."""
    p = i + w.q_offset
    j = np.arange(p + 1)
    if g[0] == "vs":
        keep = np.isin(j, g[1]) | np.isin(p - j, g[2])
    elif g[0] == "block":
        blk = w.heads[h].block
        keep = np.isin(j // blk, g[1][p // blk])
    else:
        keep = np.ones(p + 1, dtype=bool)
    return j[keep]


def check_rows(w, layer, o, lse, heads, osets, rows_per_head=40, o32=None):
    """Sampled rows of each head against the oracle's attention over the
    oracle's own index sets.  A row whose GPU row set differs from the
    oracle's (a selection inside the cutoff band) is not compared; such rows
    must be rare.  o is the bf16 output the benchmark times, o32 the same
    launch with fp32 stores."""
    B, H, Hkv, Nq, Nk, d = w.shape
    o = o.float().cpu().numpy()
    o32 = o32.cpu().numpy()
    lse = lse.cpu().numpy()
    worst = 0.0
    for h in heads:
        kvh = h // (H // Hkv)
        rows_all = sample_rows(Nq, rows_per_head, seed=h)
        rs_all = [row_set(w, osets[h], 0, h, i) for i in rows_all]
        g = gpu_sets(layer, h)
        keep = [n for n, i in enumerate(rows_all) if np.array_equal(gpu_row(w, g, h, i), np.unique(rs_all[n]))]
        assert len(keep) >= len(rows_all) - max(2, len(rows_all) // 20), \
            f"head {h}: only {len(keep)} of {len(rows_all)} rows select the oracle's set"
        rows = [rows_all[n] for n in keep]
        rs = [rs_all[n] for n in keep]
        need = np.unique(np.concatenate([r for r in rs if len(r)] + [np.zeros(1, dtype=np.int64)]))
        kk = np.zeros((Nk, d))
        vv = np.zeros((Nk, d))
        kk[need] = f64(w.k[0, kvh][torch.from_numpy(need)])
        vv[need] = f64(w.v[0, kvh][torch.from_numpy(need)])
        q = f64(w.q[0, h][torch.from_numpy(np.array(rows))])
        ref_o, ref_l = O.attention_rows(q, kk, vv, list(range(len(rows))), rs)
        mx, _ = check_outputs(o32[0, h, rows].astype(np.float64), o[0, h, rows].astype(np.float64), ref_o, ref_l,
                              lse[0, h, rows], f"head {h}")
        worst = max(worst, mx)
    return worst


def check_sets(w, layer, heads, osets):
    """The GPU's index sets against the oracle's, within the cutoff band."""
    B, H, Hkv, Nq, Nk, d = w.shape
    for h in heads:
        p = w.heads[h]
        if p.kind == dsa.VS and p.ashape:
            assert int(layer.vs_index.cols_count[0, h]) == min(p.sink, Nk)
            assert int(layer.vs_index.diags_count[0, h]) == min(p.local, Nk)
            assert layer.vs_index.cols[0, h, :min(p.sink, Nk)].tolist() == list(range(min(p.sink, Nk)))
            assert layer.vs_index.diags[0, h, :min(p.local, Nk)].tolist() == list(range(min(p.local, Nk)))
        elif p.kind == dsa.VS and p.pooled:
            _, _, _, vbar, sbar = osets[h]
            vsi = layer.vs_index
            check_pooled_sets(vsi.cols[0, h, :int(vsi.cols_count[0, h])].cpu().numpy(),
                              vsi.diags[0, h, :int(vsi.diags_count[0, h])].cpu().numpy(), vbar, sbar, p.block,
                              p.nv_blocks, p.ns_blocks, Nk, what=f"head {h}")
        elif p.kind == dsa.VS:
            _, _, _, v, s = osets[h]
            for name, sc, k, g, cnt in (("cols", v, p.nv, layer.vs_index.cols, layer.vs_index.cols_count),
                                        ("diags", s, p.ns, layer.vs_index.diags, layer.vs_index.diags_count)):
                sel, c, tol = band_topk(sc, np.arange(Nk), k, rel_only=True)
                n = int(cnt[0, h])
                assert_set_matches(g[0, h, :n].cpu().numpy(), sc, sel, c, tol, expect_count=min(k, Nk),
                                   what=f"head {h} {name}")
        elif p.kind == dsa.BLOCK:
            S = osets[h][2]
            check_block_selection(layer.blk_index.idx[0, h].cpu().numpy(), layer.blk_index.count[0, h].cpu().numpy(),
                                  S, p.mode, p.topk, p.log_alpha, p.force_first, p.force_diag, what=f"head {h}")


def osets_of(w, heads):
    return {h: oracle_head_sets(w, 0, h) for h in heads}


def run_layer(w):
    """The layer as the benchmark runs it (bf16 output), then the same attention
    launch on the same index sets with fp32 stores.  The bf16 output must be the
    fp32 one rounded to nearest even, everywhere."""
    B, H, Hkv, Nq, Nk, d = w.shape
    layer = SparsePrefillLayer(w.heads, B, H, Hkv, Nk, DEV, out_dtype=dsa.OUT_BF16, want_lse=True)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    o, lse = layer(q, k, v)
    o32, lse32 = dsa.sparse_prefill_attn(q, k, v, layer.kinds, vs=layer.vs_index, blk=layer.blk_index,
                                         out_dtype=dsa.OUT_F32, ws=layer.ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o32.to(torch.bfloat16)), "bf16 output is not the fp32 output rounded"
    assert torch.equal(lse, lse32)
    del q, k, v, lse32
    return layer, o, lse, o32


def test_config1_vertical_slash_4k():
    w = synth.config(1)
    layer, o, lse, o32 = run_layer(w)
    os_ = osets_of(w, [0])
    check_sets(w, layer, [0], os_)
    # the planted vertical keys are found
    assert set(w.extra["planted_cols"].tolist()) <= set(layer.vs_index.cols[0, 0].cpu().tolist())
    check_rows(w, layer, o, lse, [0], os_, rows_per_head=200, o32=o32)


@pytest.mark.parametrize("mode", ["topk", "thresh"])
def test_config2_block_32k(mode):
    w = synth.config(2, mode=mode)
    layer, o, lse, o32 = run_layer(w)
    os_ = osets_of(w, range(8))
    check_sets(w, layer, range(8), os_)
    check_rows(w, layer, o, lse, range(8), os_, o32=o32)


def test_config3_mixed_128k():
    w = synth.config(3)
    layer, o, lse, o32 = run_layer(w)
    os_ = osets_of(w, range(32))
    check_sets(w, layer, range(32), os_)
    check_rows(w, layer, o, lse, range(32), os_, rows_per_head=24, o32=o32)


def test_config3_pooled_discovery_128k():
    """The 128K mixed layer with its Vertical-Slash heads (11-26) discovered
    from pooled block scores (block 64, 16 key blocks, 32 block offsets): every
    head's sets against the oracle's, sampled rows of every head."""
    w = synth.config(3, vs_rule="pooled")
    layer, o, lse, o32 = run_layer(w)
    os_ = osets_of(w, range(32))
    check_sets(w, layer, range(32), os_)
    check_rows(w, layer, o, lse, range(32), os_, rows_per_head=12, o32=o32)


def test_config4_threshold_4k_every_row():
    w = synth.config(4, N=4096)
    layer, o, lse, o32 = run_layer(w)
    os_ = osets_of(w, range(32))
    check_sets(w, layer, range(32), os_)
    check_rows(w, layer, o, lse, range(32), os_, rows_per_head=4096, o32=o32)


def test_config4_threshold_256k_sampled():
    """N = 262144: the block sets of all 32 heads (every query block), and
    sampled rows of every head."""
    w = synth.config(4, N=262144)
    layer, o, lse, o32 = run_layer(w)
    os_ = osets_of(w, range(32))
    check_sets(w, layer, range(32), os_)
    check_rows(w, layer, o, lse, range(32), os_, rows_per_head=6, o32=o32)


def chunk_rows(Nq, k, seed):
    """k random query rows spread over the chunk plus its first, middle and last rows."""
    g = np.random.default_rng(seed)
    base = {0, 1, Nq // 2, Nq - 65, Nq - 33, Nq - 2, Nq - 1}
    base |= set(g.choice(Nq, min(k, Nq), replace=False).tolist())
    return sorted(x for x in base if 0 <= x < Nq)


@pytest.mark.parametrize("route,kv_heads", [(0, None), (8, None), (0, 1)])
def test_config5_indexer_128k(route, kv_heads):
    """The 8192-query chunk over 131072 keys: routing and token sets of 64+
    sampled queries spread over the whole chunk (its last rows included)
    against the oracle within the band, then attention of all 16 heads on
    those rows over the oracle's token sets, fp32 path at the acceptance bar
    (max-abs, mean-abs, LSE) and bf16 path as its rounding."""
    w = synth.config(5, route_heads=route, kv_heads=kv_heads)
    B, H, Hkv, Nq, Nk, d = w.shape
    qi, ki, wt = w.extra["q_idx"], w.extra["k_idx"], w.extra["w"]
    topk = w.extra["topk"]
    out = dsa.TokenIndex.empty(1, Nq, topk, DEV)
    rt = torch.full((Nq, max(route, 1)), -1, dtype=torch.int32, device=DEV)
    dsa.build_index_tokens(qi.to(DEV), ki.to(DEV), wt.to(DEV), topk, out, route_heads=route,
                           route=rt if route else None)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    o, lse = dsa.sparse_prefill_attn(q, k, v, [dsa.TOKEN] * H, tok=out, out_dtype=dsa.OUT_BF16)
    o32, lse32 = dsa.sparse_prefill_attn(q, k, v, [dsa.TOKEN] * H, tok=out, out_dtype=dsa.OUT_F32)
    torch.cuda.synchronize()
    assert torch.equal(o, o32.to(torch.bfloat16)) and torch.equal(lse, lse32)
    del q, k, v
    qo = w.q_offset
    kf = f64(ki)
    rows = chunk_rows(Nq, 64, seed=route + 7 * (kv_heads or 0))
    kbar = O.block_means(kf, 64) if route else None
    sets = {}      # the oracle's token set of each sampled row whose GPU set is the same
    for i in rows:
        qf = f64(qi[i])
        wf = wt[i].double().numpy()
        p = i + qo
        heads = None
        if route:
            nc = (p + 1) // 64
            r = wf * np.maximum((kbar[:nc] @ qf.T).max(axis=0), 0.0)
            sel, c, tol = band_topk(r, np.arange(qi.shape[1]), route)
            g = rt[i].cpu().numpy()
            assert_set_matches(g, r, sel, c, tol, expect_count=route, what=f"route q{i}")
            if set(g.tolist()) != sel:
                continue            # a routing choice inside the band: the token scores differ by design
            heads = np.array(sorted(sel))
        sc = O.indexer_row(qf, kf, wf, p, heads)
        sel, c, tol = band_topk(sc, np.arange(p + 1), topk)
        n = int(out.count[0, i])
        got = out.idx[0, i, :n].cpu().numpy()
        assert_set_matches(got, sc, sel, c, tol, expect_count=topk, what=f"tokens q{i}")
        if set(got.tolist()) == sel:
            sets[i] = np.array(sorted(sel))
    assert len(sets) >= len(rows) - max(2, len(rows) // 20), \
        f"only {len(sets)} of {len(rows)} sampled rows without band choices"
    rows = sorted(sets)
    assert rows[-1] >= Nq - 64, "the chunk's last rows must be among the compared ones"
    # attention of every head on the sampled rows, over the oracle's token sets (equal to the GPU's)
    o = o.float().cpu().numpy()
    o32 = o32.cpu().numpy()
    lse = lse.cpu().numpy()
    need = np.unique(np.concatenate(list(sets.values())))
    for h in range(H):
        kk = np.zeros((Nk, d))
        vv = np.zeros((Nk, d))
        kh = h // (H // Hkv)
        kk[need] = f64(w.k[0, kh][torch.from_numpy(need)])
        vv[need] = f64(w.v[0, kh][torch.from_numpy(need)])
        ref_o, ref_l = O.attention_rows(f64(w.q[0, h][torch.from_numpy(np.array(rows))]), kk, vv,
                                        list(range(len(rows))), [sets[i] for i in rows])
        check_outputs(o32[0, h, rows].astype(np.float64), o[0, h, rows].astype(np.float64), ref_o, ref_l,
                      lse[0, h, rows], f"head {h}")


def test_config5_hierarchical_128k():
    """The hierarchical indexer at the config-5 size (8192 queries over 131072
    keys, 8 of 64 heads routed, 8192 candidates, top-2048): routing,
    candidates and tokens of 64+ sampled queries spread over the whole chunk
    against the oracle's stages."""
    w = synth.config(5, route_heads=8, cand=8192)
    Nq = w.shape[3]
    qi, ki, wt = w.extra["q_idx"], w.extra["k_idx"], w.extra["w"]
    topk, route, cand = w.extra["topk"], w.extra["route_heads"], w.extra["cand"]
    out = dsa.TokenIndex.empty(1, Nq, topk, DEV)
    cands = dsa.TokenIndex.empty(1, Nq, cand, DEV)
    rt = torch.full((Nq, route), -1, dtype=torch.int32, device=DEV)
    dsa.build_index_tokens_hier(qi.to(DEV), ki.to(DEV), wt.to(DEV), cand, topk, out, route_heads=route, cands=cands,
                                route=rt)
    torch.cuda.synchronize()
    kf = f64(ki)
    kbar = O.block_means(kf, 64)
    rows = chunk_rows(Nq, 64, seed=3)
    checked = 0
    for i in rows:
        checked += check_hier_row(f64(qi[i]), kf, wt[i].double().numpy(), i + w.q_offset, route, cand, topk, kbar,
                                  rt[i].cpu().numpy(), cands.idx[0, i, :cands.count[0, i]].cpu().numpy(),
                                  out.idx[0, i, :out.count[0, i]].cpu().numpy(), what=f"q{i}")
    assert checked >= len(rows) - max(2, len(rows) // 20), f"only {checked} of {len(rows)} rows without band choices"


@pytest.mark.parametrize("block", [16, 32])
def test_block_sweep_32k_small_blocks(block):
    """The block-size sweep's data at a small block size (N=32768, 8 heads,
    top-(1024/B) + first + diagonal): selections against the oracle within the
    band, sampled rows against the oracle's attention over its own sets."""
    w = synth.token_planted(block=block)
    layer, o, lse, o32 = run_layer(w)
    heads = [0, 3, 7]
    os_ = osets_of(w, heads)
    check_sets(w, layer, heads, os_)
    check_rows(w, layer, o, lse, heads, os_, rows_per_head=24, o32=o32)


def test_block16_past_paired_limit():
    """Blocks of 16 on a sequence whose items see more than 8192 16-key blocks
    (N=135168): the items near the end take the 32-key unit gather, the
    earlier ones the paired gather; selections against the oracle within the
    band, sampled rows (the last ones included) against the oracle's
    attention over its own sets."""
    w = synth.token_planted(block=16, N=135168, H=2)
    layer, o, lse, o32 = run_layer(w)
    heads = [0, 1]
    os_ = osets_of(w, heads)
    check_sets(w, layer, heads, os_)
    check_rows(w, layer, o, lse, heads, os_, rows_per_head=24, o32=o32)

"""GPU parity of sparse attention on shapes the five workloads do not reach:
batch > 1, GQA ratios 1 and 8, Vertical-Slash heads in a chunk that starts
after key 0 (q_offset > 0, also not tile-aligned), and one call that mixes
token-list heads with Vertical-Slash, block and dense heads.  Every head is fed the oracle's own
index set and compared with the fp64 oracle on every row."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import dynamic_sparse_attention_mean_amd as dsa

from parity import assert_attention_close, f64, oracle_attention_rows, oracle_head_sets, upload_sets

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def ashape(sink, local):
    return synth.HeadPlan(dsa.VS, sink=sink, local=local, ashape=True)


def vs(last_q, nv, ns):
    return synth.HeadPlan(dsa.VS, last_q=last_q, nv=nv, ns=ns)


def blk(mode, topk=0, force=False, block=64):
    return synth.HeadPlan(dsa.BLOCK, block=block, mode=mode, topk=topk, log_alpha=-float(np.log(20.0)),
                          force_first=force, force_diag=force)


def dense():
    return synth.HeadPlan(dsa.DENSE)


def workload(seed, B, H, Hkv, Nk, heads, Nq=None):
    Nq = Nk if Nq is None else Nq
    q, k, v = synth.random_qkv(seed, B, H, Hkv, Nk, Nq=Nq)
    return synth.Workload(f"shape{seed}", q, k, v, heads, q_offset=Nk - Nq)


def run_and_check(w, what):
    B, H, Hkv, Nq, Nk, d = w.shape
    sets = {(b, h): oracle_head_sets(w, b, h) for b in range(B) for h in range(H)}
    kinds, vsi, bi = upload_sets(w, sets, DEV)
    o, lse = dsa.sparse_prefill_attn(w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), kinds, vs=vsi, blk=bi,
                                     out_dtype=dsa.OUT_F32)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    rows = list(range(Nq))
    for (b, h) in sets:
        ref_o, ref_l = oracle_attention_rows(w, sets, b, h, rows)
        assert_attention_close(o[b, h], lse[b, h], ref_o, ref_l, f"{what} b={b} h={h}")


def test_batch2_mixed_gqa_ragged():
    heads = [ashape(16, 100), vs(64, 40, 60), blk("topk", 4, True), dense(),
             vs(17, 25, 80), blk("thresh"), ashape(0, 64), vs(64, 0, 30)]
    run_and_check(workload(31, 2, 8, 2, 700, heads), "B=2")


@pytest.mark.parametrize("H,Hkv", [(4, 4), (8, 1)])
def test_gqa_ratios(H, Hkv):
    kinds = [vs(64, 30, 50), dense(), blk("topk", 3), ashape(8, 90)]
    heads = [kinds[h % 4] for h in range(H)]
    run_and_check(workload(40 + H, 1, H, Hkv, 513, heads), f"H={H} Hkv={Hkv}")


def test_vertical_slash_chunk_after_key0():
    """A 320-row chunk at the end of 1280 keys (q_offset = 960): the last
    last_q rows of the chunk score all keys, the sets are offsets from the
    rows' absolute positions."""
    heads = [vs(64, 50, 90), ashape(32, 200), dense(), vs(33, 10, 300)]
    run_and_check(workload(50, 1, 4, 2, 1280, heads, Nq=320), "chunk")


def test_chunk_offset_not_tile_aligned():
    """A 333-row chunk at the end of 1000 keys (q_offset = 667, a multiple of
    neither 32 nor 64): Vertical-Slash sub-blocks start mid-tile and the
    window heads' first tiles are partial."""
    heads = [vs(64, 50, 90), ashape(32, 200), dense(), vs(33, 10, 300)]
    run_and_check(workload(51, 1, 4, 2, 1000, heads, Nq=333), "unaligned chunk")


def test_token_heads_mixed_with_other_kinds():
    """Token-list heads (one list per query, shared by those heads) next to
    Vertical-Slash, block and dense heads in one call; some queries have an
    empty list (O = 0, LSE = -inf)."""
    N, cap = 600, 100
    kinds_plan = [synth.HeadPlan(dsa.TOKEN), vs(64, 30, 40), blk("topk", 3), synth.HeadPlan(dsa.TOKEN), dense()]
    w = workload(60, 1, 5, 5, N, kinds_plan)
    B, H, Hkv, Nq, Nk, d = w.shape
    g = np.random.default_rng(7)
    lists = []
    for i in range(Nq):
        n = 0 if i % 97 == 5 else int(g.integers(1, min(cap, i + 1) + 1))
        lists.append(np.sort(g.choice(i + 1, size=n, replace=False)).astype(np.int32))
    tok = dsa.TokenIndex.empty(1, Nq, cap, DEV)
    idx = torch.zeros(1, Nq, cap, dtype=torch.int32)
    cnt = torch.zeros(1, Nq, dtype=torch.int32)
    for i, L in enumerate(lists):
        idx[0, i, :len(L)] = torch.from_numpy(L)
        cnt[0, i] = len(L)
    tok.idx.copy_(idx)
    tok.count.copy_(cnt)
    sets = {(0, h): oracle_head_sets(w, 0, h) for h in range(H) if w.heads[h].kind != dsa.TOKEN}
    _, vsi, bi = upload_sets(w, sets, DEV)
    kinds = [int(p.kind) for p in w.heads]
    o, lse = dsa.sparse_prefill_attn(w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), kinds, vs=vsi, blk=bi, tok=tok,
                                     out_dtype=dsa.OUT_F32)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    rows = list(range(Nq))
    for h in range(H):
        if w.heads[h].kind == dsa.TOKEN:
            ref_o, ref_l = O.attention_rows(f64(w.q[0, h]), f64(w.k[0, h]), f64(w.v[0, h]), rows, lists)
        else:
            ref_o, ref_l = oracle_attention_rows(w, sets, 0, h, rows)
        assert_attention_close(o[0, h], lse[0, h], ref_o, ref_l, f"mixed-with-tokens h={h}")


def _bands(start, widths, gaps, n):
    """Offsets of bands of the given widths separated by the given gaps."""
    out, o = [], start
    for wd, gp in zip(widths, gaps):
        out.extend(range(o, min(n, o + wd)))
        o += wd + gp
    return np.array(sorted(set(x for x in out if x < n)), dtype=np.int64)


@pytest.mark.parametrize("Nk,Nq", [(1200, 1200), (1000, 333), (700, 129)])
def test_vertical_slash_constructed_sets(Nk, Nq):
    """Vertical-Slash attention on hand-built sets that stress the sub-block
    step schedule: bands of 1 to 100 consecutive diagonals separated by gaps
    on both sides of 32 and 63 (where a run may or may not continue), lone
    diagonals next to offset 0 (sub-blocks that cross the causal edge) and at
    the last offset, every offset at once, columns only, and both empty.  The
    oracle is given the same sets."""
    rng = np.random.default_rng(Nk + Nq)
    widths = [1, 1, 33, 64, 65, 31, 32, 1, 100, 2, 1, 40]
    gaps = [32, 33, 62, 63, 64, 65, 96, 97, 128, 31, 1, 0]
    S0 = _bands(0, widths, gaps, Nk)
    S1 = _bands(5, widths[::-1], gaps[::-1], Nk)
    S2 = np.array(sorted({1, 2, 31, 32, 33, 95, Nk - 1} | set(rng.choice(Nk, 40, replace=False).tolist())),
                  dtype=np.int64)
    S3 = np.arange(Nk, dtype=np.int64)
    cols = lambda n: np.sort(rng.choice(Nk, n, replace=False)).astype(np.int64)
    plan = [(cols(30), S0), (cols(5), S1), (np.array([0, 1, Nk - 1], dtype=np.int64), S2), (cols(12), S3),
            (cols(50), np.zeros(0, dtype=np.int64)), (np.zeros(0, dtype=np.int64), np.zeros(0, dtype=np.int64))]
    H = len(plan)
    heads = [vs(64, 1, 1) for _ in range(H)]
    w = workload(70 + Nq, 1, H, 2 if H % 2 == 0 else 1, Nk, heads, Nq=Nq)
    sets = {(0, h): ("vs", V, S, None, None) for h, (V, S) in enumerate(plan)}
    kinds, vsi, bi = upload_sets(w, sets, DEV)
    o, lse = dsa.sparse_prefill_attn(w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), kinds, vs=vsi, out_dtype=dsa.OUT_F32)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    rows = list(range(Nq))
    for (b, h) in sets:
        ref_o, ref_l = oracle_attention_rows(w, sets, b, h, rows)
        assert_attention_close(o[b, h], lse[b, h], ref_o, ref_l, f"constructed sets h={h}")


@pytest.mark.parametrize("Nk", [1000, 1345])
def test_block_head_pairs(Nk):
    """Neighbouring block heads of one KV group (blocks of 64) run as pairs:
    an item is one query tile of both heads, over the merge of their lists.
    Batch 2, GQA 8 / 2, an odd number of query tiles (the last pair of tiles
    has no second tile), a head whose neighbour is not a block head, and
    top-k and threshold rules side by side."""
    heads = [blk("topk", 5, True), blk("thresh"), blk("topk", 3), dense(),
             blk("thresh"), blk("topk", 7, True), vs(64, 20, 40), blk("topk", 2)]
    run_and_check(workload(80 + Nk, 2, 8, 2, Nk, heads), f"block pairs N={Nk}")


@pytest.mark.parametrize("block", [16, 32, 64, 128])
def test_block_heads_in_a_chunk(block):
    """Block heads in a prefill chunk that starts at key 512 (a multiple of every
    block size), with a ragged end: the lists are per query block of the chunk
    and hold absolute key blocks.  Batch 2, GQA 8/2, top-k and threshold heads
    beside Vertical-Slash and dense heads; for blocks of 64 the neighbouring
    block heads of a KV group run as pairs."""
    heads = [blk("topk", 3, True, block), blk("thresh", block=block), vs(64, 20, 40), dense(),
             blk("thresh", block=block), blk("topk", 5, False, block), blk("topk", 2, True, block), ashape(16, 64)]
    run_and_check(workload(140 + block, 2, 8, 2, 1300, heads, Nq=788), f"block {block} chunk")


@pytest.mark.parametrize("Nk,Nq,block", [(1025, 1, 64), (1041, 17, 16), (640, 128, 128), (2049, 1, 32)])
def test_small_chunks_at_the_end(Nk, Nq, block):
    """Chunks of one to a few queries at the end of the keys (q_offset a
    multiple of the block): block heads of both rules beside Vertical-Slash,
    A-shape and dense heads, batch 2."""
    heads = [blk("topk", 3, True, block), blk("thresh", block=block), vs(min(Nq, 64), 20, 40), dense(),
             ashape(16, 64), blk("topk", 1, False, block), vs(min(Nq, 64), 0, 30), blk("thresh", block=block)]
    run_and_check(workload(170 + Nk + Nq, 2, 8, 2, Nk, heads, Nq=Nq), f"chunk Nk={Nk} Nq={Nq} block {block}")

#!/usr/bin/env python3
"""Benchmark of dynamic sparse prefill attention on one MI355X.

Default workload (the headline): one attention layer at N = 131072 with mixed
per-head patterns (32 Q / 8 KV heads, d = 128, bf16): A-shape sets for heads
0-10, Vertical-Slash scoring + selection for heads 11-26, mean-pooled block
top-128 for heads 27-31, then sparse attention over all 32 heads.  A step is
that whole pass (index build + attention) over inputs already resident in HBM.

Other workloads (--workload) measure the remaining settings with the same
protocol; they are reported alongside, the headline line is the default.

Prints one JSON line: the metric and its value (effective TFLOP/s = selected
work / step time), ms per step and per phase, the roofline record of the
attention kernel (achieved rate on the selected work, peak, fraction; when the
stored counter record matches the attention sources, the copy-calibrated HBM
traffic and the rate on the MFMA work the launch executes) and the fp64
CPU oracle's rate on a bounded sample.  --block-sweep prints the block-size
sweep instead.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import dynamic_sparse_attention_mean_amd as dsa  # noqa: E402
from dynamic_sparse_attention_mean_amd.pipeline import SparsePrefillLayer  # noqa: E402

METRIC = "ms per attn layer (index build + sparse attn) at 128K; effective TFLOP/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "dynamic_sparse_attention_mean_amd", "csrc")
# sources the attention kernel is compiled from: a counter record holds only while these are unchanged
ATTN_SRCS = [os.path.join(CSRC, f) for f in ("attn.hip", "common.h", "internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernel_mixed128k_traffic.json")

WORKLOADS = {
    "mixed128k": ("mixed-pattern layer, 32 Q / 8 KV heads, d=128, N=131072: heads 0-10 A-shape (sink 128, local "
                  "2048), 11-26 Vertical-Slash (last_q 64, 1000 cols, 4096 diags), 27-31 block top-128 of 64",
                  lambda: synth.config(3)),
    "mixed128k-pooled": ("mixed-pattern layer as mixed128k, with the Vertical-Slash heads 11-26 discovered from "
                         "pooled block scores (block 64: 16 key blocks, 32 block offsets)",
                         lambda: synth.config(3, vs_rule="pooled")),
    "vs4k": ("one Vertical-Slash head, N=4096, last_q 64, 256 cols + 256 diags", lambda: synth.config(1)),
    "dense32k": ("dense causal attention, 32 Q / 8 KV heads, d=128, N=32768 (every key of every row selected)",
                 lambda: synth.dense_layer()),
    "block32k-topk": ("8 block heads, N=32768, block 64, top-16 + first + diagonal", lambda: synth.config(2)),
    "block32k-thresh": ("8 block heads, N=32768, block 64, threshold max - ln 20 + first + diagonal",
                        lambda: synth.config(2, mode="thresh")),
    "thresh4k": ("32 Q / 8 KV heads, N=4096, block 128, threshold max - ln 20", lambda: synth.config(4, N=4096)),
    "thresh256k": ("32 Q / 8 KV heads, N=262144, block 128, threshold max - ln 20",
                   lambda: synth.config(4, N=262144)),
    "indexer128k": ("indexer top-2048 over N=131072 for an 8192-query chunk (64 heads, dense) + token attention "
                    "(16 heads)", lambda: synth.config(5)),
    "indexer128k-routed": ("indexer top-2048 over N=131072, 8 of 64 heads routed per query + token attention "
                           "(16 heads)", lambda: synth.config(5, route_heads=8)),
    "indexer128k-mqa": ("indexer top-2048 over N=131072 for an 8192-query chunk (64 heads, dense) + token attention "
                        "(16 heads sharing one K/V, MQA)", lambda: synth.config(5, kv_heads=1)),
    "indexer128k-hier": ("hierarchical indexer top-2048 over N=131072: 8 of 64 heads routed per query pick 8192 "
                         "candidates, all 64 heads rescore them + token attention (16 heads)",
                         lambda: synth.config(5, route_heads=8, cand=8192)),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def selected_count_layer(layer, w):
    """Exact sum_h sum_i |M_h(i)| of the layer's index sets (read back from the device)."""
    B, H, Hkv, Nq, Nk, d = w.shape
    pos = torch.arange(Nq, dtype=torch.int64) + w.q_offset
    total = 0
    vsi, bi = layer.vs_index, layer.blk_index
    for b in range(B):
        for h in range(H):
            kind = layer.kinds[h]
            if kind == dsa.TOKEN:
                continue                  # token heads are counted from their token lists by the caller
            if kind == dsa.DENSE:
                total += int((pos + 1).sum())
            elif kind == dsa.VS:
                V = vsi.cols[b, h, :int(vsi.cols_count[b, h])].cpu().long().sort().values
                S = vsi.diags[b, h, :int(vsi.diags_count[b, h])].cpu().long().sort().values
                cols = torch.searchsorted(V, pos, right=True).sum()
                diags = torch.searchsorted(S, pos, right=True).sum()
                both = 0
                for i0 in range(0, V.numel(), 128):
                    s = V[i0:i0 + 128, None] + S[None, :]
                    both += int(((s >= w.q_offset) & (s < w.q_offset + Nq)).sum())
                total += int(cols + diags) - both
            else:
                block = bi.block
                cnt = bi.count[b, h].cpu()
                idx = bi.idx[b, h].cpu()
                for I in range(cnt.numel()):
                    r0, r1 = I * block, min((I + 1) * block, Nq)
                    if r1 <= r0:
                        continue
                    J = idx[I, :int(cnt[I])].long()
                    total += int((J < I).sum()) * block * (r1 - r0)
                    total += int((J == I).sum()) * ((r1 - r0) * (r1 - r0 + 1) // 2)
    return total


def _oracle_threads():
    threads = torch.get_num_threads()
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [threads])
    except Exception:
        pass
    return threads


def _host_cpu():
    """nproc and the CPU model of the host the oracle runs on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return os.cpu_count(), model


def cpu_baseline(w, sample_rows=512, seed=0):
    """The fp64 oracle on a bounded sample of the same workload, scaled to the
    layer.  Every index set is the oracle's own (index rules timed in full for
    every head); attention is timed on `sample_rows` random rows per head and
    scaled to all rows."""
    import oracle as O
    from oracle.bf16 import to_f64
    B, H, Hkv, Nq, Nk, d = w.shape
    rng = np.random.default_rng(seed)
    t_index = t_attn = 0.0
    for h, p in enumerate(w.heads):
        kvh = h // (H // Hkv)
        kf = None
        t0 = time.perf_counter()
        if p.kind == dsa.VS and p.ashape:
            V, S = O.ashape_sets(Nk, p.sink, p.local)
        elif p.kind == dsa.VS:
            kf = to_f64(w.k[0, kvh])
            v, s = O.vs_scores(to_f64(w.q[0, h, Nq - p.last_q:]), kf)
            V, S = O.vs_select(v, s, p.nv, p.ns)
        elif p.kind == dsa.BLOCK:
            kf = to_f64(w.k[0, kvh])
            S_ = O.block_scores(O.block_means(to_f64(w.q[0, h]), p.block), O.block_means(kf, p.block))
            sel = O.select_blocks(S_, p.mode, k=p.topk, log_alpha=p.log_alpha, force_first=p.force_first,
                                  force_diag=p.force_diag)
        t_index += time.perf_counter() - t0
        rows = np.sort(rng.choice(Nq, sample_rows, replace=False))
        if p.kind == dsa.VS:
            rs = [O.row_set_vs(int(i) + w.q_offset, V, S) for i in rows]
        elif p.kind == dsa.BLOCK:
            rs = [O.row_set_block(int(i), sel, p.block, Nk) for i in rows]
        else:
            rs = [O.row_set_dense(int(i) + w.q_offset) for i in rows]
        kf = to_f64(w.k[0, kvh]) if kf is None else kf
        vf = to_f64(w.v[0, kvh])
        q = to_f64(w.q[0, h][torch.from_numpy(rows)])
        t0 = time.perf_counter()
        O.attention_rows(q, kf, vf, list(range(len(rows))), rs)
        t_attn += time.perf_counter() - t0
    return dict(t_index=t_index, t_attn_layer=t_attn * (Nq / sample_rows), t_attn_sample=t_attn,
                threads=_oracle_threads(), sample=f"index rules of all {H} heads in full; attention on "
                f"{sample_rows} random rows per head, scaled to {Nq} rows")


def cpu_baseline_indexer(w, sample_queries=32, seed=0):
    """The fp64 oracle indexer (router, scores, top-k) and token attention on a
    few sampled queries of the chunk, scaled to the chunk."""
    import oracle as O
    from oracle.bf16 import to_f64
    B, H, Hkv, Nq, Nk, d = w.shape
    qi, ki, wt = w.extra["q_idx"], w.extra["k_idx"], w.extra["w"]
    topk, route, cand = w.extra["topk"], w.extra["route_heads"], w.extra.get("cand", 0)
    rows = np.sort(np.random.default_rng(seed).choice(Nq, sample_queries, replace=False))
    kf = to_f64(ki)
    t_index = t_attn = 0.0
    sets = []
    for i in rows:
        p = int(i) + w.q_offset
        t0 = time.perf_counter()
        if cand:
            sets.append(O.hierarchical_tokens(to_f64(qi[i:i + 1]), kf, wt[i:i + 1].double().numpy(), p, route, cand,
                                              topk)[0])
            t_index += time.perf_counter() - t0
            continue
        heads = None
        if route:
            heads = O.router_heads(to_f64(qi[i:i + 1]), kf, wt[i:i + 1].double().numpy(), p, route_heads=route)[0]
        sc = O.indexer_row(to_f64(qi[i]), kf, wt[i].double().numpy(), p, heads)
        sets.append(O.token_topk(sc, p, topk))
        t_index += time.perf_counter() - t0
    for h in range(H):
        kk = to_f64(w.k[0, h // (H // Hkv)])
        vv = to_f64(w.v[0, h // (H // Hkv)])
        q = to_f64(w.q[0, h][torch.from_numpy(rows)])
        t0 = time.perf_counter()
        O.attention_rows(q, kk, vv, list(range(len(rows))), sets)
        t_attn += time.perf_counter() - t0
    scale = Nq / sample_queries
    return dict(t_index=t_index * scale, t_attn_layer=t_attn * scale, t_attn_sample=t_attn,
                threads=_oracle_threads(), sample=f"router + indexer scores + top-{topk}"
                + (f" of {cand} rescored candidates" if cand else "") + f" and attention of all {H} "
                f"heads on {sample_queries} random queries of the chunk, scaled to {Nq} queries")


def time_steps(fns, steps, warmup, stream):
    """Run `fns` (list of phases) per step; HIP events bracket every phase on `stream`."""
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        for j, f in enumerate(fns):
            f()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    phases = [float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)])) for j in range(len(fns))]
    total = float(np.mean([ev[i][0].elapsed_time(ev[i][-1]) for i in range(steps)]))
    return total, phases, wall


def time_cold(fns, reps, stream, flush_bytes=512 << 20):
    """Cold-cache steps: before each, a write of `flush_bytes` of scratch evicts the inputs from L2
    and the 256 MB Infinity Cache; HIP events bracket only the step's phases."""
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device=torch.device("cuda", 0))
    tot, ph = [], []
    for r in range(reps):
        scratch.fill_(r & 0xFF)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
        ev[0].record(stream)
        for j, f in enumerate(fns):
            f()
            ev[j + 1].record(stream)
        torch.cuda.synchronize()
        tot.append(ev[0].elapsed_time(ev[-1]))
        ph.append([ev[j].elapsed_time(ev[j + 1]) for j in range(len(fns))])
    del scratch
    return float(np.mean(tot)), [float(np.mean([x[j] for x in ph])) for j in range(len(fns))]


def attn_src_digest():
    h = hashlib.sha256()
    for p in ATTN_SRCS:
        h.update(open(p, "rb").read())
    return h.hexdigest()


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size: the reference run that
    scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps, "attn_src_sha256": attn_src_digest()}),
          flush=True)


def counter_record():
    """The committed rocprofv3 counter record of the attention launch on the
    mixed128k layer, if it was taken on the attention sources as they are now."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE))
        return rec if rec.get("attn_src_sha256") == attn_src_digest() else None
    except Exception:
        return None


def traffic_record():
    """HBM bytes (read + written) per attention launch, from committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs scaled by the copy calibration, if they were
    taken on the attention sources as they are now."""
    rec = counter_record()
    try:
        return rec["bytes_per_launch"]["total"] if rec else None
    except Exception:
        return None


def executed_record(ms_attn):
    """MFMA work the attention launch executes (SQ_INSTS_VALU_MFMA_MOPS_BF16 x
    512 FLOP, from the committed counter record) against the measured attention
    time: the rate counted on executed rather than selected FLOPs."""
    rec = counter_record()
    try:
        flop = rec["mfma_mops_bf16"] * rec["mfma_flop_per_mop"]
    except Exception:
        return None
    tf = flop / (ms_attn * 1e-3) / 1e12
    return {"flop": flop, "achieved": round(tf, 3), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "source": "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 per launch (profiles/attn_kernel_mixed128k_traffic.json)"}


def block_sweep(args, dev, stream):
    """Block-size sweep on single planted keys (MoBA: the router's SNR grows as
    sqrt(d / B)): the same data and the same key budget (1024 keys per query
    block) for B = 16, 32, 64, 128.  Recall = planted keys in blocks before the
    query block that the GPU's selection keeps, over all such keys; time = one
    step of the layer (index build + attention).  One JSON line."""
    sweep = []
    for blk in (16, 32, 64, 128):
        w = synth.token_planted(block=blk)
        B, H, Hkv, Nq, Nk, d = w.shape
        q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
        layer = SparsePrefillLayer(w.heads, B, H, Hkv, Nk, dev, out_dtype=dsa.OUT_BF16, want_lse=True)
        phases = [lambda: layer.build_indices(q, k), lambda: layer.attention(q, k, v)]
        ms_step, (ms_index, ms_attn), _ = time_steps(phases, args.steps, args.warmup, stream)
        f_sel = 4 * d * selected_count_layer(layer, w)
        idx = layer.blk_index.idx[0].cpu().numpy()
        cnt = layer.blk_index.count[0].cpu().numpy()
        hit = tot = 0
        for h in range(H):
            pb = w.extra["planted_keys"][h].numpy() // blk
            for I in range(idx.shape[1]):
                rel = pb[pb < I]
                if rel.size:
                    hit += int(np.isin(rel, idx[h, I, :cnt[h, I]]).sum())
                    tot += int(rel.size)
        sweep.append({"block": blk, "recall": round(hit / tot, 4), "snr_model": round(w.extra["alpha"] * math.sqrt(d / blk), 3),
                      "ms_index": round(ms_index, 4), "ms_attn": round(ms_attn, 4), "ms_step": round(ms_step, 4),
                      "effective_tflops": round(f_sel / (ms_step * 1e-3) / 1e12, 2),
                      "density": round(f_sel / (2 * d * H * Nq * (Nq + 1)), 5)})
        log(f"[bench] block {blk}: recall {sweep[-1]['recall']}, {ms_step:.3f} ms/step")
        del layer
        torch.cuda.synchronize()
    rec = {"metric": "recall of planted keys and ms per layer against the block size", "unit": "ms", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "block-size sweep: 8 heads, N=32768, d=128, 64 single planted keys per head "
                                  "(alpha 1), top-(1024 / B) blocks + first + diagonal", "name": "blocksweep32k",
                      "sweep": sweep}}
    print(json.dumps(rec), flush=True)


def vs_compare(args, dev, stream):
    """Vertical-Slash discovery on the 128K mixed layer's data: last_q scoring
    against pooled block scores, for the 16 Vertical-Slash heads.  For each
    rule: time of its index build (those heads only) and of the whole layer,
    recall of the planted vertical keys (the heads' KV group's 64 planted rows),
    the attention mass the sets keep (the dense softmax weight of the selected
    keys, exp(LSE_sparse - LSE_dense), averaged over every row of the heads),
    and the heads' attention output against dense causal attention (mean and
    max abs difference over every row).  One JSON line."""
    w = synth.config(3)
    B, H, Hkv, Nq, Nk, d = w.shape
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    vs_heads = [h for h, p in enumerate(w.heads) if p.kind == dsa.VS and not p.ashape]
    # dense causal reference (every head; only the Vertical-Slash heads are compared)
    dense_o = torch.empty(B, H, Nq, d, dtype=torch.float32, device=dev)
    dense_lse = torch.empty(B, H, Nq, dtype=torch.float32, device=dev)
    dws = torch.empty(dsa.workspace_size(dsa.OP_ATTN, dsa.make_shape(q, k)), dtype=torch.uint8, device=dev)
    dsa.sparse_prefill_attn(q, k, v, [dsa.DENSE] * H, out_dtype=dsa.OUT_F32, o=dense_o, lse=dense_lse, ws=dws)
    torch.cuda.synchronize()
    del dws
    out = {}
    for rule in ("last_q", "pooled"):
        pooled_plan = synth.HeadPlan(dsa.VS, pooled=True, block=64, nv_blocks=16, ns_blocks=32)
        plan = [pooled_plan if (rule == "pooled" and h in vs_heads) else w.heads[h] for h in range(H)]
        wr = synth.Workload(w.name, w.q, w.k, w.v, plan, w.q_offset, w.extra)
        layer = SparsePrefillLayer(plan, B, H, Hkv, Nk, dev, out_dtype=dsa.OUT_F32, want_lse=True)
        vsi = layer.vs_index
        if rule == "pooled":
            (blk, nvb, nsb), hs = next(iter(layer.pooled.items()))
            build_vs = lambda: dsa.build_index_vs_pooled(q, k, hs, blk, nvb, nsb, vsi, ws=layer.ws)
        else:
            (lq, nv, ns), hs = next(iter(layer.vs.items()))
            build_vs = lambda: dsa.build_index_vs(q, k, hs, lq, nv, ns, vsi, ws=layer.ws)
        ms_vs, _, _ = time_steps([build_vs], args.steps, args.warmup, stream)
        phases = [lambda: layer.build_indices(q, k), lambda: layer.attention(q, k, v)]
        ms_step, (ms_index, ms_attn), _ = time_steps(phases, args.steps, args.warmup, stream)
        rv = 0.0
        for h in vs_heads:
            cols = vsi.cols[0, h, :int(vsi.cols_count[0, h])].cpu().numpy()
            rv += np.isin(w.extra["planted_cols"][h // (H // Hkv)].numpy(), cols).mean()
        mass = torch.exp(layer.lse[0, vs_heads].double() - dense_lse[0, vs_heads].double())
        diff = (layer.o[0, vs_heads] - dense_o[0, vs_heads]).abs()
        f_sel = 4 * d * selected_count_layer(layer, wr)
        out[rule] = {"ms_vs_index": round(ms_vs, 4), "ms_index": round(ms_index, 4), "ms_attn": round(ms_attn, 4),
                     "ms_step": round(ms_step, 4), "effective_tflops": round(f_sel / (ms_step * 1e-3) / 1e12, 2),
                     "recall_vertical": round(rv / len(vs_heads), 4),
                     "attention_mass_kept": round(float(mass.mean()), 4),
                     "attention_mass_kept_min_row": round(float(mass.min()), 4),
                     "vs_heads_vs_dense_mean_abs": round(float(diff.mean()), 5),
                     "vs_heads_vs_dense_max_abs": round(float(diff.max()), 4)}
        log(f"[bench] {rule}: {out[rule]}")
        del layer
        torch.cuda.synchronize()
    rec = {"metric": "Vertical-Slash discovery on the 128K mixed layer: last_q scoring vs pooled block scores",
           "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": WORKLOADS["mixed128k"][0], "name": "vscompare128k", "vs_heads": vs_heads,
                      "pooled": "block 64, 16 key blocks (1024 columns), 32 block offsets (<= 4064 diagonals)",
                      "rules": out}}
    print(json.dumps(rec), flush=True)


def attn_kind(args, dev, stream):
    """One pattern kind of the headline layer on its own, through the public
    ABI: a layer of the 128K mixed workload's heads of three or four whole KV
    groups, every head given that kind's plan (A-shape: heads 0-11 on KV heads
    0-2; Vertical-Slash: heads 12-27 on KV heads 3-6; block top-128 of 64:
    heads 24-31 on KV heads 6-7), on those heads' own data.  Its index build
    and attention are timed like a layer step.  One JSON line."""
    w = synth.config(3)
    B, H, Hkv, Nq, Nk, d = w.shape
    rep = H // Hkv
    span = {"ashape": (0, 12), "vs": (12, 28), "block": (24, 32)}[args.attn_kind]
    plan_of = {"ashape": w.heads[0], "vs": w.heads[12], "block": w.heads[31]}[args.attn_kind]
    h0, h1 = span
    q = w.q[:, h0:h1].contiguous().to(dev)
    k = w.k[:, h0 // rep:h1 // rep].contiguous().to(dev)
    v = w.v[:, h0 // rep:h1 // rep].contiguous().to(dev)
    sub = synth.Workload(f"{w.name}-{args.attn_kind}", q, k, v, [plan_of] * (h1 - h0), w.q_offset, w.extra)
    Hs, Hkvs = h1 - h0, (h1 - h0) // rep
    layer = SparsePrefillLayer(sub.heads, B, Hs, Hkvs, Nk, dev, out_dtype=dsa.OUT_BF16, want_lse=True)
    phases = [lambda: layer.build_indices(q, k), lambda: layer.attention(q, k, v)]
    ms_step, (ms_index, ms_attn), _ = time_steps(phases, args.steps, args.warmup, stream)
    f_sel = 4 * d * selected_count_layer(layer, sub)
    rec = {"metric": f"attention of the 128K mixed layer's data, {args.attn_kind} heads only", "unit": "TFLOP/s",
           "value": round(f_sel / (ms_attn * 1e-3) / 1e12, 2), "ms_attn": round(ms_attn, 4),
           "ms_index": round(ms_index, 4), "heads": list(range(h0, h1)), "kv_heads": list(range(h0 // rep, h1 // rep)),
           "f_sel": f_sel, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "dtype": "bf16",
           "data": "synthetic", "config": {"workload": WORKLOADS["mixed128k"][0], "name": f"mixed128k-{args.attn_kind}"}}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixed128k", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache steps (profiling runs: every launch is then a warm one)")
    ap.add_argument("--block-sweep", action="store_true",
                    help="only run the block-size sweep (recall of planted keys, time per block size) and exit")
    ap.add_argument("--vs-compare", action="store_true",
                    help="only compare Vertical-Slash discovery by last_q scoring and by pooled block scores on the "
                         "128K mixed layer (time, recall, output against dense) and exit")
    ap.add_argument("--attn-kind", choices=["ashape", "vs", "block"],
                    help="only time a layer of one pattern kind on the 128K mixed layer's data and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy three times (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: heads (KV groups) shard across GPUs with no exchange, so each GPU runs "
              f"this step on its share; --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    dev = torch.device("cuda", 0)
    if args.block_sweep:
        block_sweep(args, dev, torch.cuda.current_stream(dev))
        return
    if args.vs_compare:
        vs_compare(args, dev, torch.cuda.current_stream(dev))
        return
    if args.attn_kind:
        attn_kind(args, dev, torch.cuda.current_stream(dev))
        return
    desc, make = WORKLOADS[args.workload]
    log(f"[bench] generating {args.workload}")
    w = make()
    B, H, Hkv, Nq, Nk, d = w.shape
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    stream = torch.cuda.current_stream(dev)
    extra = {}

    if args.workload.startswith("indexer"):
        qi, ki, wt = w.extra["q_idx"].to(dev), w.extra["k_idx"].to(dev), w.extra["w"].to(dev)
        topk, route, cand = w.extra["topk"], w.extra["route_heads"], w.extra.get("cand", 0)
        tok = dsa.TokenIndex.empty(1, Nq, topk, dev)
        shape = dsa.Shape(1, 1, 1, Nq, Nk, 128, Nk - Nq)
        if cand:
            ws = torch.empty(dsa.workspace_size(dsa.OP_TOKENS_HIER, shape, [qi.shape[1], route, cand, topk]),
                             dtype=torch.uint8, device=dev)
        else:
            ws = torch.empty(dsa.workspace_size(dsa.OP_TOKENS, shape, [qi.shape[1], route, topk]), dtype=torch.uint8,
                             device=dev)
        o = torch.empty(1, H, Nq, d, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(1, H, Nq, dtype=torch.float32, device=dev)
        aws = torch.empty(dsa.workspace_size(dsa.OP_ATTN, dsa.make_shape(q, k)), dtype=torch.uint8, device=dev)
        if cand:
            build = lambda: dsa.build_index_tokens_hier(qi, ki, wt, cand, topk, tok, route_heads=route, ws=ws)
        else:
            build = lambda: dsa.build_index_tokens(qi, ki, wt, topk, tok, route_heads=route, ws=ws)
        attn = lambda: dsa.sparse_prefill_attn(q, k, v, [dsa.TOKEN] * H, tok=tok, out_dtype=dsa.OUT_BF16, o=o,
                                               lse=lse, ws=aws)
        log(f"[bench] timing {args.steps} steps")
        ms_step, (ms_index, ms_attn), wall = time_steps([build, attn], args.steps, args.warmup, stream)
        if not args.no_cold:
            cold, (cold_i, cold_a) = time_cold([build, attn], 3, stream)
            extra.update(ms_step_cold=round(cold, 4), ms_index_cold=round(cold_i, 4), ms_attn_cold=round(cold_a, 4))
        n_sel = int(tok.count.sum().item()) * H
        f_sel = 4 * d * n_sel
        hsel = qi.shape[1] if route == 0 else route
        pos = np.arange(Nq, dtype=np.float64) + (Nk - Nq)
        extra["indexer_flop"] = float(2 * 128 * hsel * (pos + 1).sum())
        if cand:
            # the rescoring of the candidates by every head
            extra["indexer_flop"] += float(2 * 128 * qi.shape[1] * np.minimum(pos + 1, cand).sum())
        extra["indexer_tflops"] = round(extra["indexer_flop"] / (ms_index * 1e-3) / 1e12, 2)
        # K and V rows gathered: once per head, or once per group of up to 16
        # heads when 8 or more heads share a KV head (the grouped kernel)
        rep = H // Hkv
        n_gather = Hkv * math.ceil(rep / 16) if rep >= 8 else H
        extra["gather_bytes"] = (n_sel // H) * n_gather * 2 * d * 2
        extra["token_attn_gbs"] = round(extra["gather_bytes"] / (ms_attn * 1e-3) / 1e9, 1)
    else:
        layer = SparsePrefillLayer(w.heads, B, H, Hkv, Nk, dev, out_dtype=dsa.OUT_BF16, want_lse=True)
        torch.cuda.synchronize()
        log(f"[bench] timing {args.steps} steps")
        phases = [lambda: layer.build_indices(q, k), lambda: layer.attention(q, k, v)]
        ms_step, (ms_index, ms_attn), wall = time_steps(phases, args.steps, args.warmup, stream)
        if not args.no_cold:
            cold, (cold_i, cold_a) = time_cold(phases, 3, stream)
            extra.update(ms_step_cold=round(cold, 4), ms_index_cold=round(cold_i, 4), ms_attn_cold=round(cold_a, 4))
        f_sel = 4 * d * selected_count_layer(layer, w)
        if args.workload.startswith("thresh"):
            # the dense causal comparison on the same inputs (informative)
            dense_o = torch.empty(B, H, Nq, d, dtype=torch.bfloat16, device=dev)
            dws = torch.empty(dsa.workspace_size(dsa.OP_ATTN, dsa.make_shape(q, k)), dtype=torch.uint8, device=dev)
            dense = lambda: dsa.sparse_prefill_attn(q, k, v, [dsa.DENSE] * H, out_dtype=dsa.OUT_BF16, o=dense_o,
                                                    ws=dws, want_lse=False)
            ms_dense, _, _ = time_steps([dense], 2, 1, stream)
            diff = (layer.o.float() - dense_o.float()).abs()
            extra["ms_dense_attn"] = round(ms_dense, 3)
            extra["speedup_vs_dense"] = round(ms_dense / ms_step, 2)
            extra["sparse_vs_dense_max_abs"] = round(float(diff.max()), 4)
            extra["sparse_vs_dense_mean_abs"] = round(float(diff.mean()), 5)
    log(f"[bench] {ms_step:.3f} ms/step (index {ms_index:.3f}, attention {ms_attn:.3f}); wall {wall:.2f}s")
    dense_flop = 4 * d * H * (Nq * (Nq + 1) // 2 + Nq * w.q_offset)
    tflops = f_sel / (ms_step * 1e-3) / 1e12
    attn_tflops = f_sel / (ms_attn * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "name": args.workload, "batch": B, "seq_len": Nk, "heads": H, "kv_heads": Hkv,
                   "ms_index": round(ms_index, 4), "ms_attn": round(ms_attn, 4), "f_sel": f_sel,
                   "density": round(f_sel / dense_flop, 5), **extra},
    }
    if args.workload.startswith("indexer"):
        rec["roofline"] = {"bound": "mfma", "achieved": extra["indexer_tflops"], "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(extra["indexer_tflops"] / PEAK_BF16_TFLOPS, 4),
                           "traffic": None,
                           "kernel": ("qk_heads_kernel + token_select_kernel + cand_score_kernel + cand_select_kernel "
                                      "(build_index_tokens_hier)") if w.extra.get("cand", 0) else
                                     "qk_heads_kernel + token_select_kernel (build_index_tokens)"}
    else:
        rec["roofline"] = {"bound": "mfma", "achieved": round(attn_tflops, 3), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                           "traffic": traffic_record() if args.workload == "mixed128k" else None,
                           "kernel": "attn_kernel (sparse_prefill_attn)"}
        if args.workload == "mixed128k":
            rec["roofline"]["executed"] = executed_record(ms_attn)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        cb = cpu_baseline_indexer(w) if args.workload.startswith("indexer") else cpu_baseline(w)
        t_cpu = cb["t_index"] + cb["t_attn_layer"]
        nproc, model = _host_cpu()
        rec["cpu_baseline"] = {
            "value": round(f_sel / t_cpu / 1e12, 6), "unit": "TFLOP/s", "cores": cb["threads"], "kind": "oracle",
            "nproc": nproc, "cpu_model": model,
            "sample": f"fp64 numpy oracle, {cb['sample']}; t_index {cb['t_index']:.2f}s, attention sample "
                      f"{cb['t_attn_sample']:.2f}s, layer estimate {t_cpu:.1f}s ({t_cpu * 1e3:.0f} ms per layer); "
                      f"BLAS and torch use {cb['threads']} threads (the process's thread setting, "
                      f"OMP_NUM_THREADS={os.environ.get('OMP_NUM_THREADS', 'unset')}) of the host's {nproc}",
        }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

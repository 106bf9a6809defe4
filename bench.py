#!/usr/bin/env python3
"""Benchmark of one dynamic sparse prefill attention layer on one MI355X.

A step is one pass of the whole hot path over the mixed-pattern 128K layer
(32 Q / 8 KV heads, d = 128, N = 131072, bf16): A-shape sets for heads 0-10,
Vertical-Slash scoring + selection for heads 11-26, mean-pooled block top-128
for heads 27-31, then sparse attention over all 32 heads.  Inputs are seeded and
synthetic and already resident in HBM when the timed region starts.

Prints one JSON line (see the design doc for the fields).
"""
import argparse
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def selected_count(layer, w):
    """Exact sum_h sum_i |M_h(i)| of the layer's index sets (read back from the device)."""
    B, H, Hkv, Nq, Nk, d = w.shape
    pos = torch.arange(Nq, dtype=torch.int64) + w.q_offset
    total = 0
    vsi = layer.vs_index
    bi = layer.blk_index
    for b in range(B):
        for h in range(H):
            kind = layer.kinds[h]
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
                    full = int((J < I).sum()) * block * (r1 - r0)
                    diag = int((J == I).sum()) * ((r1 - r0) * (r1 - r0 + 1) // 2)
                    total += full + diag
    return total


def cpu_baseline(w, layer, sample_rows=64, seed=0):
    """The fp64 oracle on a bounded sample of the same workload, scaled to the layer."""
    import oracle as O
    from oracle.bf16 import to_f64
    threads = torch.get_num_threads()
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    except Exception:
        pass
    B, H, Hkv, Nq, Nk, d = w.shape
    rng = np.random.default_rng(seed)
    t_index = 0.0
    # one head of each dynamic rule, timed, scaled by the number of such heads
    n_vs = sum(1 for p in w.heads if p.kind == dsa.VS and not p.ashape)
    n_blk = sum(1 for p in w.heads if p.kind == dsa.BLOCK)
    sets = {}
    for h, p in enumerate(w.heads):
        kvh = h // (H // Hkv)
        if p.kind == dsa.VS and not p.ashape and "vs" not in sets:
            t0 = time.perf_counter()
            v, s = O.vs_scores(to_f64(w.q[0, h, Nq - p.last_q:]), to_f64(w.k[0, kvh]))
            O.vs_select(v, s, p.nv, p.ns)
            t_index += (time.perf_counter() - t0) * n_vs
            sets["vs"] = 1
        if p.kind == dsa.BLOCK and "blk" not in sets:
            t0 = time.perf_counter()
            S = O.block_scores(O.block_means(to_f64(w.q[0, h]), p.block), O.block_means(to_f64(w.k[0, kvh]), p.block))
            O.select_blocks(S, p.mode, k=p.topk)
            t_index += (time.perf_counter() - t0) * n_blk
            sets["blk"] = 1
    # attention: `sample_rows` random rows per head on the layer's own index sets
    t_attn = 0.0
    flops_sample = 0
    vsi, bi = layer.vs_index, layer.blk_index
    for h in range(H):
        kvh = h // (H // Hkv)
        rows = np.sort(rng.choice(Nq, sample_rows, replace=False))
        if layer.kinds[h] == dsa.VS:
            V = vsi.cols[0, h, :int(vsi.cols_count[0, h])].cpu().numpy()
            S = vsi.diags[0, h, :int(vsi.diags_count[0, h])].cpu().numpy()
            rs = [O.row_set_vs(int(i), V, S) for i in rows]
        elif layer.kinds[h] == dsa.BLOCK:
            sel = [bi.idx[0, h, I, :int(bi.count[0, h, I])].cpu().numpy() for I in range(bi.idx.shape[2])]
            rs = [O.row_set_block(int(i), sel, bi.block, Nk) for i in rows]
        else:
            rs = [O.row_set_dense(int(i)) for i in rows]
        need = np.unique(np.concatenate(rs))
        kk = np.zeros((Nk, d))
        vv = np.zeros((Nk, d))
        kk[need] = to_f64(w.k[0, kvh][torch.from_numpy(need)])
        vv[need] = to_f64(w.v[0, kvh][torch.from_numpy(need)])
        q = to_f64(w.q[0, h][torch.from_numpy(rows)])
        t0 = time.perf_counter()
        O.attention_rows(q, kk, vv, list(range(len(rows))), rs)
        t_attn += time.perf_counter() - t0
        flops_sample += 4 * d * sum(len(r) for r in rs)
    t_attn_layer = t_attn * (Nq / sample_rows)
    return dict(t_index=t_index, t_attn_layer=t_attn_layer, t_attn_sample=t_attn, flops_sample=flops_sample,
                threads=threads, sample_rows=sample_rows)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--n", type=int, default=131072, help="sequence length (the workload is stated at 131072)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the hot path is measured on one device's share; --gpus {args.gpus} is "
              f"not supported (multi-GPU sharding is a design in DESIGN.md, not built).", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    log(f"[bench] generating the mixed-pattern workload N={args.n}")
    w = synth.mixed_layer(N=args.n)
    B, H, Hkv, Nq, Nk, d = w.shape
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    layer = SparsePrefillLayer(w.heads, B, H, Hkv, Nk, dev, out_dtype=dsa.OUT_BF16, want_lse=True)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        layer(q, k, v)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        layer.build_indices(q, k)
        ev[i][1].record(stream)
        layer.attention(q, k, v)
        ev[i][2].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    ms_index = float(np.mean([a.elapsed_time(b) for a, b, c in ev]))
    ms_attn = float(np.mean([b.elapsed_time(c) for a, b, c in ev]))
    log(f"[bench] {ms_step:.3f} ms/step (index {ms_index:.3f}, attention {ms_attn:.3f}); wall {wall:.2f}s")
    f_sel = 4 * d * selected_count(layer, w)
    dense = 4 * d * H * (Nq * (Nq + 1) // 2)
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
        "config": {"workload": f"mixed-pattern layer, 32 Q / 8 KV heads, d=128, N={Nk}, heads 0-10 A-shape "
                               f"(sink 128, local 2048), 11-26 Vertical-Slash (last_q 64, 1000 cols, 4096 diags), "
                               f"27-31 block top-128 of 64",
                   "batch": B, "seq_len": Nk, "heads": H, "kv_heads": Hkv,
                   "ms_index": round(ms_index, 4), "ms_attn": round(ms_attn, 4),
                   "f_sel": f_sel, "density": round(f_sel / dense, 5)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "attn_kernel (sparse_prefill_attn)"},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        cb = cpu_baseline(w, layer)
        t_cpu = cb["t_index"] + cb["t_attn_layer"]
        rec["cpu_baseline"] = {
            "value": round(f_sel / t_cpu / 1e12, 6), "unit": "TFLOP/s", "cores": cb["threads"], "kind": "oracle",
            "sample": f"fp64 numpy oracle: one Vertical-Slash head and one block head index build (scaled by head "
                      f"count) + attention on {cb['sample_rows']} random rows per head (scaled to {Nq} rows); "
                      f"t_index {cb['t_index']:.2f}s, t_attn(sample) {cb['t_attn_sample']:.2f}s, "
                      f"layer estimate {t_cpu:.1f}s",
        }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

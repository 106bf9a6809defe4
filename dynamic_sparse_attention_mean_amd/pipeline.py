"""One attention layer of dynamic sparse prefill: per-head index build + sparse attention.

The per-head pattern table is the product of the method's offline search
("MInference 1.0" explainer, offline per-head pattern search; authors' abstract):
here it is an input, a list with one entry per Q head carrying the fields

  kind   : 1 (Vertical-Slash, with ashape=True for an A-shape head, pooled=True
           for sets discovered from pooled block scores) or 2 (block) or 0 (dense)
  sink, local              (A-shape)
  last_q, nv, ns           (Vertical-Slash)
  block, nv_blocks, ns_blocks  (Vertical-Slash from pooled block scores)
  block, mode, topk, log_alpha, force_first, force_diag   (block rule)

All buffers (index sets, workspaces, outputs) are allocated once in the
constructor, so a call only enqueues library kernels.  When a layer has both
Vertical-Slash and block heads, the block index is built on a second stream
(default priority, with its own workspace) beside the Vertical-Slash index on
the current stream: the two builders read the same Q and K and write disjoint
index sets, and neither fills the chip on its own.  The current stream waits
for both before the attention.
"""
from __future__ import annotations

import math
from collections import OrderedDict

import torch

from . import (BLOCK, DENSE, OUT_F32, OP_ATTN, OP_BLOCK, OP_VS, OP_VS_POOLED, THRESHOLD, TOPK, VS, BlockIndex,
               VSIndex, build_index_ashape, build_index_block, build_index_vs, build_index_vs_pooled, make_shape,
               sparse_prefill_attn, workspace_size)


class SparsePrefillLayer:
    def __init__(self, plan, B, H, Hkv, N, device, out_dtype=OUT_F32, want_lse=True):
        assert len(plan) == H
        self.B, self.H, self.Hkv, self.N = B, H, Hkv, N
        self.device = device
        self.out_dtype = out_dtype
        self.kinds = [int(p.kind) for p in plan]
        self.ashape = OrderedDict()   # (sink, local) -> heads
        self.vs = OrderedDict()       # (last_q, nv, ns) -> heads
        self.pooled = OrderedDict()   # (block, nv_blocks, ns_blocks) -> heads
        self.blk = OrderedDict()      # (block, mode, topk, log_alpha, ff, fd) -> heads
        for h, p in enumerate(plan):
            if p.kind == VS and getattr(p, "ashape", False):
                self.ashape.setdefault((p.sink, p.local), []).append(h)
            elif p.kind == VS and getattr(p, "pooled", False):
                self.pooled.setdefault((p.block, p.nv_blocks, p.ns_blocks), []).append(h)
            elif p.kind == VS:
                self.vs.setdefault((p.last_q, p.nv, p.ns), []).append(h)
            elif p.kind == BLOCK:
                mode = TOPK if p.mode == "topk" else THRESHOLD
                key = (p.block, mode, int(p.topk), float(p.log_alpha), bool(p.force_first), bool(p.force_diag))
                self.blk.setdefault(key, []).append(h)
            elif p.kind != DENSE:
                raise ValueError(f"head {h}: kind {p.kind} is not a layer pattern")
        blocks = {k[0] for k in self.blk}
        if len(blocks) > 1:
            raise ValueError("one block size per layer")
        shape = make_shape(torch.empty(B, H, N, 128, device="meta"), torch.empty(B, Hkv, N, 128, device="meta"))
        self.shape = shape
        cols_cap = max([min(s, N) for s, _ in self.ashape] + [nv for _, nv, _ in self.vs] +
                       [min(N, b * nvb) for b, nvb, _ in self.pooled] + [1])
        diags_cap = max([min(l, N) for _, l in self.ashape] + [ns for _, _, ns in self.vs] +
                        [min(N, (2 * b - 1) * nsb) for b, _, nsb in self.pooled] + [1])
        have_vs = bool(self.ashape or self.vs or self.pooled)
        self.vs_index = VSIndex.empty(B, H, cols_cap, diags_cap, device) if have_vs else None
        self.blk_index = None
        if self.blk:
            block = blocks.pop()
            nqb = -(-N // block)
            cap = 1
            for (blk, mode, topk, _, ff, fd) in self.blk:
                cap = max(cap, nqb if mode == THRESHOLD else min(nqb, topk + int(ff) + int(fd)))
            self.blk_index = BlockIndex.empty(B, H, nqb, cap, block, device)
        ws = workspace_size(OP_ATTN, shape)
        for (lq, nv, ns), hs in self.vs.items():
            ws = max(ws, workspace_size(OP_VS, shape, [len(hs), lq]))
        for key, hs in self.blk.items():
            ws = max(ws, workspace_size(OP_BLOCK, shape, [len(hs), key[0]]))
        for (blk, _, _), hs in self.pooled.items():
            ws = max(ws, workspace_size(OP_VS_POOLED, shape, [len(hs), blk]))
        self.ws = torch.empty(ws, dtype=torch.uint8, device=device)
        # the block builder's own stream and workspace (see the module docstring)
        self.side = None
        if self.blk and (self.vs or self.pooled) and torch.device(device).type == "cuda":
            ws_blk = max(workspace_size(OP_BLOCK, shape, [len(hs), key[0]]) for key, hs in self.blk.items())
            self.ws_blk = torch.empty(ws_blk, dtype=torch.uint8, device=device)
            self.side = torch.cuda.Stream(device=device)
            self.ev_fork = torch.cuda.Event()
            self.ev_join = torch.cuda.Event()
        odt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
        self.o = torch.empty(B, H, N, 128, dtype=odt, device=device)
        self.lse = torch.empty(B, H, N, dtype=torch.float32, device=device) if want_lse else None

    def _build_block(self, q, k, ws):
        for (block, mode, topk, la, ff, fd), hs in self.blk.items():
            build_index_block(q, k, hs, block, mode, topk, self.blk_index, log_alpha=la, force_first=ff,
                              force_diag=fd, ws=ws)

    def build_indices(self, q, k):
        main = None
        if self.side is not None:
            main = torch.cuda.current_stream(q.device)
            self.ev_fork.record(main)
            self.side.wait_event(self.ev_fork)
            with torch.cuda.stream(self.side):
                self._build_block(q, k, self.ws_blk)
            self.ev_join.record(self.side)
        for (sink, local), hs in self.ashape.items():
            build_index_ashape(q, k, hs, sink, local, self.vs_index)
        for (lq, nv, ns), hs in self.vs.items():
            build_index_vs(q, k, hs, lq, nv, ns, self.vs_index, ws=self.ws)
        for (blk, nvb, nsb), hs in self.pooled.items():
            build_index_vs_pooled(q, k, hs, blk, nvb, nsb, self.vs_index, ws=self.ws)
        if main is not None:
            main.wait_event(self.ev_join)
        else:
            self._build_block(q, k, self.ws)

    def attention(self, q, k, v):
        return sparse_prefill_attn(q, k, v, self.kinds, vs=self.vs_index, blk=self.blk_index,
                                   out_dtype=self.out_dtype, o=self.o, lse=self.lse, ws=self.ws,
                                   want_lse=self.lse is not None)

    def __call__(self, q, k, v):
        self.build_indices(q, k)
        return self.attention(q, k, v)

"""Seeded synthetic inputs for dynamic sparse prefill attention.

This module only draws random tensors and plants structure in them.  It holds
none of the method's arithmetic (no pooling, scoring, selection or attention),
so both the fp64 oracle and the HIP path can take their inputs from here.

Recipe (shared by every workload):
  * torch CPU ``Generator(seed)``, fp32 ``randn`` / ``rand``, then ``.to(bfloat16)``
    (round to nearest even).
  * A "direction" is a random N(0, I) vector rescaled to norm sqrt(d), i.e. the
    per-element RMS of an N(0, 1) row.  This keeps a planted dot product at the
    scale of the logits it must stand out from.
  * Planted structure is applied in fp32 before the single rounding to bf16.

The five workloads follow the descriptions of the method's settings: a single
Vertical-Slash head at 4K, block-sparse heads at 32K, a mixed-pattern GQA layer
at 128K, a threshold sweep at 4K / 256K and an indexer top-k chunk at 128K.
The pages measure on public long-context suites (InfiniteBench, RULER, PG-19,
Needle-In-A-Haystack, LongBench); none of those is used.  These seeded shapes
and planted patterns stand in for them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

D = 128

# Pattern kinds, in the order the attention boundary numbers them.
DENSE, VS, BLOCK, TOKEN = 0, 1, 2, 3


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(int(seed))
    return g


def _direction(g: torch.Generator, d: int = D) -> torch.Tensor:
    u = torch.randn(d, generator=g)
    return u * (math.sqrt(d) / u.norm())


def _distinct(g: torch.Generator, count: int, lo: int, hi: int) -> torch.Tensor:
    """`count` distinct integers drawn uniformly from [lo, hi), sorted."""
    span = hi - lo
    count = min(count, span)
    perm = torch.randperm(span, generator=g)[:count]
    return torch.sort(perm + lo).values


@dataclass
class HeadPlan:
    """Per-head pattern assignment (the product of the offline search)."""
    kind: int
    sink: int = 0          # A-shape: sink tokens
    local: int = 0         # A-shape: local window (counts the query itself)
    last_q: int = 0        # Vertical-Slash: scored query rows
    nv: int = 0            # Vertical-Slash: columns kept
    ns: int = 0            # Vertical-Slash: diagonals kept
    ashape: bool = False   # A-shape heads are VS heads with closed-form sets
    pooled: bool = False   # VS heads whose sets come from pooled block scores
    nv_blocks: int = 0     # pooled discovery: key blocks kept
    ns_blocks: int = 0     # pooled discovery: block offsets kept
    block: int = 0         # Block rule: block size
    mode: str = ""         # Block rule: "topk" or "thresh"
    topk: int = 0
    log_alpha: float = 0.0
    force_first: bool = False
    force_diag: bool = False


@dataclass
class Workload:
    name: str
    q: torch.Tensor                 # [B, H, Nq, d] bf16
    k: torch.Tensor                 # [B, Hkv, Nk, d] bf16
    v: torch.Tensor                 # [B, Hkv, Nk, d] bf16
    heads: List[HeadPlan]
    q_offset: int = 0
    extra: Dict[str, object] = field(default_factory=dict)

    @property
    def shape(self):
        B, H, Nq, d = self.q.shape
        return B, H, self.k.shape[1], Nq, self.k.shape[2], d


def _qkv(g, B, H, Hkv, N, d=D, Nq=None):
    Nq = N if Nq is None else Nq
    q = torch.randn(B, H, Nq, d, generator=g)
    k = torch.randn(B, Hkv, N, d, generator=g)
    v = torch.randn(B, Hkv, N, d, generator=g)
    return q, k, v


def _bf(*xs):
    return tuple(x.to(torch.bfloat16).contiguous() for x in xs)


# ---------------------------------------------------------------------------
# Workload 1: one Vertical-Slash head, N = 4096.
# ---------------------------------------------------------------------------
def vs_single(seed: int = 1, N: int = 4096, last_q: int = 64, nv: int = 256, ns: int = 256,
              n_plant: int = 8) -> Workload:
    """Q, K, V ~ N(0,1); `n_plant` key rows at distinct positions in [0, N-last_q)
    are set to 4 x the direction of the mean of the last `last_q` queries."""
    g = _gen(seed)
    q, k, v = _qkv(g, 1, 1, 1, N)
    qb = q.to(torch.bfloat16).float()
    m = qb[0, 0, N - last_q:].mean(0)
    direc = m * (math.sqrt(D) / m.norm())
    pos = _distinct(g, n_plant, 0, max(1, N - last_q))
    k[0, 0, pos] = 4.0 * direc
    q, k, v = _bf(q, k, v)
    plan = [HeadPlan(VS, last_q=last_q, nv=nv, ns=ns)]
    return Workload(f"vs_single_N{N}", q, k, v, plan, extra={"planted_cols": pos})


def vs_multi(seed: int, B: int, H: int, Hkv: int, Nk: int, Nq: Optional[int] = None, last_q: int = 64,
             n_plant: int = 4) -> Workload:
    """Vertical-Slash inputs for several batches and heads, possibly a chunk
    (Nq < Nk, the chunk ends at the last key).  Per (batch, KV head), `n_plant`
    distinct key rows in [0, Nk - last_q) are set to 4 x the direction of the
    mean of the group's last `last_q` queries."""
    Nq = Nk if Nq is None else Nq
    g = _gen(seed)
    q, k, v = _qkv(g, B, H, Hkv, Nk, Nq=Nq)
    qb = q.to(torch.bfloat16).float()
    rep = H // Hkv
    planted = []
    for b in range(B):
        for kvh in range(Hkv):
            m = qb[b, kvh * rep:(kvh + 1) * rep, Nq - last_q:].reshape(-1, D).mean(0)
            pos = _distinct(g, n_plant, 0, max(1, Nk - last_q))
            k[b, kvh, pos] = 4.0 * m * (math.sqrt(D) / m.norm())
            planted.append(pos)
    q, k, v = _bf(q, k, v)
    plan = [HeadPlan(VS, last_q=last_q) for _ in range(H)]
    return Workload(f"vs_multi{seed}", q, k, v, plan, q_offset=Nk - Nq, extra={"planted_cols": planted})


# ---------------------------------------------------------------------------
# Workload 2: block-sparse heads, N = 32768, block 64.
# ---------------------------------------------------------------------------
def block_planted(seed: int = 2, B: int = 1, H: int = 8, N: int = 32768, block: int = 64,
                  n_plant: int = 16, plant_range: Optional[int] = None, mode: str = "topk",
                  topk: int = 16, force: bool = True, Hkv: Optional[int] = None,
                  log_alpha: float = -math.log(20.0)) -> Workload:
    """Per head a direction u_h and `n_plant` distinct key blocks drawn from the
    first `plant_range` blocks; keys in those blocks get +3 u_h and every query
    gets +u_h (causality limits the match to later query blocks)."""
    Hkv = H if Hkv is None else Hkv
    g = _gen(seed)
    q, k, v = _qkv(g, B, H, Hkv, N)
    nb = -(-N // block)
    plant_range = nb if plant_range is None else min(plant_range, nb)
    planted = []
    for b in range(B):
        for h in range(H):
            u = _direction(g)
            blocks = _distinct(g, n_plant, 0, plant_range)
            kvh = h // (H // Hkv)
            for J in blocks.tolist():
                k[b, kvh, J * block:(J + 1) * block] += 3.0 * u
            q[b, h] += u
            planted.append(blocks)
    q, k, v = _bf(q, k, v)
    plan = [HeadPlan(BLOCK, block=block, mode=mode, topk=topk, log_alpha=log_alpha,
                     force_first=force, force_diag=force) for _ in range(H)]
    return Workload(f"block_{mode}_N{N}", q, k, v, plan, extra={"planted_blocks": planted})


def token_planted(seed: int = 6, N: int = 32768, H: int = 8, block: int = 64, n_plant: int = 64,
                  alpha: float = 1.0, budget: int = 1024) -> Workload:
    """Single planted keys for the block-size sweep: per head a direction u_h
    (RMS 1 per element) and `n_plant` distinct key positions whose keys get
    += alpha u_h; every query gets += u_h.  A planted key adds alpha sqrt(d)
    to its token logit; mean pooling over a block of B keys leaves alpha
    sqrt(d) / B of it against pooled noise of about 1 / sqrt(B), a ratio of
    alpha sqrt(d / B).  The data do not depend on `block`; the plan keeps the
    same key budget for every block size: top-(budget / block) blocks plus the
    first and the diagonal block."""
    g = _gen(seed)
    q, k, v = _qkv(g, 1, H, H, N)
    planted = []
    for h in range(H):
        u = _direction(g)
        pos = _distinct(g, n_plant, 0, N)
        k[0, h, pos] += alpha * u
        q[0, h] += u
        planted.append(torch.sort(pos).values)
    q, k, v = _bf(q, k, v)
    plan = [HeadPlan(BLOCK, block=block, mode="topk", topk=max(1, budget // block), force_first=True,
                     force_diag=True) for _ in range(H)]
    return Workload(f"token_planted_N{N}_B{block}", q, k, v, plan,
                    extra={"planted_keys": planted, "alpha": alpha, "budget": budget})


# ---------------------------------------------------------------------------
# Workload 3: mixed per-head patterns, GQA 32/8, N = 131072.
# ---------------------------------------------------------------------------
def mixed_layer(seed: int = 3, N: int = 131072, H: int = 32, Hkv: int = 8, period: int = 4096,
                n_vert: int = 64, last_q: int = 64, sink: int = 128, local: int = 2048,
                nv: int = 1000, ns: int = 4096, block: int = 64, topk: int = 128,
                n_ashape: int = 11, n_vs: int = 16, vs_rule: str = "last_q", nv_blocks: int = 16,
                ns_blocks: int = 32) -> Workload:
    """Periodic slash structure plus planted vertical keys.

    Slash: dims 0-1 of every q and k at position t get a*(cos 2 pi t/P, sin 2 pi t/P)
    with a^2 = 3 sqrt(d), which adds 3 cos(2 pi (i-j)/P) to the logit of (i, j):
    offsets near multiples of P are favoured.  Vertical: per KV head, `n_vert`
    distinct key rows in [0, N - last_q) are set to 4 x the direction of the mean
    of the group's last `last_q` queries (over all its Q heads).  vs_rule
    "pooled" plans the Vertical-Slash heads with sets discovered from the
    pooled block scores (nv_blocks key blocks, ns_blocks block offsets of
    `block`) instead of last_q scoring; the data are the same."""
    g = _gen(seed)
    q, k, v = _qkv(g, 1, H, Hkv, N)
    t = torch.arange(N, dtype=torch.float64)
    a = math.sqrt(3.0 * math.sqrt(D))
    c = (a * torch.cos(2 * math.pi * t / period)).float()
    s = (a * torch.sin(2 * math.pi * t / period)).float()
    q[..., 0] += c
    q[..., 1] += s
    k[..., 0] += c
    k[..., 1] += s
    rep = H // Hkv
    qb = q.to(torch.bfloat16)
    planted = []
    for kvh in range(Hkv):
        m = qb[0, kvh * rep:(kvh + 1) * rep, N - last_q:].float().reshape(-1, D).mean(0)
        direc = m * (math.sqrt(D) / m.norm())
        pos = _distinct(g, n_vert, 0, max(1, N - last_q))
        k[0, kvh, pos] = 4.0 * direc
        planted.append(pos)
    del qb
    q, k, v = _bf(q, k, v)
    plan = []
    for h in range(H):
        if h < n_ashape:
            plan.append(HeadPlan(VS, sink=sink, local=local, ashape=True))
        elif h < n_ashape + n_vs and vs_rule == "pooled":
            plan.append(HeadPlan(VS, pooled=True, block=block, nv_blocks=nv_blocks, ns_blocks=ns_blocks))
        elif h < n_ashape + n_vs:
            plan.append(HeadPlan(VS, last_q=last_q, nv=nv, ns=ns))
        else:
            plan.append(HeadPlan(BLOCK, block=block, mode="topk", topk=topk))
    return Workload(f"mixed_N{N}", q, k, v, plan, extra={"planted_cols": planted})


# ---------------------------------------------------------------------------
# Workload 4: threshold sweep, GQA 32/8, block 128.
# ---------------------------------------------------------------------------
def threshold_sweep(seed: int = 4, N: int = 4096, H: int = 32, Hkv: int = 8, block: int = 128,
                    frac: float = 0.01, log_alpha: float = -math.log(20.0)) -> Workload:
    """Per KV head a direction u_g and max(1, round(frac * N / block)) distinct
    planted key blocks; their keys get +3 u_g and the group's Q heads get +u_g."""
    g = _gen(seed)
    q, k, v = _qkv(g, 1, H, Hkv, N)
    nb = -(-N // block)
    n_plant = max(1, int(round(frac * N / block)))
    rep = H // Hkv
    planted = []
    for kvh in range(Hkv):
        u = _direction(g)
        blocks = _distinct(g, n_plant, 0, nb)
        for J in blocks.tolist():
            k[0, kvh, J * block:(J + 1) * block] += 3.0 * u
        q[0, kvh * rep:(kvh + 1) * rep] += u
        planted.append(blocks)
    q, k, v = _bf(q, k, v)
    plan = [HeadPlan(BLOCK, block=block, mode="thresh", log_alpha=log_alpha) for _ in range(H)]
    return Workload(f"thresh_N{N}", q, k, v, plan, extra={"planted_blocks": planted})


# ---------------------------------------------------------------------------
# Workload 5: indexer-style token top-k on the last query chunk.
# ---------------------------------------------------------------------------
def indexer_chunk(seed: int = 5, N: int = 131072, Nq: int = 8192, Hi: int = 64, di: int = 128,
                  H: int = 16, topk: int = 2048, route_heads: int = 0, cand: int = 0,
                  kv_heads: Optional[int] = None) -> Workload:
    """q_idx [Nq, Hi, di], k_idx [N, di] bf16, w [Nq, Hi] fp32 ~ U(0,1), attention
    Q [1, H, Nq, d] and K, V [1, H, N, d]; everything N(0,1), nothing planted.
    The chunk is the last Nq positions: q_offset = N - Nq.  cand > 0 asks for
    the hierarchical indexer with that many routed candidates per query;
    kv_heads = 1 gives the attention one K/V shared by all heads (MQA)."""
    g = _gen(seed)
    q_idx = torch.randn(Nq, Hi, di, generator=g).to(torch.bfloat16).contiguous()
    k_idx = torch.randn(N, di, generator=g).to(torch.bfloat16).contiguous()
    w = torch.rand(Nq, Hi, generator=g).contiguous()
    q, k, v = _qkv(g, 1, H, H if kv_heads is None else kv_heads, N, Nq=Nq)
    q, k, v = _bf(q, k, v)
    plan = [HeadPlan(TOKEN) for _ in range(H)]
    name = f"indexer_N{N}_r{route_heads}" + (f"_c{cand}" if cand else "") + (f"_kv{kv_heads}" if kv_heads else "")
    return Workload(name, q, k, v, plan, q_offset=N - Nq,
                    extra={"q_idx": q_idx, "k_idx": k_idx, "w": w, "topk": topk,
                           "route_heads": route_heads, "route_block": 64, "cand": cand})


def dense_layer(seed: int = 7, N: int = 32768, H: int = 32, Hkv: int = 8) -> Workload:
    """Q, K, V ~ N(0, 1), every head dense causal: the all-selected special case."""
    g = _gen(seed)
    q, k, v = _bf(*_qkv(g, 1, H, Hkv, N))
    return Workload(f"dense_N{N}", q, k, v, [HeadPlan(DENSE) for _ in range(H)])


def config(c: int, **kw) -> Workload:
    """The five workloads at their stated sizes (keyword arguments shrink them)."""
    if c == 1:
        return vs_single(**kw)
    if c == 2:
        return block_planted(**kw)
    if c == 3:
        return mixed_layer(**kw)
    if c == 4:
        return threshold_sweep(**kw)
    if c == 5:
        return indexer_chunk(**kw)
    raise ValueError(c)


def random_qkv(seed: int, B: int, H: int, Hkv: int, Nk: int, d: int = D, Nq: Optional[int] = None,
               scale: float = 1.0):
    """Plain N(0, scale^2) bf16 tensors for small parity cases."""
    g = _gen(seed)
    q, k, v = _qkv(g, B, H, Hkv, Nk, d, Nq)
    return _bf(q * scale, k * scale, v)

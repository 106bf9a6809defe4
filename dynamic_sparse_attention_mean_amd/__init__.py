"""Python binding of the MI355X dynamic sparse prefill attention library (libdsa.so).

Argument marshalling only: every step of the index build and of the attention
runs in the library's HIP kernels.  PyTorch provides device memory (tensors,
workspaces) and the current HIP stream.  The library must be built
(``python -m dynamic_sparse_attention_mean_amd.build``); nothing here falls back
to another implementation when it is missing.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = 0, 1, 2, 3, 4
DENSE, VS, BLOCK, TOKEN = 0, 1, 2, 3
TOPK, THRESHOLD = 0, 1
OUT_BF16, OUT_F32 = 0, 1
OP_VS, OP_BLOCK, OP_TOKENS, OP_ATTN, OP_TOKENS_HIER, OP_VS_POOLED = 1, 2, 3, 4, 5, 6

EXPORTS = (
    "dsa_status_string", "dsa_last_error", "dsa_workspace_size", "build_index_ashape",
    "build_index_vs", "build_index_vs_pooled", "build_index_block", "build_index_tokens", "build_index_tokens_hier", "sparse_prefill_attn",
    "sparse_prefill_attn_noalloc",
)


class DsaError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q_offset", ctypes.c_int32)]


class _VsIndexC(ctypes.Structure):
    _fields_ = [("cols", ctypes.c_void_p), ("cols_count", ctypes.c_void_p), ("cols_cap", ctypes.c_int32),
                ("diags", ctypes.c_void_p), ("diags_count", ctypes.c_void_p), ("diags_cap", ctypes.c_int32)]


class _BlockIndexC(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("count", ctypes.c_void_p), ("cap", ctypes.c_int32),
                ("block", ctypes.c_int32)]


class _TokenIndexC(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("count", ctypes.c_void_p), ("cap", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m dynamic_sparse_attention_mean_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.dsa_status_string.restype = ctypes.c_char_p
        L.dsa_status_string.argtypes = [I32]
        L.dsa_last_error.restype = ctypes.c_char_p
        L.dsa_last_error.argtypes = []
        L.dsa_workspace_size.restype = I32
        L.dsa_workspace_size.argtypes = [I32, ctypes.POINTER(Shape), P, I32, ctypes.POINTER(SZ)]
        L.build_index_ashape.restype = I32
        L.build_index_ashape.argtypes = [ctypes.POINTER(Shape), P, I32, I32, I32, _VsIndexC, P]
        L.build_index_vs.restype = I32
        L.build_index_vs.argtypes = [ctypes.POINTER(Shape), P, P, P, I32, I32, I32, I32, _VsIndexC, P, P, P, SZ, P]
        L.build_index_vs_pooled.restype = I32
        L.build_index_vs_pooled.argtypes = [ctypes.POINTER(Shape), P, P, P, I32, I32, I32, I32, _VsIndexC, P, P, P,
                                            SZ, P]
        L.build_index_block.restype = I32
        L.build_index_block.argtypes = [ctypes.POINTER(Shape), P, P, P, I32, I32, I32, I32, ctypes.c_float, I32, I32,
                                        _BlockIndexC, P, P, P, P, SZ, P]
        L.build_index_tokens.restype = I32
        L.build_index_tokens.argtypes = [ctypes.POINTER(Shape), P, P, P, I32, I32, I32, I32, _TokenIndexC, P, P, SZ,
                                         P]
        L.build_index_tokens_hier.restype = I32
        L.build_index_tokens_hier.argtypes = [ctypes.POINTER(Shape), P, P, P, I32, I32, I32, I32, I32, _TokenIndexC,
                                              ctypes.POINTER(_TokenIndexC), P, P, SZ, P]
        L.sparse_prefill_attn.restype = I32
        L.sparse_prefill_attn.argtypes = [ctypes.POINTER(Shape), P, P, P, P, ctypes.POINTER(_VsIndexC),
                                          ctypes.POINTER(_BlockIndexC), ctypes.POINTER(_TokenIndexC), I32, P, P, P,
                                          SZ, P]
        L.sparse_prefill_attn_noalloc.restype = I32
        L.sparse_prefill_attn_noalloc.argtypes = [ctypes.POINTER(Shape), P, P, P, P, ctypes.POINTER(_VsIndexC),
                                                  ctypes.POINTER(_BlockIndexC), ctypes.POINTER(_TokenIndexC), I32, P,
                                                  P, P]
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != DSA_OK:
        L = lib()
        raise DsaError(status, where, f"{L.dsa_status_string(status).decode()}: {L.dsa_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must live on {device}")


def make_shape(q: torch.Tensor, k: torch.Tensor, q_offset: Optional[int] = None) -> Shape:
    B, H, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    qo = Nk - Nq if q_offset is None else q_offset
    return Shape(B, H, Hkv, Nq, Nk, d, qo)


def workspace_size(op: int, shape: Shape, params: Sequence[int] = ()) -> int:
    arr = (ctypes.c_int32 * max(1, len(params)))(*params)
    out = ctypes.c_size_t(0)
    _check(lib().dsa_workspace_size(op, ctypes.byref(shape), arr, len(params), ctypes.byref(out)), "dsa_workspace_size")
    return out.value


def _workspace(op, shape, params, device, ws):
    need = workspace_size(op, shape, params)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws


# ---------------------------------------------------------------------------
# Index containers (device tensors)
# ---------------------------------------------------------------------------
@dataclass
class VSIndex:
    cols: torch.Tensor          # [B, H, cols_cap] int32
    cols_count: torch.Tensor    # [B, H] int32
    diags: torch.Tensor         # [B, H, diags_cap] int32
    diags_count: torch.Tensor   # [B, H] int32

    @staticmethod
    def empty(B, H, cols_cap, diags_cap, device):
        z = lambda *s: torch.zeros(*s, dtype=torch.int32, device=device)
        return VSIndex(z(B, H, max(1, cols_cap)), z(B, H), z(B, H, max(1, diags_cap)), z(B, H))

    def c(self):
        return _VsIndexC(self.cols.data_ptr(), self.cols_count.data_ptr(), self.cols.shape[-1],
                         self.diags.data_ptr(), self.diags_count.data_ptr(), self.diags.shape[-1])


@dataclass
class BlockIndex:
    idx: torch.Tensor           # [B, H, nqb, cap] int32
    count: torch.Tensor         # [B, H, nqb] int32
    block: int

    @staticmethod
    def empty(B, H, nqb, cap, block, device):
        return BlockIndex(torch.zeros(B, H, nqb, max(1, cap), dtype=torch.int32, device=device),
                          torch.zeros(B, H, nqb, dtype=torch.int32, device=device), block)

    def c(self):
        return _BlockIndexC(self.idx.data_ptr(), self.count.data_ptr(), self.idx.shape[-1], self.block)


@dataclass
class TokenIndex:
    idx: torch.Tensor           # [B, Nq, cap] int32
    count: torch.Tensor         # [B, Nq] int32

    @staticmethod
    def empty(B, Nq, cap, device):
        return TokenIndex(torch.zeros(B, Nq, max(1, cap), dtype=torch.int32, device=device),
                          torch.zeros(B, Nq, dtype=torch.int32, device=device))

    def c(self):
        return _TokenIndexC(self.idx.data_ptr(), self.count.data_ptr(), self.idx.shape[-1])


def _heads_arr(heads):
    heads = [int(h) for h in heads]
    return (ctypes.c_int32 * len(heads))(*heads), len(heads)


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def build_index_ashape(q, k, heads, sink, local, out: VSIndex):
    shape = make_shape(q, k)
    arr, n = _heads_arr(heads)
    _check(lib().build_index_ashape(ctypes.byref(shape), arr, n, sink, local, out.c(), _stream(q.device)),
           "build_index_ashape")
    return out


def build_index_vs(q, k, heads, last_q, nv, ns, out: VSIndex, v_scores=None, s_scores=None, ws=None):
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, q.device)
    shape = make_shape(q, k)
    arr, n = _heads_arr(heads)
    ws = _workspace(OP_VS, shape, [n, last_q], q.device, ws)
    _check(lib().build_index_vs(ctypes.byref(shape), _ptr(q), _ptr(k), arr, n, last_q, nv, ns, out.c(),
                                _ptr(v_scores), _ptr(s_scores), _ptr(ws), ws.numel(), _stream(q.device)),
           "build_index_vs")
    return out


def build_index_vs_pooled(q, k, heads, block, nv_blocks, ns_blocks, out: VSIndex, v_scores=None, s_scores=None,
                          ws=None):
    """Vertical-Slash sets from the pooled block scores (the library's rule for
    discovering vertical and slash shapes from one block search)."""
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, q.device)
    shape = make_shape(q, k)
    arr, n = _heads_arr(heads)
    ws = _workspace(OP_VS_POOLED, shape, [n, block], q.device, ws)
    _check(lib().build_index_vs_pooled(ctypes.byref(shape), _ptr(q), _ptr(k), arr, n, block, nv_blocks, ns_blocks,
                                       out.c(), _ptr(v_scores), _ptr(s_scores), _ptr(ws), ws.numel(),
                                       _stream(q.device)),
           "build_index_vs_pooled")
    return out


def build_index_block(q, k, heads, block, mode, topk, out: BlockIndex, log_alpha=-math.log(20.0),
                      force_first=False, force_diag=False, qbar=None, kbar=None, scores=None, ws=None):
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, q.device)
    shape = make_shape(q, k)
    arr, n = _heads_arr(heads)
    ws = _workspace(OP_BLOCK, shape, [n, block], q.device, ws)
    _check(lib().build_index_block(ctypes.byref(shape), _ptr(q), _ptr(k), arr, n, block, mode, topk,
                                   float(log_alpha), int(force_first), int(force_diag), out.c(), _ptr(qbar),
                                   _ptr(kbar), _ptr(scores), _ptr(ws), ws.numel(), _stream(q.device)),
           "build_index_block")
    return out


def _indexer_shape(q_idx, k_idx, w):
    """Shape of an indexer call: q_idx [Nq, Hi, d] or [B, Nq, Hi, d], k_idx [Nk, d] or
    [B, Nk, d], w [Nq, Hi] or [B, Nq, Hi] (the sequences of a batch run one after another)."""
    if q_idx.dim() == 3:
        Nq, Hi, di = q_idx.shape
        B = 1
    else:
        B, Nq, Hi, di = q_idx.shape
    Nk = k_idx.shape[-2]
    if k_idx.numel() != B * Nk * di or w.numel() != B * Nq * Hi:
        raise ValueError("q_idx, k_idx and w disagree on the batch or sizes")
    return Shape(B, 1, 1, Nq, Nk, di, Nk - Nq), Hi


def build_index_tokens(q_idx, k_idx, w, topk, out: TokenIndex, route_heads=0, route=None, ws=None, route_block=64):
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(k_idx, "k_idx", torch.bfloat16, q_idx.device)
    _need(w, "w", torch.float32, q_idx.device)
    shape, Hi = _indexer_shape(q_idx, k_idx, w)
    ws = _workspace(OP_TOKENS, shape, [Hi, route_heads, topk], q_idx.device, ws)
    _check(lib().build_index_tokens(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(w), Hi, route_heads,
                                    route_block, topk, out.c(), _ptr(route), _ptr(ws), ws.numel(),
                                    _stream(q_idx.device)),
           "build_index_tokens")
    return out


def build_index_tokens_hier(q_idx, k_idx, w, cand, topk, out: TokenIndex, route_heads=8, cands=None, route=None,
                            ws=None, route_block=64):
    """Hierarchical indexer: routed top-`cand` candidates, rescored by every head, top-`topk` of them."""
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(k_idx, "k_idx", torch.bfloat16, q_idx.device)
    _need(w, "w", torch.float32, q_idx.device)
    shape, Hi = _indexer_shape(q_idx, k_idx, w)
    ws = _workspace(OP_TOKENS_HIER, shape, [Hi, route_heads, cand, topk], q_idx.device, ws)
    cc = cands.c() if cands is not None else None
    _check(lib().build_index_tokens_hier(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(w), Hi, route_heads,
                                         route_block, cand, topk, out.c(),
                                         ctypes.byref(cc) if cc is not None else None, _ptr(route), _ptr(ws),
                                         ws.numel(), _stream(q_idx.device)),
           "build_index_tokens_hier")
    return out


def sparse_prefill_attn(q, k, v, head_kind, vs: Optional[VSIndex] = None, blk: Optional[BlockIndex] = None,
                        tok: Optional[TokenIndex] = None, out_dtype=OUT_F32, o=None, lse=None, ws=None,
                        want_lse=True):
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, q.device)
    _need(v, "v", torch.bfloat16, q.device)
    shape = make_shape(q, k)
    B, H, Nq, d = q.shape
    if o is None:
        o = torch.empty(B, H, Nq, d, dtype=torch.float32 if out_dtype == OUT_F32 else torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(B, H, Nq, dtype=torch.float32, device=q.device)
    kinds = (ctypes.c_int32 * H)(*[int(x) for x in head_kind])
    ws = _workspace(OP_ATTN, shape, [], q.device, ws)
    vsc = vs.c() if vs is not None else None
    bc = blk.c() if blk is not None else None
    tc = tok.c() if tok is not None else None
    _check(lib().sparse_prefill_attn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), kinds,
                                     ctypes.byref(vsc) if vsc is not None else None,
                                     ctypes.byref(bc) if bc is not None else None,
                                     ctypes.byref(tc) if tc is not None else None,
                                     out_dtype, _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(q.device)),
           "sparse_prefill_attn")
    return o, lse


def sparse_prefill_attn_noalloc(q, k, v, head_kind, o, lse=None, vs: Optional[VSIndex] = None,
                                blk: Optional[BlockIndex] = None, tok: Optional[TokenIndex] = None, out_dtype=OUT_F32):
    """sparse_prefill_attn with the library's static scratch instead of a
    workspace: nothing is allocated, the caller passes the outputs (o, and lse
    or None).  Calls that overlap on one device race."""
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, q.device)
    _need(v, "v", torch.bfloat16, q.device)
    _need(o, "o", torch.float32 if out_dtype == OUT_F32 else torch.bfloat16, q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, q.device)
    shape = make_shape(q, k)
    kinds = (ctypes.c_int32 * q.shape[1])(*[int(x) for x in head_kind])
    vsc = vs.c() if vs is not None else None
    bc = blk.c() if blk is not None else None
    tc = tok.c() if tok is not None else None
    _check(lib().sparse_prefill_attn_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), kinds,
                                             ctypes.byref(vsc) if vsc is not None else None,
                                             ctypes.byref(bc) if bc is not None else None,
                                             ctypes.byref(tc) if tc is not None else None,
                                             out_dtype, _ptr(o), _ptr(lse), _stream(q.device)),
           "sparse_prefill_attn_noalloc")
    return o, lse

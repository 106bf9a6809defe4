"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host (before any HIP call), with the documented status codes."""
import ctypes
import os
import re

import pytest

import dynamic_sparse_attention_mean_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dsa.LIB_PATH), reason="libdsa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_and_binding_agree():
    names = declared_functions()
    assert set(names) == set(dsa.EXPORTS), names


def test_every_declared_symbol_is_exported():
    L = dsa.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    nm = os.popen(f"nm -D --defined-only {dsa.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", nm), name


def test_status_strings():
    L = dsa.lib()
    assert L.dsa_status_string(0) == b"ok"
    assert L.dsa_status_string(3).startswith(b"workspace")
    assert L.dsa_status_string(99) == b"unknown status"


def shape(**kw):
    s = dict(batch=1, heads=4, kv_heads=2, q_len=256, kv_len=256, head_dim=128, q_offset=0)
    s.update(kw)
    return dsa.Shape(**s)


def ws_size(op, sh, params):
    arr = (ctypes.c_int32 * max(1, len(params)))(*params)
    out = ctypes.c_size_t(0)
    st = dsa.lib().dsa_workspace_size(op, ctypes.byref(sh), arr, len(params), ctypes.byref(out))
    return st, out.value


def test_workspace_sizes():
    st, n = ws_size(dsa.OP_ATTN, shape(), [])
    assert st == 0 and n > 0
    st, n_vs = ws_size(dsa.OP_VS, shape(), [2, 64])
    assert st == 0 and n_vs >= 2 * 2 * 256 * 4
    st, n_b = ws_size(dsa.OP_BLOCK, shape(), [4, 64])
    assert st == 0 and n_b >= 4 * 4 * 4 * 4
    # sizes depend on shape only and grow with it
    st, big = ws_size(dsa.OP_ATTN, shape(q_len=4096, kv_len=4096), [])
    assert big > n
    assert ws_size(99, shape(), [])[0] == dsa.DSA_ERR_INVALID_ARG
    assert ws_size(dsa.OP_BLOCK, shape(), [4, 48])[0] == dsa.DSA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), dsa.DSA_ERR_UNSUPPORTED),
    (dict(heads=5), dsa.DSA_ERR_INVALID_ARG),
    (dict(q_len=100), dsa.DSA_ERR_INVALID_ARG),
    (dict(batch=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(q_len=0, kv_len=0), dsa.DSA_ERR_INVALID_ARG),      # empty input: rejected, not run
    (dict(q_len=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(kv_heads=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(kv_len=1 << 30, q_len=1 << 30), dsa.DSA_ERR_INVALID_ARG),   # beyond the largest key count
    (dict(q_offset=-1, q_len=257), dsa.DSA_ERR_INVALID_ARG),
    (dict(heads=512, kv_heads=1), dsa.DSA_ERR_UNSUPPORTED),
])
def test_bad_shapes(kw, code):
    assert ws_size(dsa.OP_ATTN, shape(**kw), [])[0] == code


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def vs_c(cap_c=16, cap_d=16, null=False):
    p = 0 if null else 0x2000
    return dsa._VsIndexC(p, p, cap_c, p, p, cap_d)


def test_vs_validation_paths():
    L = dsa.lib()
    heads = (ctypes.c_int32 * 2)(0, 1)
    sh = shape()
    _, need = ws_size(dsa.OP_VS, sh, [2, 64])
    call = lambda **kw: L.build_index_vs(ctypes.byref(kw.get("sh", sh)), kw.get("q", FAKE), FAKE, kw.get("heads", heads),
                                         kw.get("n", 2), kw.get("lq", 64), kw.get("nv", 8), kw.get("ns", 8),
                                         kw.get("out", vs_c()), None, None, kw.get("ws", FAKE),
                                         kw.get("wsb", need), None)
    assert call(q=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(lq=0) == dsa.DSA_ERR_INVALID_ARG
    assert call(lq=65) == dsa.DSA_ERR_INVALID_ARG
    assert call(nv=-1) == dsa.DSA_ERR_INVALID_ARG
    assert call(nv=17) == dsa.DSA_ERR_INVALID_ARG                 # above cols_cap
    assert call(out=vs_c(null=True)) == dsa.DSA_ERR_INVALID_ARG
    assert call(wsb=need - 1) == dsa.DSA_ERR_WORKSPACE
    assert call(ws=None) == dsa.DSA_ERR_WORKSPACE
    bad = (ctypes.c_int32 * 2)(0, 9)
    assert call(heads=bad) == dsa.DSA_ERR_INVALID_ARG
    dup = (ctypes.c_int32 * 2)(1, 1)
    assert call(heads=dup) == dsa.DSA_ERR_INVALID_ARG
    assert call(n=0) == dsa.DSA_ERR_INVALID_ARG
    assert b"workspace" in L.dsa_last_error() or True


def test_vs_pooled_validation_paths():
    L = dsa.lib()
    heads = (ctypes.c_int32 * 1)(1)
    sh = shape()
    _, need = ws_size(dsa.OP_VS_POOLED, sh, [1, 64])

    def call(**kw):
        return L.build_index_vs_pooled(ctypes.byref(kw.get("sh", sh)), FAKE, FAKE, heads, 1, kw.get("block", 64),
                                       kw.get("nv", 2), kw.get("ns", 2), kw.get("out", vs_c(128, 254)), None, None,
                                       kw.get("ws", FAKE), kw.get("wsb", need), None)
    assert call(block=48) == dsa.DSA_ERR_UNSUPPORTED
    assert call(nv=1025) == dsa.DSA_ERR_UNSUPPORTED and call(ns=-1) == dsa.DSA_ERR_UNSUPPORTED
    assert call(out=vs_c(127, 254)) == dsa.DSA_ERR_INVALID_ARG      # two key blocks of 64 need 128 columns
    assert call(out=vs_c(128, 253)) == dsa.DSA_ERR_INVALID_ARG      # two offsets need 2 * 127 diagonals
    assert call(out=vs_c(128, 254, null=True)) == dsa.DSA_ERR_INVALID_ARG
    assert call(wsb=need - 1) == dsa.DSA_ERR_WORKSPACE
    assert call(sh=shape(q_len=200, q_offset=56)) == dsa.DSA_ERR_UNSUPPORTED   # chunk not block-aligned
    # a chunk adds no workspace beyond the whole prompt's (the slash masses have one entry per key block)
    st, need_c = ws_size(dsa.OP_VS_POOLED, shape(q_len=128, q_offset=128), [1, 64])
    assert st == 0 and need_c <= need


def test_block_validation_paths():
    L = dsa.lib()
    heads = (ctypes.c_int32 * 1)(0)
    sh = shape()
    _, need = ws_size(dsa.OP_BLOCK, sh, [1, 64])
    good = dsa._BlockIndexC(0x2000, 0x2000, 4, 64)

    def call(**kw):
        return L.build_index_block(ctypes.byref(kw.get("sh", sh)), FAKE, FAKE, heads, 1, kw.get("block", 64),
                                   kw.get("mode", 0), kw.get("topk", 2), ctypes.c_float(kw.get("la", -3.0)),
                                   kw.get("ff", 1), kw.get("fd", 1), kw.get("out", good), None, None, None,
                                   kw.get("ws", FAKE), kw.get("wsb", need), None)
    assert call(block=48) == dsa.DSA_ERR_UNSUPPORTED
    assert call(mode=7) == dsa.DSA_ERR_INVALID_ARG
    assert call(topk=-1) == dsa.DSA_ERR_INVALID_ARG
    # nqb = 4: top-3 plus two forced blocks needs min(4, 5) = 4 slots
    assert call(topk=3, out=dsa._BlockIndexC(0x2000, 0x2000, 3, 64)) == dsa.DSA_ERR_INVALID_ARG
    assert call(mode=1, la=0.5) == dsa.DSA_ERR_INVALID_ARG
    assert call(out=dsa._BlockIndexC(0x2000, 0x2000, 4, 128)) == dsa.DSA_ERR_INVALID_ARG
    assert call(out=dsa._BlockIndexC(0, 0x2000, 4, 64)) == dsa.DSA_ERR_INVALID_ARG
    assert call(wsb=need - 1) == dsa.DSA_ERR_WORKSPACE
    assert call(sh=shape(q_len=200, q_offset=56)) == dsa.DSA_ERR_UNSUPPORTED   # chunk not block-aligned
    # a chunk at q_offset 128 (two query blocks, absolute 2 and 3): its last block
    # has four candidates, so the threshold rule needs cap >= 4
    assert call(sh=shape(q_len=128, q_offset=128), mode=1,
                out=dsa._BlockIndexC(0x2000, 0x2000, 3, 64)) == dsa.DSA_ERR_INVALID_ARG


def test_attention_validation_paths():
    L = dsa.lib()
    sh = shape()
    _, need = ws_size(dsa.OP_ATTN, sh, [])
    kinds = (ctypes.c_int32 * 4)(0, 1, 2, 0)

    def call(**kw):
        vs = kw.get("vs", vs_c())
        blk = kw.get("blk", dsa._BlockIndexC(0x2000, 0x2000, 4, 64))
        return L.sparse_prefill_attn(ctypes.byref(kw.get("sh", sh)), FAKE, FAKE, kw.get("v", FAKE), kw.get("kinds", kinds),
                                     ctypes.byref(vs) if vs is not None else None,
                                     ctypes.byref(blk) if blk is not None else None, None, kw.get("dt", 1),
                                     FAKE, None, kw.get("ws", FAKE), kw.get("wsb", need), None)
    assert call(v=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(vs=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(blk=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(dt=5) == dsa.DSA_ERR_INVALID_ARG
    assert call(kinds=(ctypes.c_int32 * 4)(0, 1, 2, 7)) == dsa.DSA_ERR_INVALID_ARG
    assert call(kinds=(ctypes.c_int32 * 4)(0, 3, 0, 0)) in (dsa.DSA_ERR_INVALID_ARG, dsa.DSA_ERR_UNSUPPORTED)
    assert call(wsb=need - 1) == dsa.DSA_ERR_WORKSPACE
    assert call(sh=shape(head_dim=96)) == dsa.DSA_ERR_UNSUPPORTED
    assert call(v=ctypes.c_void_p(0x1008)) == dsa.DSA_ERR_INVALID_ARG      # rows need 16-byte alignment
    assert call(sh=shape(q_len=200, q_offset=56)) == dsa.DSA_ERR_UNSUPPORTED   # block heads: chunk not block-aligned


def test_ashape_validation_paths():
    L = dsa.lib()
    heads = (ctypes.c_int32 * 1)(2)
    sh = shape()
    assert L.build_index_ashape(ctypes.byref(sh), heads, 1, -1, 8, vs_c(), None) == dsa.DSA_ERR_INVALID_ARG
    assert L.build_index_ashape(ctypes.byref(sh), heads, 1, 4, 0, vs_c(), None) == dsa.DSA_ERR_INVALID_ARG
    assert L.build_index_ashape(ctypes.byref(sh), heads, 1, 32, 8, vs_c(16, 16), None) == dsa.DSA_ERR_INVALID_ARG
    assert L.build_index_ashape(ctypes.byref(sh), heads, 1, 4, 8, vs_c(null=True), None) == dsa.DSA_ERR_INVALID_ARG


def tok_c(cap, null=False):
    return dsa._TokenIndexC(None if null else FAKE, None if null else FAKE, cap)


def test_tokens_validation_paths():
    """Both indexer entry points reject bad budgets, head counts and index sets
    on the host (the hierarchical one also its candidate count and list)."""
    L = dsa.lib()
    sh = shape(heads=1, kv_heads=1, q_len=64, kv_len=1024, q_offset=960)
    st, need = ws_size(dsa.OP_TOKENS, sh, [64, 8, 100])
    assert st == 0 and need >= 64 * 1024 * 4
    st, need_h = ws_size(dsa.OP_TOKENS_HIER, sh, [64, 8, 400, 100])
    assert st == 0 and need_h >= need + 2 * 64 * 400 * 4
    assert ws_size(dsa.OP_TOKENS_HIER, sh, [64, 0, 400, 100])[0] == dsa.DSA_ERR_INVALID_ARG     # no routing
    assert ws_size(dsa.OP_TOKENS_HIER, sh, [64, 8, 50, 100])[0] == dsa.DSA_ERR_INVALID_ARG      # cand < topk

    def tok(**kw):
        return L.build_index_tokens(ctypes.byref(kw.get("sh", sh)), FAKE, FAKE, FAKE, kw.get("hi", 64),
                                    kw.get("r", 8), kw.get("rb", 64), kw.get("topk", 100), kw.get("out", tok_c(100)),
                                    None, kw.get("ws", FAKE), kw.get("wsb", need), None)

    assert tok(hi=65) == dsa.DSA_ERR_UNSUPPORTED
    assert L.build_index_tokens(ctypes.byref(sh), ctypes.c_void_p(0x1002), FAKE, FAKE, 64, 8, 64, 100, tok_c(100),
                                None, FAKE, need, None) == dsa.DSA_ERR_INVALID_ARG   # q_idx not 16-byte aligned
    assert tok(r=9) == dsa.DSA_ERR_UNSUPPORTED
    assert tok(rb=48) == dsa.DSA_ERR_UNSUPPORTED and tok(rb=256) == dsa.DSA_ERR_UNSUPPORTED
    assert tok(topk=0) == dsa.DSA_ERR_INVALID_ARG
    assert tok(out=tok_c(50)) == dsa.DSA_ERR_INVALID_ARG
    assert tok(out=tok_c(100, null=True)) == dsa.DSA_ERR_INVALID_ARG
    assert tok(wsb=need - 1) == dsa.DSA_ERR_WORKSPACE

    def hier(**kw):
        c = kw.get("cands")
        return L.build_index_tokens_hier(ctypes.byref(sh), FAKE, FAKE, FAKE, kw.get("hi", 64), kw.get("r", 8),
                                         kw.get("rb", 64), kw.get("cand", 400), kw.get("topk", 100),
                                         kw.get("out", tok_c(100)),
                                         ctypes.byref(c) if c is not None else None, None, FAKE,
                                         kw.get("wsb", need_h), None)

    assert hier(r=0) == dsa.DSA_ERR_INVALID_ARG
    assert hier(r=9, hi=64) == dsa.DSA_ERR_UNSUPPORTED
    assert hier(rb=0) == dsa.DSA_ERR_UNSUPPORTED
    assert hier(cand=99) == dsa.DSA_ERR_INVALID_ARG
    assert hier(cand=65537, topk=100) == dsa.DSA_ERR_INVALID_ARG
    assert hier(topk=4097, cand=5000, out=tok_c(4097)) == dsa.DSA_ERR_UNSUPPORTED
    assert hier(out=tok_c(99)) == dsa.DSA_ERR_INVALID_ARG
    assert hier(cands=tok_c(399)) == dsa.DSA_ERR_INVALID_ARG
    assert hier(cands=tok_c(400, null=True)) == dsa.DSA_ERR_INVALID_ARG
    assert hier(wsb=need_h - 1) == dsa.DSA_ERR_WORKSPACE


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU and says so for --gpus above 1 (before any GPU work)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr

"""The attention entry point that allocates nothing (sparse_prefill_attn_noalloc)
against the workspace entry point (sparse_prefill_attn) through the C ABI: two
calls in a row on one device, the second with a smaller input, each bit-equal
to the workspace call on the same inputs and index sets."""
import numpy as np
import pytest
import torch

import synth
import dynamic_sparse_attention_mean_amd as dsa

from parity import oracle_head_sets, upload_sets

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def mixed(N, seed, H=8, Hkv=2):
    return synth.mixed_layer(seed=seed, N=N, H=H, Hkv=Hkv, period=256, n_vert=8, last_q=64, sink=32, local=200,
                             nv=40, ns=160, block=64, topk=6, n_ashape=3, n_vs=3)


def run_both(w, out_dtype):
    B, H, Hkv, Nq, Nk, d = w.shape
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    sets = {(0, h): oracle_head_sets(w, 0, h) for h in range(H)}
    kinds, vsi, bi = upload_sets(w, sets, DEV)
    odt = torch.float32 if out_dtype == dsa.OUT_F32 else torch.bfloat16
    o_ref, l_ref = dsa.sparse_prefill_attn(q, k, v, kinds, vs=vsi, blk=bi, out_dtype=out_dtype)
    o = torch.full((B, H, Nq, d), float("nan"), dtype=odt, device=DEV)
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=DEV)
    dsa.sparse_prefill_attn_noalloc(q, k, v, kinds, o, lse, vs=vsi, blk=bi, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, lse, o_ref, l_ref


def test_noalloc_matches_workspace_entry_point_twice():
    # first a larger call (dirties the static scratch: bitmaps, counters), then a smaller one
    for N, seed, odt in ((4096 + 37, 11, dsa.OUT_F32), (1000, 12, dsa.OUT_BF16)):
        o, lse, o_ref, l_ref = run_both(mixed(N, seed), odt)
        assert not torch.isnan(o.float()).any() and not torch.isnan(lse).any(), f"N={N}: outputs not written"
        assert torch.equal(o, o_ref), f"N={N}: output differs from sparse_prefill_attn"
        assert torch.equal(lse, l_ref), f"N={N}: LSE differs from sparse_prefill_attn"


def test_noalloc_rejects_shapes_beyond_its_scratch():
    # B * H * Nk / 2 bytes of scratch: 4 x 128 heads at 2^20 keys needs ~256 MiB > 32 MiB
    B, H, Hkv, Nk = 4, 128, 8, 1 << 20
    shape = dsa.Shape(B, H, Hkv, Nk, Nk, 128, 0)
    kinds = (dsa.ctypes.c_int32 * H)(*([dsa.DENSE] * H))
    fake = dsa.ctypes.c_void_p(1 << 12)      # aligned, never dereferenced: the size check comes first
    st = dsa.lib().sparse_prefill_attn_noalloc(dsa.ctypes.byref(shape), fake, fake, fake, kinds, None, None, None,
                                               dsa.OUT_F32, fake, None, None)
    assert st == dsa.DSA_ERR_UNSUPPORTED
    assert b"static buffer" in dsa.lib().dsa_last_error()

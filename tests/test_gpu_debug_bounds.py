"""The debug-bounds build (libfsa_debug.so, -DFSA_DEBUG_BOUNDS) against the
release library: on inputs the kernels skip (block-list entries outside
[0, i], decode indices past the sequence, bad page ids, unsorted segments) it
raises the documented FSA_DBG_* bits and still returns exactly the release
library's results; on clean inputs it raises nothing; the release library
reports FSA_DBG_UNAVAILABLE only.  Every call goes through the C ABI of the
library under test (the binding's library handle is swapped for the test)."""

import ctypes
import os

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    from free_sparse_attention_head_amd import _lib
    rel = _lib.load()
    path = os.path.join(_lib.PKG, "libfsa_debug.so")
    if not os.path.exists(path):
        from free_sparse_attention_head_amd import build
        build.build(debug_bounds=True)
    dbg = ctypes.CDLL(path)
    for name, (res, args) in _lib.SIGNATURES.items():
        fn = getattr(dbg, name)
        fn.restype, fn.argtypes = res, args
    return _lib, rel, dbg


def _flags(lib, clear=1):
    f = ctypes.c_uint32(0)
    torch.cuda.synchronize()
    assert lib.fsa_debug_flags(ctypes.byref(f), clear) == 0
    return f.value


def _with(L, lib, fn):
    """Run fn with the binding routed through lib."""
    saved = L._lib
    L._lib = lib
    try:
        out = fn()
        torch.cuda.synchronize()
        return out
    finally:
        L._lib = saved


def test_release_library_reports_unavailable(libs):
    L, rel, dbg = libs
    assert _flags(rel) == L.FSA_DBG_UNAVAILABLE
    _flags(dbg)
    assert _flags(dbg) == 0


def test_prefill_bad_block_entries_flagged_and_skipped(libs):
    L, rel, dbg = libs
    import free_sparse_attention_head_amd as fsa
    B, S, H, D, T = 1, 512, 2, 128, 64
    nB = S // T
    print(f"[debug-bounds prefill] S={S} H={H} D={D} T={T}", flush=True)
    inp = workloads.prefill_inputs(B, S, H, H, D, T, model="iid", n_spikes=0, seed=9, device="cuda")
    q, k, v = inp["q"], inp["k"], inp["v"]
    bidx = torch.zeros((B, H, nB, nB), dtype=torch.int32)
    bcnt = torch.zeros((B, H, nB), dtype=torch.int32)
    for i in range(nB):
        bidx[0, :, i, :2] = torch.tensor([0, i], dtype=torch.int32)
        bcnt[0, :, i] = 2 if i else 1
    clean = (bidx.cuda(), bcnt.cuda())
    _flags(dbg)
    o_d, l_d = _with(L, dbg, lambda: fsa.sparse_prefill_attn(q, k, v, T, *clean))
    assert _flags(dbg) == 0
    bad_idx = bidx.clone()
    bad_idx[0, 1, 3, 2] = 7          # a block after the diagonal of row 3
    bad_idx[0, 0, 5, 2] = -4
    bad_cnt = bcnt.clone()
    bad_cnt[0, 1, 3] = 3
    bad_cnt[0, 0, 5] = 3
    bad = (bad_idx.cuda(), bad_cnt.cuda())
    o_r, l_r = fsa.sparse_prefill_attn(q, k, v, T, *bad)
    o_b, l_b = _with(L, dbg, lambda: fsa.sparse_prefill_attn(q, k, v, T, *bad))
    assert _flags(dbg) == L.FSA_DBG_BLOCK_INDEX
    assert torch.equal(o_b, o_r) and torch.equal(l_b, l_r)
    assert torch.equal(o_b, o_d) and torch.equal(l_b, l_d)   # the skipped entries change nothing
    # fp32 inputs run the other prefill kernel
    qf, kf, vf = q.float(), k.float(), v.float()
    _with(L, dbg, lambda: fsa.sparse_prefill_attn(qf, kf, vf, T, *bad))
    assert _flags(dbg) == L.FSA_DBG_BLOCK_INDEX


def test_decode_bad_indices_pages_and_segments_flagged(libs):
    L, rel, dbg = libs
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, k = 2, 4096, 8, 2, 128, 64
    print(f"[debug-bounds decode] B={B} N={N} Hq={Hq} Hkv={Hkv} k={k}", flush=True)
    d = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=1, seq_lens=[4096, 3000], seed=12,
                                device="cuda")
    Lr, pt, sl = d["layers"][0], d["page_table"], d["seq_lens"]
    args = (Lr["q"], Lr["k"], Lr["v"], pt, sl)
    idx, _ = fsa.topk_indices(Lr["q"], Lr["k"], pt, sl, k)
    _flags(dbg)
    _with(L, dbg, lambda: fsa.topk_indices(Lr["q"], Lr["k"], pt, sl, k))
    _with(L, dbg, lambda: fsa.sparse_decode_attn(*args, mode=fsa.SEL_INDEX, idx=idx))
    assert _flags(dbg) == 0
    # -1 marks an empty slot: not flagged
    empty = idx.clone()
    empty[0, 0, -5:] = -1
    _with(L, dbg, lambda: fsa.sparse_decode_attn(*args, mode=fsa.SEL_INDEX, idx=empty))
    assert _flags(dbg) == 0
    # an index past sequence 1's 3000 tokens and one below -1
    badi = idx.clone()
    badi[1, 2, 0] = 3500
    badi[0, 3, 1] = -7
    o_r, l_r = fsa.sparse_decode_attn(*args, mode=fsa.SEL_INDEX, idx=badi)
    o_b, l_b = _with(L, dbg, lambda: fsa.sparse_decode_attn(*args, mode=fsa.SEL_INDEX, idx=badi))
    assert _flags(dbg) == L.FSA_DBG_TOKEN_INDEX
    assert torch.equal(o_b, o_r) and torch.equal(l_b, l_r)
    # a bad page id inside sequence 0 (decode reads it, top-k scores it)
    badpt = pt.clone()
    badpt[0, 10] = -3
    badpt[0, 11] = d["num_pages"] + 5
    a2 = (Lr["q"], Lr["k"], Lr["v"], badpt, sl)
    o_r, _ = fsa.sparse_decode_attn(*a2, mode=fsa.SEL_ALL)
    o_b, _ = _with(L, dbg, lambda: fsa.sparse_decode_attn(*a2, mode=fsa.SEL_ALL))
    assert _flags(dbg) == L.FSA_DBG_PAGE_ID
    assert torch.equal(o_b, o_r)
    _with(L, dbg, lambda: fsa.topk_indices(Lr["q"], Lr["k"], badpt, sl, k))
    assert _flags(dbg) == L.FSA_DBG_PAGE_ID
    # segments out of order, and a count beyond max_seg
    segs = torch.tensor([[[2000, 2100], [100, 200]], [[0, 64], [128, 256]]], dtype=torch.int32,
                        device="cuda")
    nseg = torch.tensor([2, 2], dtype=torch.int32, device="cuda")
    _with(L, dbg, lambda: fsa.sparse_decode_attn(*args, mode=fsa.SEL_SEGMENT, segments=segs,
                                                 n_seg=nseg))
    assert _flags(dbg) == L.FSA_DBG_SEGMENT
    good = torch.tensor([[[100, 200], [2000, 2100]], [[0, 64], [128, 256]]], dtype=torch.int32,
                        device="cuda")
    _with(L, dbg, lambda: fsa.sparse_decode_attn(*args, mode=fsa.SEL_SEGMENT, segments=good,
                                                 n_seg=nseg))
    assert _flags(dbg) == 0
    _with(L, dbg, lambda: fsa.sparse_decode_attn(*args, mode=fsa.SEL_SEGMENT, segments=good,
                                                 n_seg=torch.tensor([3, 1], dtype=torch.int32,
                                                                    device="cuda")))
    assert _flags(dbg) == L.FSA_DBG_SEGMENT

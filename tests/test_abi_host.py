"""Host-side checks of the C ABI (CPU only: no kernel is launched).

* libfsa.so loads and exports every function declared in include/fsa.h;
* host validation returns the documented status codes before any device
  work (so these calls are safe without a GPU);
* the host segment builder agrees with the oracle's builder and with the
  block-alignment facts.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from free_sparse_attention_head_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        from free_sparse_attention_head_amd import build
        build.build()
    return L, L.load()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "fsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "return")))


def test_library_exports_every_declared_symbol():
    L, lib = _lib()
    names = _declared_functions()
    for required in ("block_stats", "select_blocks", "sparse_prefill_attn", "topk_indices",
                     "sparse_decode_attn", "fsa_workspace_size", "fsa_build_segments",
                     "fsa_build_segments_nb", "fsa_status_string", "fsa_device_check"):
        assert required in names
    for n in names:
        assert hasattr(lib, n), f"libfsa.so does not export {n}"
        assert n in L.SIGNATURES, f"binding lacks a signature for {n}"


def test_status_strings():
    L, lib = _lib()
    for code in range(0, -8, -1):
        assert lib.fsa_status_string(code)
    assert lib.fsa_status_string(-99) == b"unknown status"


def _shape(L, **kw):
    d = dict(B=1, S=1024, Hq=2, Hkv=2, D=64, T=64)
    d.update(kw)
    return L.PrefillShape(*[d[k] for k in ("B", "S", "Hq", "Hkv", "D", "T")])


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), -2), (dict(T=32), -2), (dict(S=1000), -2), (dict(Hq=3, Hkv=2), -2),
    (dict(B=0), -2), (dict(S=64 * 5000), -2), (dict(Hq=2048, Hkv=2), -2),
    (dict(B=600, S=262144, Hq=1024, Hkv=1), -2)])
def test_prefill_shape_validation(kw, code):
    L, lib = _lib()
    s = _shape(L, **kw)
    rc = lib.block_stats(L.FSA_BF16, FAKE, ctypes.byref(s), FAKE, FAKE, None)
    assert rc == code
    rc = lib.sparse_prefill_attn(L.FSA_BF16, FAKE, FAKE, FAKE, ctypes.byref(s), None, None,
                                 0.125, FAKE, None, None, 0, None)
    assert rc == code


def test_prefill_null_and_dtype_validation():
    L, lib = _lib()
    s = _shape(L)
    assert lib.block_stats(L.FSA_BF16, None, ctypes.byref(s), FAKE, FAKE, None) == L.FSA_ERR_NULL
    assert lib.block_stats(7, FAKE, ctypes.byref(s), FAKE, FAKE, None) == L.FSA_ERR_DTYPE
    assert lib.block_stats(L.FSA_BF16, FAKE, None, FAKE, FAKE, None) == L.FSA_ERR_NULL
    # block_idx without block_cnt
    assert lib.sparse_prefill_attn(L.FSA_BF16, FAKE, FAKE, FAKE, ctypes.byref(s), FAKE, None,
                                   0.125, FAKE, None, None, 0, None) == L.FSA_ERR_NULL
    assert lib.sparse_prefill_attn(L.FSA_BF16, FAKE, FAKE, FAKE, ctypes.byref(s), None, None,
                                   float("inf"), FAKE, None, None, 0, None) == L.FSA_ERR_ARG


def test_select_validation_and_workspace():
    L, lib = _lib()
    s = _shape(L)
    ws = lib.fsa_workspace_size(L.FSA_OP_SELECT_BLOCKS, ctypes.byref(s), None)
    nB = 1024 // 64
    assert ws >= 2 * nB * 64 * 4 + 2 * nB * nB * 4
    p = L.SelectParams(0.25, 0.1, 0, 0)
    args = lambda wsb, pp=p: (L.FSA_F32, FAKE, FAKE, FAKE, ctypes.byref(s), ctypes.byref(pp),
                              FAKE, FAKE, FAKE, None, None, FAKE, wsb, None)
    assert lib.select_blocks(*args(ws - 1)) == L.FSA_ERR_WORKSPACE
    bad = L.SelectParams(float("nan"), 0.1, 0, 0)
    assert lib.select_blocks(*args(ws, bad)) == L.FSA_ERR_ARG
    neg = L.SelectParams(0.25, 0.1, -1, 0)
    assert lib.select_blocks(*args(ws, neg)) == L.FSA_ERR_ARG
    assert lib.fsa_workspace_size(L.FSA_OP_PREFILL_ATTN, ctypes.byref(s), None) == 0
    assert lib.fsa_workspace_size(99, ctypes.byref(s), None) == 0


def test_misaligned_pointers_are_rejected():
    """Data tensors and workspaces off a 16-byte boundary, and index arrays off
    a 4-byte one, come back as FSA_ERR_ARG before anything is launched."""
    L, lib = _lib()
    OFF16 = ctypes.c_void_p(0x1004)  # 4-byte aligned, not 16
    OFF4 = ctypes.c_void_p(0x1002)
    s = _shape(L)
    assert lib.block_stats(L.FSA_BF16, OFF16, ctypes.byref(s), FAKE, FAKE, None) == L.FSA_ERR_ARG
    assert lib.block_stats(L.FSA_BF16, FAKE, ctypes.byref(s), FAKE, OFF16, None) == L.FSA_ERR_ARG
    ws = lib.fsa_workspace_size(L.FSA_OP_SELECT_BLOCKS, ctypes.byref(s), None)
    p = L.SelectParams(0.25, 0.1, 0, 0)
    sel_args = dict(q=FAKE, c=FAKE, r=FAKE, m=FAKE, bi=FAKE, bc=FAKE, sc=None, ws=FAKE)
    for key, val in (("q", OFF16), ("c", OFF16), ("sc", OFF16), ("ws", OFF16), ("bi", OFF4)):
        a = dict(sel_args, **{key: val})
        assert lib.select_blocks(L.FSA_F32, a["q"], a["c"], a["r"], ctypes.byref(s),
                                 ctypes.byref(p), a["m"], a["bi"], a["bc"], a["sc"], None,
                                 a["ws"], ws, None) == L.FSA_ERR_ARG, key
    for q, k, v, out in ((OFF16, FAKE, FAKE, FAKE), (FAKE, FAKE, OFF16, FAKE),
                         (FAKE, FAKE, FAKE, OFF16)):
        assert lib.sparse_prefill_attn(L.FSA_BF16, q, k, v, ctypes.byref(s), None, None, 0.125,
                                       out, None, None, 0, None) == L.FSA_ERR_ARG
    assert lib.sparse_prefill_attn(L.FSA_BF16, FAKE, FAKE, FAKE, ctypes.byref(s), OFF4, FAKE,
                                   0.125, FAKE, None, None, 0, None) == L.FSA_ERR_ARG
    ds = _dshape(L)
    k = ctypes.c_int(16)
    tws = lib.fsa_workspace_size(L.FSA_OP_TOPK, ctypes.byref(ds), ctypes.byref(k))
    for q, kp, pt, ws_ in ((OFF16, FAKE, FAKE, FAKE), (FAKE, OFF16, FAKE, FAKE),
                           (FAKE, FAKE, OFF4, FAKE), (FAKE, FAKE, FAKE, OFF16)):
        assert lib.topk_indices(L.FSA_BF16, q, kp, pt, FAKE, ctypes.byref(ds), 16, FAKE, None,
                                ws_, tws, None) == L.FSA_ERR_ARG
    sel = L.KvSelect(L.FSA_SEL_INDEX, FAKE.value, 16, None, None, 0, 0)
    for q, kp, vp, out in ((OFF16, FAKE, FAKE, FAKE), (FAKE, FAKE, OFF16, FAKE),
                           (FAKE, FAKE, FAKE, OFF16)):
        assert lib.sparse_decode_attn(L.FSA_BF16, q, kp, vp, FAKE, FAKE, ctypes.byref(ds),
                                      ctypes.byref(sel), 0.1, out, None, FAKE, 1 << 30,
                                      None) == L.FSA_ERR_ARG
        assert lib.sparse_decode_attn_noalloc(L.FSA_BF16, q, kp, vp, FAKE, FAKE, ctypes.byref(ds),
                                              ctypes.byref(sel), 0.1, out, None,
                                              None) == L.FSA_ERR_ARG
    bad_idx = L.KvSelect(L.FSA_SEL_INDEX, OFF4.value, 16, None, None, 0, 0)
    assert lib.sparse_decode_attn(L.FSA_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(ds),
                                  ctypes.byref(bad_idx), 0.1, FAKE, None, FAKE, 1 << 30,
                                  None) == L.FSA_ERR_ARG
    assert lib.topk_union_kv(OFF4, 2, 8, 2, 16, FAKE, None, None) == L.FSA_ERR_ARG


def _dshape(L, **kw):
    d = dict(B=2, Hq=8, Hkv=2, D=128, page_size=16, num_pages=64, max_pages=32, max_seq_len=512)
    d.update(kw)
    return L.DecodeShape(*[d[k] for k in ("B", "Hq", "Hkv", "D", "page_size", "num_pages",
                                          "max_pages", "max_seq_len")])


@pytest.mark.parametrize("kw", [dict(page_size=32), dict(Hq=6, Hkv=4), dict(Hq=32, Hkv=2),
                                dict(D=80), dict(max_seq_len=16 * 32 + 1), dict(B=0),
                                dict(num_pages=1 << 27, Hq=16, Hkv=2)])
def test_decode_shape_validation(kw):
    L, lib = _lib()
    s = _dshape(L, **kw)
    rc = lib.topk_indices(L.FSA_BF16, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s), 8, FAKE, None,
                          FAKE, 1 << 30, None)
    assert rc == L.FSA_ERR_SHAPE


def test_topk_and_decode_argument_validation():
    L, lib = _lib()
    s = _dshape(L)
    k = ctypes.c_int(16)
    ws = lib.fsa_workspace_size(L.FSA_OP_TOPK, ctypes.byref(s), ctypes.byref(k))
    assert ws >= 2 * 8 * 512 * 4
    call = lambda dt, kk, wsb: lib.topk_indices(dt, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s), kk,
                                                FAKE, None, FAKE, wsb, None)
    assert call(L.FSA_F32, 16, ws) == L.FSA_ERR_DTYPE
    assert call(L.FSA_BF16, 0, ws) == L.FSA_ERR_ARG
    assert call(L.FSA_BF16, 513, ws) == L.FSA_ERR_ARG
    assert call(L.FSA_BF16, 16, ws - 1) == L.FSA_ERR_WORKSPACE

    sel = L.KvSelect(L.FSA_SEL_INDEX, None, 16, None, None, 0, 0)
    dcall = lambda sl, wsb=1 << 30, dt=L.FSA_BF16: lib.sparse_decode_attn(
        dt, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s), ctypes.byref(sl), 0.1, FAKE, None,
        FAKE, wsb, None)
    assert dcall(sel) == L.FSA_ERR_NULL                      # index mode without idx
    sel = L.KvSelect(L.FSA_SEL_INDEX_KV, None, 16, None, None, 0, 0)
    assert dcall(sel) == L.FSA_ERR_NULL                      # per-KV-head mode without idx
    sel = L.KvSelect(L.FSA_SEL_INDEX_KV, FAKE.value, 0, None, None, 0, 0)
    assert dcall(sel) == L.FSA_ERR_ARG                       # k = 0
    sel = L.KvSelect(L.FSA_SEL_INDEX_KV, FAKE.value, 16, None, None, 0, 2)
    assert lib.fsa_workspace_size(L.FSA_OP_DECODE_ATTN, ctypes.byref(s),
                                  ctypes.byref(sel)) == 2 * 8 * 2 * (128 + 2) * 4
    kcall = lambda dt, kk, wsb: lib.topk_indices_kv(dt, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s),
                                                    kk, FAKE, None, FAKE, wsb, None)
    assert kcall(L.FSA_F32, 16, ws) == L.FSA_ERR_DTYPE
    assert kcall(L.FSA_BF16, 0, ws) == L.FSA_ERR_ARG
    assert kcall(L.FSA_BF16, 16, ws - 1) == L.FSA_ERR_WORKSPACE
    # top-k supports sequences of up to 2^23 tokens (its select kernel keeps the
    # lengths of every tile's candidate list in LDS)
    big = _dshape(L, max_pages=(1 << 19) + 1, num_pages=64, max_seq_len=(1 << 23) + 16)
    assert lib.topk_indices(L.FSA_BF16, FAKE, FAKE, FAKE, FAKE, ctypes.byref(big), 16, FAKE,
                            None, FAKE, 1 << 62, None) == L.FSA_ERR_SHAPE
    assert lib.topk_indices_kv(L.FSA_BF16, FAKE, FAKE, FAKE, FAKE, ctypes.byref(big), 16, FAKE,
                               None, FAKE, 1 << 62, None) == L.FSA_ERR_SHAPE
    sel = L.KvSelect(L.FSA_SEL_SEGMENT, None, 0, FAKE.value, FAKE.value, 0, 0)
    assert dcall(sel) == L.FSA_ERR_ARG                       # max_seg 0
    sel = L.KvSelect(9, None, 0, None, None, 0, 0)
    assert dcall(sel) == L.FSA_ERR_ARG                       # unknown mode
    sel = L.KvSelect(L.FSA_SEL_ALL, None, 0, None, None, 0, -1)
    assert dcall(sel) == L.FSA_ERR_ARG                       # negative split
    sel = L.KvSelect(L.FSA_SEL_ALL, None, 0, None, None, 0, 4)
    assert dcall(sel, dt=L.FSA_F32) == L.FSA_ERR_DTYPE
    need = lib.fsa_workspace_size(L.FSA_OP_DECODE_ATTN, ctypes.byref(s), ctypes.byref(sel))
    assert need == 2 * 8 * 4 * (128 + 2) * 4
    assert dcall(sel, wsb=need - 1) == L.FSA_ERR_WORKSPACE


SEG_CASES = [(oracle.SEG_GLOBAL, 1 << 20, 0), (oracle.SEG_LOCAL, 1 << 20, 0),
             (oracle.SEG_LOCAL, 1000, 0), (oracle.SEG_LOCAL, 3000, 0),
             (oracle.SEG_STREAMING, 1 << 20, 0), (oracle.SEG_STREAMING, 600, 0),
             (oracle.SEG_STREAMING, 3, 0)] + \
            [(oracle.SEG_FOCUS, 1 << 20, s) for s in (0, 1, 15, 16, 100003, (1 << 20) - 2048,
                                                        (1 << 20) - 3000)] + \
            [(oracle.SEG_FOCUS, 5000, s) for s in (0, 2000, 2950, 3100)]


@pytest.mark.parametrize("mode,n,start", SEG_CASES)
def test_build_segments_matches_oracle(mode, n, start):
    import free_sparse_attention_head_amd as fsa
    got = fsa.build_segments(mode, n, chunk_start=start, chunk_len=2048, local_len=1024,
                             n_sink=4, page=16)
    want = oracle.build_segments(mode, n, start, 2048, 1024, 4, 16)
    assert got == [tuple(int(x) for x in r) for r in want]


@pytest.mark.parametrize("n,start,m", [(1 << 20, 100003, 0), (1 << 20, 100003, 1),
                                       (1 << 20, 100003, 4096), (1 << 20, 5, 70),
                                       (1 << 20, (1 << 20) - 2100, 100), (5000, 2000, 3000),
                                       (5000, 0, 1 << 20)])
def test_build_segments_neighbourhood_matches_oracle(n, start, m):
    import free_sparse_attention_head_amd as fsa
    for mode in (oracle.SEG_GLOBAL, oracle.SEG_FOCUS, oracle.SEG_LOCAL, oracle.SEG_STREAMING):
        got = fsa.build_segments(mode, n, chunk_start=start, chunk_len=2048, local_len=1024,
                                 n_sink=4, page=16, min_neighbourhood=m)
        want = oracle.build_segments(mode, n, start, 2048, 1024, 4, 16, min_nb=m)
        assert got == [tuple(int(x) for x in r) for r in want]


def test_build_segments_errors():
    L, lib = _lib()
    buf = (ctypes.c_int32 * 4)()
    cnt = ctypes.c_int(0)
    assert lib.fsa_build_segments(7, 100, 0, 10, 10, 0, 16, buf, ctypes.byref(cnt)) == L.FSA_ERR_ARG
    assert lib.fsa_build_segments(0, 100, 0, 10, 10, 0, 0, buf, ctypes.byref(cnt)) == L.FSA_ERR_ARG
    assert lib.fsa_build_segments(0, 100, 0, 10, 10, 0, 16, None, ctypes.byref(cnt)) == L.FSA_ERR_NULL
    assert lib.fsa_build_segments_nb(1, 100, 0, 10, 10, 0, 16, -1, buf, ctypes.byref(cnt)) == L.FSA_ERR_ARG


def test_missing_device_is_reported_not_crashed():
    """With no GPU visible, the device probe and a fully valid call both return
    FSA_ERR_NO_DEVICE (validation passes, nothing is launched)."""
    import torch
    if torch.cuda.device_count() != 0:
        pytest.skip("a GPU is visible: this checks the no-device path only")
    L, lib = _lib()
    assert lib.fsa_device_check() == L.FSA_ERR_NO_DEVICE
    s = _shape(L)
    rc = lib.block_stats(L.FSA_BF16, FAKE, ctypes.byref(s), FAKE, FAKE, None)
    assert rc == L.FSA_ERR_NO_DEVICE


def test_prefill_scale_must_be_positive():
    """The kernels order scores by their unscaled values, which agrees with
    the scaled order only for scale > 0."""
    L, lib = _lib()
    s = _shape(L)
    for bad in (0.0, -0.125, float("nan")):
        assert lib.sparse_prefill_attn(L.FSA_BF16, FAKE, FAKE, FAKE, ctypes.byref(s), None, None,
                                       bad, FAKE, None, None, 0, None) == L.FSA_ERR_ARG


def test_noalloc_entry_point_validation():
    """sparse_decode_attn_noalloc: the checks of sparse_decode_attn, and split
    partials beyond its 16 MiB array are refused before any device work."""
    L, lib = _lib()
    s = _dshape(L, B=2, Hq=32, Hkv=8)
    call = lambda sel, dt=L.FSA_BF16: lib.sparse_decode_attn_noalloc(
        dt, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s), ctypes.byref(sel), 0.1, FAKE, None,
        None)
    big = L.KvSelect(L.FSA_SEL_ALL, None, 0, None, None, 0, 1024)   # 34 MB of partials
    assert call(big) == L.FSA_ERR_WORKSPACE
    assert call(L.KvSelect(L.FSA_SEL_INDEX, None, 16, None, None, 0, 0)) == L.FSA_ERR_NULL
    assert call(L.KvSelect(L.FSA_SEL_ALL, None, 0, None, None, 0, 2), dt=L.FSA_F32) == L.FSA_ERR_DTYPE
    assert L.FSA_NOALLOC_SCRATCH_BYTES == 16 << 20


def test_binding_rejects_mismatched_tensors():
    """The Python binding checks dtypes and shapes against each other before
    any pointer reaches the library (CPU tensors: every rejection happens
    before the device is touched)."""
    import torch
    import free_sparse_attention_head_amd as fsa
    B, S, Hq, Hkv, D, T = 1, 256, 4, 2, 64, 64
    nB = S // T
    q = torch.zeros((B, S, Hq, D), dtype=torch.float32)
    k = torch.zeros((B, S, Hkv, D), dtype=torch.bfloat16)
    v = torch.zeros((B, S, Hkv, D), dtype=torch.bfloat16)
    bidx = torch.zeros((B, Hq, nB, nB), dtype=torch.int32)
    bcnt = torch.zeros((B, Hq, nB), dtype=torch.int32)

    def rejects(fn, what):
        with pytest.raises(ValueError, match=what):
            fn()

    rejects(lambda: fsa.sparse_prefill_attn(q, k, v, T), "dtype")            # fp32 q, bf16 k/v
    qb = q.to(torch.bfloat16)
    rejects(lambda: fsa.sparse_prefill_attn(qb, k, v[:, :128], T), "shape")  # short v
    rejects(lambda: fsa.sparse_prefill_attn(qb, k[:, :128], v[:, :128], T), "k must be")
    rejects(lambda: fsa.sparse_prefill_attn(qb, k, v, T, bidx[:, :, :2], bcnt), "block_idx")
    rejects(lambda: fsa.sparse_prefill_attn(qb, k, v, T, bidx.long(), bcnt), "block_idx")
    rejects(lambda: fsa.sparse_prefill_attn(qb, k, v, T, bidx, None), "together")
    rejects(lambda: fsa.sparse_prefill_attn(qb, k, v, 100), "multiple")
    c = torch.zeros((B, Hkv, nB, D), dtype=torch.float32)
    r = torch.zeros((B, Hkv, nB), dtype=torch.float32)
    rejects(lambda: fsa.select_blocks(qb, c.double(), r, T, 0.1, 0.04), "centroid")
    rejects(lambda: fsa.select_blocks(qb, c, r[:, :, :2], T, 0.1, 0.04), "radius")
    rejects(lambda: fsa.block_stats(k, T, centroid=c[:, :, :1]), "centroid")
    # decode
    Bd, N, P = 2, 512, 16
    qd = torch.zeros((Bd, 8, 128), dtype=torch.bfloat16)
    pool = torch.zeros((64, 2, P, 128), dtype=torch.bfloat16)
    pt = torch.zeros((Bd, N // P), dtype=torch.int32)
    sl = torch.full((Bd,), N, dtype=torch.int32)
    idx = torch.zeros((Bd, 8, 16), dtype=torch.int64)
    rejects(lambda: fsa.sparse_decode_attn(qd, pool, pool, pt, sl, mode=fsa.SEL_INDEX, idx=idx), "idx")
    rejects(lambda: fsa.sparse_decode_attn(qd, pool, pool, pt, sl, mode=fsa.SEL_INDEX_KV,
                                           idx=idx.int()), r"idx must be \[2, 2, k\]")
    rejects(lambda: fsa.sparse_decode_attn(qd, pool, pool[:32], pt, sl), "v_pool")
    rejects(lambda: fsa.sparse_decode_attn(qd.float(), pool, pool, pt, sl), "q must be")
    rejects(lambda: fsa.sparse_decode_attn(qd, pool, pool, pt.long(), sl), "page_table")
    rejects(lambda: fsa.sparse_decode_attn(qd, pool, pool, pt, sl[:1]), "seq_lens")
    rejects(lambda: fsa.sparse_decode_attn(qd, pool, pool, pt, sl, mode=fsa.SEL_SEGMENT,
                                           segments=torch.zeros((Bd, 2, 3), dtype=torch.int32),
                                           n_seg=sl), "segments")
    rejects(lambda: fsa.topk_indices(qd, pool[..., :64], pt, sl, 16), "head dim")
    rejects(lambda: fsa.topk_indices(qd, pool, pt, sl, 16, idx=torch.zeros((Bd, 8, 8), dtype=torch.int32)),
            "idx")
    rejects(lambda: fsa.sparse_decode_attn_noalloc(qd, pool, pool, pt, sl, mode=fsa.SEL_INDEX, idx=idx),
            "idx")


def test_topk_union_kv_validation():
    L, lib = _lib()
    call = lambda B, Hq, Hkv, k, idx=FAKE, out=FAKE: lib.topk_union_kv(idx, B, Hq, Hkv, k, out, None, None)
    assert call(2, 8, 2, 16, idx=None) == L.FSA_ERR_NULL
    assert call(2, 8, 2, 16, out=None) == L.FSA_ERR_NULL
    assert call(2, 8, 3, 16) == L.FSA_ERR_SHAPE
    assert call(0, 8, 2, 16) == L.FSA_ERR_SHAPE
    assert call(2, 8, 2, 0) == L.FSA_ERR_ARG
    assert call(2, 16, 1, 1025) == L.FSA_ERR_ARG     # 16 x 1025 entries: beyond the sort


def test_scored_mode_validation():
    """FSA_SEL_INDEX_SCORED needs idx and scores; the key pool may be NULL
    there (keys are not read) but nowhere else."""
    L, lib = _lib()
    s = _dshape(L)
    call = lambda sel, kp=FAKE: lib.sparse_decode_attn(
        L.FSA_BF16, FAKE, kp, FAKE, FAKE, FAKE, ctypes.byref(s), ctypes.byref(sel), 0.1, FAKE,
        None, FAKE, 1 << 30, None)
    sel = L.KvSelect(L.FSA_SEL_INDEX_SCORED, FAKE.value, 16, None, None, 0, 0, None)
    assert call(sel) == L.FSA_ERR_NULL                       # no scores
    sel = L.KvSelect(L.FSA_SEL_INDEX_SCORED, FAKE.value, 16, None, None, 0, 0, FAKE.value)
    assert call(sel, kp=None) == L.FSA_ERR_NO_DEVICE         # valid: reaches the device check
    sel = L.KvSelect(L.FSA_SEL_INDEX, FAKE.value, 16, None, None, 0, 0, FAKE.value)
    assert call(sel, kp=None) == L.FSA_ERR_NULL              # other modes read the keys
    assert lib.fsa_workspace_size(L.FSA_OP_DECODE_ATTN, ctypes.byref(s), ctypes.byref(
        L.KvSelect(L.FSA_SEL_INDEX_SCORED, None, 16, None, None, 0, 2, None))) == 2 * 8 * 2 * 130 * 4
    k = 16
    assert lib.topk_indices_scored(L.FSA_BF16, FAKE, FAKE, FAKE, FAKE, ctypes.byref(s), k, FAKE,
                                   None, None, FAKE, 1 << 30, None) == L.FSA_ERR_NULL

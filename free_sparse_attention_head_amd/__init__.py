"""Head-aware sparse attention for long-context inference on AMD MI355X (gfx950).

Thin Python binding over the C-ABI library libfsa.so (include/fsa.h).  Each
function only marshals arguments: it reads shapes from the tensors, allocates
outputs and workspace with torch on the tensors' device, passes raw pointers
and the current HIP stream, and raises on a non-zero status.  Every step of
the computation runs in the library's HIP kernels; if the library is missing
the call raises.

Functions keep the library's names:
  block_stats, select_blocks, sparse_prefill_attn   (RBS-style sparse prefill)
  topk_indices, sparse_decode_attn                  (Kascade / segment decode)
  build_segments, workspace_size                    (helpers)
"""

import ctypes
import math

import torch

from . import _lib as L

__all__ = ["block_stats", "select_blocks", "sparse_prefill_attn", "topk_indices",
           "topk_indices_kv", "topk_indices_scored", "topk_union_kv", "sparse_decode_attn", "sparse_decode_attn_noalloc", "build_segments", "workspace_size", "FsaError",
           "SEL_ALL", "SEL_INDEX", "SEL_SEGMENT", "SEL_INDEX_KV", "SEL_INDEX_SCORED", "SEG_GLOBAL", "SEG_FOCUS",
           "SEG_LOCAL", "SEG_STREAMING"]

FsaError = L.FsaError
SEL_ALL, SEL_INDEX, SEL_SEGMENT, SEL_INDEX_KV, SEL_INDEX_SCORED = (
    L.FSA_SEL_ALL, L.FSA_SEL_INDEX, L.FSA_SEL_SEGMENT, L.FSA_SEL_INDEX_KV, L.FSA_SEL_INDEX_SCORED)
SEG_GLOBAL, SEG_FOCUS, SEG_LOCAL, SEG_STREAMING = (L.FSA_SEG_GLOBAL, L.FSA_SEG_FOCUS,
                                                   L.FSA_SEG_LOCAL, L.FSA_SEG_STREAMING)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return L.FSA_BF16
    if t.dtype == torch.float32:
        return L.FSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


# Argument checks.  The library receives raw pointers and trusts the shapes it
# is given, so every tensor is checked against them here, before any call:
# a wrong dtype or a short buffer would otherwise be read or written past its
# end on the device.

def _need(t, name, dtype=None, shape=None, ndim=None):
    """Raise ValueError unless tensor t has the given dtype / shape / rank."""
    if t is None:
        raise ValueError(f"{name} is required")
    if dtype is not None:
        ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
        if not ok:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


_FLOATS = (torch.bfloat16, torch.float32)


def _same_device(ref, *ts):
    for t in ts:
        if t is not None and t.device != ref.device:
            raise ValueError(f"every tensor must live on {ref.device}, found one on {t.device}")


def _same_dtype(ref, *named):
    for t, name in named:
        if t.dtype != ref.dtype:
            raise ValueError(f"{name} must have the query's dtype {ref.dtype}, got {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _prefill_shape(q, k, T):
    B, S, Hq, D = q.shape
    return L.PrefillShape(B, S, Hq, k.shape[2], D, T)


def _ws(nbytes, device, ws=None):
    if nbytes == 0:
        return None, 0
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small")
        return ws, ws.numel() * ws.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def workspace_size(op, shape, params=None):
    """Bytes of workspace op needs (op: 'select', 'prefill', 'topk', 'decode')."""
    lib = L.load()
    code = {"select": L.FSA_OP_SELECT_BLOCKS, "prefill": L.FSA_OP_PREFILL_ATTN,
            "topk": L.FSA_OP_TOPK, "decode": L.FSA_OP_DECODE_ATTN}[op]
    pp = None
    if isinstance(params, int):
        pp = ctypes.byref(ctypes.c_int(params))
    elif params is not None:
        pp = ctypes.byref(params)
    return lib.fsa_workspace_size(code, ctypes.byref(shape), pp)


def block_stats(k, T, centroid=None, radius=None):
    """Centroid [B,Hkv,nB,D] and radius [B,Hkv,nB] (fp32) of every key block of
    k [B,S,Hkv,D] (bf16 or fp32)."""
    lib = L.load()
    _need(k, "k", _FLOATS, ndim=4)
    B, S, Hkv, D = k.shape
    if T <= 0 or S % T:
        raise ValueError("the prompt length must be a multiple of the block size")
    nB = S // T
    shape = L.PrefillShape(B, S, Hkv, Hkv, D, T)
    if centroid is None:
        centroid = torch.empty((B, Hkv, nB, D), dtype=torch.float32, device=k.device)
    if radius is None:
        radius = torch.empty((B, Hkv, nB), dtype=torch.float32, device=k.device)
    _need(centroid, "centroid", torch.float32, (B, Hkv, nB, D))
    _need(radius, "radius", torch.float32, (B, Hkv, nB))
    _same_device(k, centroid, radius)
    L.check("block_stats", lib.block_stats(_dtype_code(k), _ptr(k), ctypes.byref(shape),
                                           _ptr(centroid), _ptr(radius), _stream(k.device)))
    return centroid, radius


def select_blocks(q, centroid, radius, T, p_centroid, p_rescue, band_blocks=0, sink_blocks=0,
                  want_scores=False, out=None, ws=None):
    """Two-branch block selection.  q [B,S,Hq,D]; stats from block_stats.
    Returns dict(mask [B,Hq,nB,ceil(nB/32)] int32 view of uint32 bits,
    block_idx [B,Hq,nB,nB], block_cnt [B,Hq,nB], score_c, score_r)."""
    lib = L.load()
    _need(q, "q", _FLOATS, ndim=4)
    B, S, Hq, D = q.shape
    if T <= 0 or S % T:
        raise ValueError("the prompt length must be a multiple of the block size")
    nB = S // T
    _need(centroid, "centroid", torch.float32, ndim=4)
    Hkv = centroid.shape[1]
    _need(centroid, "centroid", shape=(B, Hkv, nB, D))
    _need(radius, "radius", torch.float32, (B, Hkv, nB))
    shape = L.PrefillShape(B, S, Hq, Hkv, D, T)
    params = L.SelectParams(float(p_centroid), float(p_rescue), int(band_blocks), int(sink_blocks))
    dev = q.device
    o = out or {}
    mask = o.get("mask")
    if mask is None:
        mask = torch.empty((B, Hq, nB, (nB + 31) // 32), dtype=torch.int32, device=dev)
    bidx = o.get("block_idx")
    if bidx is None:
        bidx = torch.empty((B, Hq, nB, nB), dtype=torch.int32, device=dev)
    bcnt = o.get("block_cnt")
    if bcnt is None:
        bcnt = torch.empty((B, Hq, nB), dtype=torch.int32, device=dev)
    _need(mask, "mask", torch.int32, (B, Hq, nB, (nB + 31) // 32))
    _need(bidx, "block_idx", torch.int32, (B, Hq, nB, nB))
    _need(bcnt, "block_cnt", torch.int32, (B, Hq, nB))
    sc = sr = None
    if want_scores:
        sc = torch.full((B, Hq, nB, nB), float("nan"), dtype=torch.float32, device=dev)
        sr = torch.full((B, Hq, nB, nB), float("nan"), dtype=torch.float32, device=dev)
    _same_device(q, centroid, radius, mask, bidx, bcnt, ws)
    wsb = workspace_size("select", shape)
    ws, wsn = _ws(wsb, dev, ws)
    L.check("select_blocks", lib.select_blocks(
        _dtype_code(q), _ptr(q), _ptr(centroid), _ptr(radius), ctypes.byref(shape),
        ctypes.byref(params), _ptr(mask), _ptr(bidx), _ptr(bcnt), _ptr(sc), _ptr(sr), _ptr(ws),
        wsn, _stream(dev)))
    return {"mask": mask, "block_idx": bidx, "block_cnt": bcnt, "score_c": sc, "score_r": sr}


def sparse_prefill_attn(q, k, v, T, block_idx=None, block_cnt=None, scale=None, want_lse=True,
                        out=None, lse=None):
    """Block-sparse causal attention; block_idx None means dense causal.
    Returns (out [B,S,Hq,D] in q's dtype, lse [B,Hq,S] fp32 or None)."""
    lib = L.load()
    _need(q, "q", _FLOATS, ndim=4)
    B, S, Hq, D = q.shape
    _need(k, "k", ndim=4)
    _same_dtype(q, (k, "k"), (v, "v"))
    if k.shape[0] != B or k.shape[1] != S or k.shape[3] != D:
        raise ValueError(f"k must be [B, S, Hkv, D] = [{B}, {S}, Hkv, {D}], got {tuple(k.shape)}")
    _need(v, "v", shape=k.shape)
    if T <= 0 or S % T:
        raise ValueError("the prompt length must be a multiple of the block size")
    nB = S // T
    if (block_idx is None) != (block_cnt is None):
        raise ValueError("block_idx and block_cnt go together")
    if block_idx is not None:
        _need(block_idx, "block_idx", torch.int32, (B, Hq, nB, nB))
        _need(block_cnt, "block_cnt", torch.int32, (B, Hq, nB))
    shape = _prefill_shape(q, k, T)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, q.shape)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    if not want_lse:
        lse = None
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq, S))
    _same_device(q, k, v, block_idx, block_cnt, out, lse)
    L.check("sparse_prefill_attn", lib.sparse_prefill_attn(
        _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(shape), _ptr(block_idx),
        _ptr(block_cnt), float(scale), _ptr(out), _ptr(lse), None, 0, _stream(q.device)))
    return out, lse


def _decode_shape(q, k_pool, page_table, max_seq_len, seq_lens=None):
    _need(q, "q", torch.bfloat16, ndim=3)
    B, Hq, D = q.shape
    _need(k_pool, "k_pool", torch.bfloat16, ndim=4)
    num_pages, Hkv, P, Dk = k_pool.shape
    if Dk != D:
        raise ValueError(f"k_pool head dim {Dk} differs from the query's {D}")
    _need(page_table, "page_table", torch.int32, ndim=2)
    if page_table.shape[0] != B:
        raise ValueError(f"page_table must have {B} rows, got {page_table.shape[0]}")
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", torch.int32, (B,))
    max_pages = page_table.shape[1]
    if max_seq_len is None:
        max_seq_len = P * max_pages
    return L.DecodeShape(B, Hq, Hkv, D, P, num_pages, max_pages, int(max_seq_len))


def _topk(name, rows, q, k_pool, page_table, seq_lens, k, max_seq_len, idx, kth, ws):
    lib = L.load()
    shape = _decode_shape(q, k_pool, page_table, max_seq_len, seq_lens)
    B = q.shape[0]
    if idx is None:
        idx = torch.empty((B, rows, k), dtype=torch.int32, device=q.device)
    if kth is None:
        kth = torch.empty((B, rows), dtype=torch.float32, device=q.device)
    _need(idx, "idx", torch.int32, (B, rows, k))
    _need(kth, "kth", torch.float32, (B, rows))
    _same_device(q, k_pool, page_table, seq_lens, idx, kth, ws)
    wsb = workspace_size("topk", shape, int(k))
    ws, wsn = _ws(wsb, q.device, ws)
    L.check(name, getattr(lib, name)(
        _dtype_code(q), _ptr(q), _ptr(k_pool), _ptr(page_table), _ptr(seq_lens),
        ctypes.byref(shape), int(k), _ptr(idx), _ptr(kth), _ptr(ws), wsn, _stream(q.device)))
    return idx, kth


def topk_indices(q, k_pool, page_table, seq_lens, k, max_seq_len=None, idx=None, kth=None,
                 ws=None):
    """Exact per-head top-k token indices (ascending) and k-th score.
    q [B,Hq,D] bf16, k_pool [pages,Hkv,16,D] bf16, page_table [B,max_pages] int32,
    seq_lens [B] int32.  Returns idx [B,Hq,k], kth [B,Hq]."""
    return _topk("topk_indices", q.shape[1], q, k_pool, page_table, seq_lens, k, max_seq_len,
                 idx, kth, ws)


def topk_indices_scored(q, k_pool, page_table, seq_lens, k, max_seq_len=None, idx=None,
                        scores=None, kth=None, ws=None):
    """topk_indices plus each kept key's raw fp32 score.  Returns idx
    [B,Hq,k], scores [B,Hq,k] and kth [B,Hq]; idx and scores feed
    sparse_decode_attn with mode=SEL_INDEX_SCORED, which then reads only V."""
    lib = L.load()
    shape = _decode_shape(q, k_pool, page_table, max_seq_len, seq_lens)
    B, Hq = q.shape[0], q.shape[1]
    if idx is None:
        idx = torch.empty((B, Hq, k), dtype=torch.int32, device=q.device)
    if scores is None:
        scores = torch.empty((B, Hq, k), dtype=torch.float32, device=q.device)
    if kth is None:
        kth = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(idx, "idx", torch.int32, (B, Hq, k))
    _need(scores, "scores", torch.float32, (B, Hq, k))
    _need(kth, "kth", torch.float32, (B, Hq))
    _same_device(q, k_pool, page_table, seq_lens, idx, scores, kth, ws)
    wsb = workspace_size("topk", shape, int(k))
    ws, wsn = _ws(wsb, q.device, ws)
    L.check("topk_indices_scored", lib.topk_indices_scored(
        _dtype_code(q), _ptr(q), _ptr(k_pool), _ptr(page_table), _ptr(seq_lens),
        ctypes.byref(shape), int(k), _ptr(idx), _ptr(scores), _ptr(kth), _ptr(ws), wsn,
        _stream(q.device)))
    return idx, scores, kth


def topk_indices_kv(q, k_pool, page_table, seq_lens, k, max_seq_len=None, idx=None, kth=None,
                    ws=None):
    """Exact top-k per KV head of the max over its query heads' scores.
    Returns idx [B,Hkv,k] (ascending) and kth [B,Hkv]; feed idx to
    sparse_decode_attn with mode=SEL_INDEX_KV."""
    return _topk("topk_indices_kv", k_pool.shape[1], q, k_pool, page_table, seq_lens, k,
                 max_seq_len, idx, kth, ws)


def topk_union_kv(idx, Hkv, out=None, cnt=None):
    """Union of each KV head's G query-head index sets (idx [B,Hq,k] int32,
    as topk_indices returns it).  Returns out [B,Hkv,G*k] (distinct entries
    ascending, then -1) and cnt [B,Hkv]; feed out to sparse_decode_attn with
    mode=SEL_INDEX_KV."""
    lib = L.load()
    _need(idx, "idx", torch.int32, ndim=3)
    B, Hq, k = idx.shape
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"{Hq} query heads do not divide into {Hkv} KV heads")
    G = Hq // Hkv
    if out is None:
        out = torch.empty((B, Hkv, G * k), dtype=torch.int32, device=idx.device)
    if cnt is None:
        cnt = torch.empty((B, Hkv), dtype=torch.int32, device=idx.device)
    _need(out, "out", torch.int32, (B, Hkv, G * k))
    _need(cnt, "cnt", torch.int32, (B, Hkv))
    _same_device(idx, out, cnt)
    L.check("topk_union_kv", lib.topk_union_kv(_ptr(idx), B, Hq, Hkv, k, _ptr(out), _ptr(cnt),
                                               _stream(idx.device)))
    return out, cnt


def _decode_args(q, k_pool, v_pool, page_table, seq_lens, mode, idx, segments, n_seg, n_split,
                 max_seq_len, want_lse, out, lse, scores=None):
    """Checks of a decode call's tensors; returns (KvSelect, out, lse)."""
    _decode_shape(q, k_pool, page_table, max_seq_len, seq_lens)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    _need(v_pool, "v_pool", torch.bfloat16, k_pool.shape)
    if mode in (SEL_INDEX, SEL_INDEX_KV, SEL_INDEX_SCORED):
        _need(idx, "idx", torch.int32, ndim=3)
        heads = Hkv if mode == SEL_INDEX_KV else Hq
        if idx.shape[0] != B or idx.shape[1] != heads:
            raise ValueError(f"idx must be [{B}, {heads}, k], got {tuple(idx.shape)}")
        if mode == SEL_INDEX_SCORED:
            _need(scores, "scores", torch.float32, idx.shape)
    elif mode == SEL_SEGMENT:
        _need(segments, "segments", torch.int32, ndim=3)
        if segments.shape[0] != B or segments.shape[2] != 2:
            raise ValueError(f"segments must be [{B}, max_seg, 2], got {tuple(segments.shape)}")
        _need(n_seg, "n_seg", torch.int32, (B,))
    elif mode != SEL_ALL:
        raise ValueError(f"unknown mode {mode}")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, Hq, D))
    if want_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if not want_lse:
        lse = None
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq))
    _same_device(q, k_pool, v_pool, page_table, seq_lens, idx, segments, n_seg, out, lse, scores)
    sel = L.KvSelect(int(mode), None, 0, None, None, 0, int(n_split), None)
    if mode in (SEL_INDEX, SEL_INDEX_KV, SEL_INDEX_SCORED):
        sel.idx = _ptr(idx).value
        sel.k = idx.shape[2]
        if mode == SEL_INDEX_SCORED:
            sel.scores = _ptr(scores).value
    elif mode == SEL_SEGMENT:
        sel.segments = _ptr(segments).value
        sel.n_seg = _ptr(n_seg).value
        sel.max_seg = segments.shape[1]
    return sel, out, lse


def sparse_decode_attn(q, k_pool, v_pool, page_table, seq_lens, mode=SEL_ALL, idx=None,
                       segments=None, n_seg=None, scale=None, n_split=0, max_seq_len=None,
                       want_lse=True, out=None, lse=None, ws=None, scores=None):
    """Split-KV paged decode attention.  mode SEL_ALL / SEL_INDEX (idx [B,Hq,k]) /
    SEL_INDEX_KV (idx [B,Hkv,k]) / SEL_INDEX_SCORED (idx and scores [B,Hq,k],
    V read only) / SEL_SEGMENT (segments [B,max_seg,2], n_seg [B]).
    Returns (out bf16 [B,Hq,D], lse fp32 [B,Hq] or None)."""
    lib = L.load()
    sel, out, lse = _decode_args(q, k_pool, v_pool, page_table, seq_lens, mode, idx, segments,
                                 n_seg, n_split, max_seq_len, want_lse, out, lse, scores)
    shape = _decode_shape(q, k_pool, page_table, max_seq_len, seq_lens)
    D = q.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    wsb = workspace_size("decode", shape, sel)
    ws, wsn = _ws(wsb, q.device, ws)
    L.check("sparse_decode_attn", lib.sparse_decode_attn(
        _dtype_code(q), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table), _ptr(seq_lens),
        ctypes.byref(shape), ctypes.byref(sel), float(scale), _ptr(out), _ptr(lse), _ptr(ws),
        wsn, _stream(q.device)))
    return out, lse


def sparse_decode_attn_noalloc(q, k_pool, v_pool, page_table, seq_lens, mode=SEL_ALL, idx=None,
                               segments=None, n_seg=None, scale=None, n_split=0,
                               max_seq_len=None, want_lse=True, out=None, lse=None,
                               scores=None):
    """sparse_decode_attn without a workspace: the library keeps the split
    partials in its own device array (FSA_NOALLOC_SCRATCH_BYTES per GPU).
    Calls that overlap on one GPU race.  Pass out (and lse) to allocate
    nothing here either."""
    lib = L.load()
    sel, out, lse = _decode_args(q, k_pool, v_pool, page_table, seq_lens, mode, idx, segments,
                                 n_seg, n_split, max_seq_len, want_lse, out, lse, scores)
    shape = _decode_shape(q, k_pool, page_table, max_seq_len, seq_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[2])
    L.check("sparse_decode_attn_noalloc", lib.sparse_decode_attn_noalloc(
        _dtype_code(q), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table), _ptr(seq_lens),
        ctypes.byref(shape), ctypes.byref(sel), float(scale), _ptr(out), _ptr(lse),
        _stream(q.device)))
    return out, lse


def build_segments(mode, n, chunk_start=0, chunk_len=2048, local_len=1024, n_sink=4, page=16,
                   min_neighbourhood=0):
    """Host-side segment builder: sorted merged [start, end) token ranges.
    min_neighbourhood widens a focus chunk by that many tokens on each side."""
    lib = L.load()
    buf = (ctypes.c_int32 * 4)()
    cnt = ctypes.c_int(0)
    L.check("fsa_build_segments_nb", lib.fsa_build_segments_nb(
        int(mode), int(n), int(chunk_start), int(chunk_len), int(local_len), int(n_sink),
        int(page), int(min_neighbourhood), buf, ctypes.byref(cnt)))
    return [(buf[2 * i], buf[2 * i + 1]) for i in range(cnt.value)]

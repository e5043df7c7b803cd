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
           "topk_indices_kv", "sparse_decode_attn", "build_segments", "workspace_size", "FsaError",
           "SEL_ALL", "SEL_INDEX", "SEL_SEGMENT", "SEL_INDEX_KV", "SEG_GLOBAL", "SEG_FOCUS",
           "SEG_LOCAL", "SEG_STREAMING"]

FsaError = L.FsaError
SEL_ALL, SEL_INDEX, SEL_SEGMENT, SEL_INDEX_KV = (L.FSA_SEL_ALL, L.FSA_SEL_INDEX, L.FSA_SEL_SEGMENT,
                                             L.FSA_SEL_INDEX_KV)
SEG_GLOBAL, SEG_FOCUS, SEG_LOCAL, SEG_STREAMING = (L.FSA_SEG_GLOBAL, L.FSA_SEG_FOCUS,
                                                   L.FSA_SEG_LOCAL, L.FSA_SEG_STREAMING)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return L.FSA_BF16
    if t.dtype == torch.float32:
        return L.FSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


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
    B, S, Hkv, D = k.shape
    nB = S // T
    shape = L.PrefillShape(B, S, Hkv, Hkv, D, T)
    if centroid is None:
        centroid = torch.empty((B, Hkv, nB, D), dtype=torch.float32, device=k.device)
    if radius is None:
        radius = torch.empty((B, Hkv, nB), dtype=torch.float32, device=k.device)
    L.check("block_stats", lib.block_stats(_dtype_code(k), _ptr(k), ctypes.byref(shape),
                                           _ptr(centroid), _ptr(radius), _stream(k.device)))
    return centroid, radius


def select_blocks(q, centroid, radius, T, p_centroid, p_rescue, band_blocks=0, sink_blocks=0,
                  want_scores=False, out=None, ws=None):
    """Two-branch block selection.  q [B,S,Hq,D]; stats from block_stats.
    Returns dict(mask [B,Hq,nB,ceil(nB/32)] int32 view of uint32 bits,
    block_idx [B,Hq,nB,nB], block_cnt [B,Hq,nB], score_c, score_r)."""
    lib = L.load()
    B, S, Hq, D = q.shape
    Hkv = centroid.shape[1]
    nB = S // T
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
    sc = sr = None
    if want_scores:
        sc = torch.full((B, Hq, nB, nB), float("nan"), dtype=torch.float32, device=dev)
        sr = torch.full((B, Hq, nB, nB), float("nan"), dtype=torch.float32, device=dev)
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
    B, S, Hq, D = q.shape
    shape = _prefill_shape(q, k, T)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    if not want_lse:
        lse = None
    L.check("sparse_prefill_attn", lib.sparse_prefill_attn(
        _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(shape), _ptr(block_idx),
        _ptr(block_cnt), float(scale), _ptr(out), _ptr(lse), None, 0, _stream(q.device)))
    return out, lse


def _decode_shape(q, k_pool, page_table, max_seq_len):
    B, Hq, D = q.shape
    num_pages, Hkv, P, _ = k_pool.shape
    max_pages = page_table.shape[1]
    if max_seq_len is None:
        max_seq_len = P * max_pages
    return L.DecodeShape(B, Hq, Hkv, D, P, num_pages, max_pages, int(max_seq_len))


def _topk(name, rows, q, k_pool, page_table, seq_lens, k, max_seq_len, idx, kth, ws):
    lib = L.load()
    shape = _decode_shape(q, k_pool, page_table, max_seq_len)
    B = q.shape[0]
    if idx is None:
        idx = torch.empty((B, rows, k), dtype=torch.int32, device=q.device)
    if kth is None:
        kth = torch.empty((B, rows), dtype=torch.float32, device=q.device)
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


def topk_indices_kv(q, k_pool, page_table, seq_lens, k, max_seq_len=None, idx=None, kth=None,
                    ws=None):
    """Exact top-k per KV head of the max over its query heads' scores.
    Returns idx [B,Hkv,k] (ascending) and kth [B,Hkv]; feed idx to
    sparse_decode_attn with mode=SEL_INDEX_KV."""
    return _topk("topk_indices_kv", k_pool.shape[1], q, k_pool, page_table, seq_lens, k,
                 max_seq_len, idx, kth, ws)


def sparse_decode_attn(q, k_pool, v_pool, page_table, seq_lens, mode=SEL_ALL, idx=None,
                       segments=None, n_seg=None, scale=None, n_split=0, max_seq_len=None,
                       want_lse=True, out=None, lse=None, ws=None):
    """Split-KV paged decode attention.  mode SEL_ALL / SEL_INDEX (idx [B,Hq,k]) /
    SEL_INDEX_KV (idx [B,Hkv,k]) / SEL_SEGMENT (segments [B,max_seg,2], n_seg [B]).
    Returns (out bf16 [B,Hq,D], lse fp32 [B,Hq] or None)."""
    lib = L.load()
    shape = _decode_shape(q, k_pool, page_table, max_seq_len)
    B, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    sel = L.KvSelect(int(mode), None, 0, None, None, 0, int(n_split))
    if mode in (SEL_INDEX, SEL_INDEX_KV):
        sel.idx = _ptr(idx).value
        sel.k = idx.shape[2]
    elif mode == SEL_SEGMENT:
        sel.segments = _ptr(segments).value
        sel.n_seg = _ptr(n_seg).value
        sel.max_seg = segments.shape[1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if not want_lse:
        lse = None
    wsb = workspace_size("decode", shape, sel)
    ws, wsn = _ws(wsb, q.device, ws)
    L.check("sparse_decode_attn", lib.sparse_decode_attn(
        _dtype_code(q), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table), _ptr(seq_lens),
        ctypes.byref(shape), ctypes.byref(sel), float(scale), _ptr(out), _ptr(lse), _ptr(ws),
        wsn, _stream(q.device)))
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

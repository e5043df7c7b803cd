"""fp64 softmax attention over explicit key sets (test infrastructure only).

Everything here is the textbook definition of scaled softmax attention,
o = sum_s softmax_s(scale * q.k_s) v_s and lse = log sum_s exp(scale * q.k_s),
evaluated on exactly the key set that a mask, an index list or a token-range
list admits.  The sources fix *which* keys are read, never how the softmax is
computed:
  * RBS-Attention post, "Key technical points" 2: the merged block mask is
    executed by an unchanged block-sparse FlashAttention, i.e. the result is
    exact softmax attention restricted to the admitted blocks.
  * Kascade post, "What Kascade got right": reuse layers attend only at the k
    anchor indices.
  * Declarative Attention post, "Declarative attention protocol": the
    segment mask is consumed by an unmodified FlashAttention.
  * LoZA post, "4. From food delivery to AI": SplitKV-and-Combine merges
    partial results computed over disjoint slices of the KV cache.
Inputs are widened to float64 by the caller-visible np.asarray(..., float64);
no re-rounding happens here.
"""

import math

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _softmax_row(scores, values):
    """Exact softmax-weighted sum of `values` rows for one query.

    scores [n], values [n, Dv].  Returns (o [Dv], lse).  An empty key set
    gives o = 0 and lse = -inf (nothing is attended).
    """
    if scores.size == 0:
        return np.zeros(values.shape[1], dtype=np.float64), -math.inf
    m = scores.max()
    w = np.exp(scores - m)
    l = w.sum()
    o = (w[:, None] * values).sum(axis=0) / l
    return o, m + math.log(l)


def dense_attention(q, k, v, scale, causal=True):
    """Dense (causal) softmax attention for one head.

    q [Sq, D], k [Sk, D], v [Sk, Dv].  With causal=True query t sees keys
    s <= t (prefill self-attention, Sq == Sk, same token positions).
    Returns o [Sq, Dv] and lse [Sq] (natural log).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    sq = q.shape[0]
    o = np.zeros((sq, v.shape[1]), dtype=np.float64)
    lse = np.zeros(sq, dtype=np.float64)
    for t in range(sq):
        n = t + 1 if causal else k.shape[0]
        s = scale * (k[:n] @ q[t])
        o[t], lse[t] = _softmax_row(s, v[:n])
    return o, lse


def _visible_keys(t, T, mask_row):
    """Token indices s <= t whose key block is set in mask_row (block mask row
    of query block t // T)."""
    keys = []
    for j in np.flatnonzero(mask_row):
        lo = j * T
        hi = min((j + 1) * T, t + 1)
        if lo < hi:
            keys.append(np.arange(lo, hi))
    if not keys:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(keys)


def masked_attention_rows(q, k, v, mask, T, scale, rows):
    """Block-masked causal attention for selected query rows of one head.

    mask [nB, nB] bool: mask[i, j] admits key block j for query block i.
    Query t attends A(t) = {s <= t : mask[t // T, s // T]} (RBS-Attention post,
    "Key technical points" 2: the block-sparse FlashAttention path executes
    the merged mask unchanged; causality is applied element-wise).
    Returns o [len(rows), Dv], lse [len(rows)].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    mask = np.asarray(mask, dtype=bool)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.zeros(rows.size, dtype=np.float64)
    for n, t in enumerate(rows):
        keys = _visible_keys(int(t), T, mask[t // T])
        s = scale * (k[keys] @ q[t])
        o[n], lse[n] = _softmax_row(s, v[keys])
    return o, lse


def masked_attention(q, k, v, mask, T, scale):
    """Block-masked causal attention for every query row of one head."""
    return masked_attention_rows(q, k, v, mask, T, scale, np.arange(q.shape[0]))


def index_attention(q, kseq, vseq, idx, scale):
    """Softmax attention of one query over the keys listed in idx.

    Kascade post, "What Kascade got right": a reuse layer attends only at the
    anchor's k indices.  Negative entries are empty slots and are skipped.
    q [D], kseq [N, D], vseq [N, Dv].  Returns (o [Dv], lse).
    """
    q, kseq, vseq = _f64(q), _f64(kseq), _f64(vseq)
    idx = np.asarray(idx, dtype=np.int64)
    idx = idx[idx >= 0]
    s = scale * (kseq[idx] @ q)
    return _softmax_row(s, vseq[idx])


def segment_attention(q, kseq, vseq, ranges, scale):
    """Softmax attention of one query over the union of token ranges.

    Declarative Attention post, "Declarative attention protocol": the mode
    (global/focus/local) becomes a set of kept token ranges that an unmodified
    attention kernel reads.  ranges: iterable of [start, end) pairs; a token in
    several ranges is attended once.
    """
    n = np.asarray(kseq).shape[0]
    keep = np.zeros(n, dtype=bool)
    for a, b in ranges:
        keep[int(a):int(b)] = True
    return index_attention(q, kseq, vseq, np.flatnonzero(keep), scale)


def attention_partial(q, kseq, vseq, idx, scale):
    """Un-combined partial (m, l, o) of one query over one slice of keys:
    m = max score, l = sum exp(score - m), o = normalised output of the slice.
    An empty slice gives (-inf, 0, 0)."""
    q, kseq, vseq = _f64(q), _f64(kseq), _f64(vseq)
    idx = np.asarray(idx, dtype=np.int64)
    if idx.size == 0:
        return -math.inf, 0.0, np.zeros(vseq.shape[1], dtype=np.float64)
    s = scale * (kseq[idx] @ q)
    m = s.max()
    w = np.exp(s - m)
    l = w.sum()
    return m, l, (w[:, None] * vseq[idx]).sum(axis=0) / l


def lse_combine(parts):
    """Merge split-KV partials (LoZA post, "4. From food delivery to AI":
    SplitKV-and-Combine).

    parts: list of (m_s, l_s, o_s).  M = max m_s;
    o = sum e^(m_s - M) l_s o_s / sum e^(m_s - M) l_s;
    lse = M + log sum e^(m_s - M) l_s.  Empty slices (m = -inf) add nothing.
    """
    live = [(m, l, np.asarray(o, dtype=np.float64)) for m, l, o in parts if l > 0]
    if not live:
        dv = np.asarray(parts[0][2]).shape[0]
        return np.zeros(dv, dtype=np.float64), -math.inf
    M = max(m for m, _, _ in live)
    wsum = sum(math.exp(m - M) * l for m, l, _ in live)
    o = sum(math.exp(m - M) * l * o for m, l, o in live) / wsum
    return o, M + math.log(wsum)

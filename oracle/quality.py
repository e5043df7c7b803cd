"""Selector quality: actual retention and the ideal block mask (test
infrastructure only).

RBS-Attention post, "Experimental data": the supporting experiments measure
the actual retention of tokens and compare selectors at matched density.  The
page defines neither quantity; the readings here:
  * the retention of query token t under a block mask M is the share of its
    causal softmax mass, softmax_s(scale * q_t . k_s) over keys s <= t, that
    falls on keys of the blocks M admits for t's query block;
  * the ideal mask at a given block count per row takes, for query block i,
    the visible key blocks with the largest mass averaged over the block's T
    queries (ties to the lower block index): by this measure no block
    selector does better at that count.
Plain definitions in float64: explicit scores, an explicit softmax per query,
sums over the admitted keys.  Parity status: pinned (tests/test_oracle_facts.py).
"""

import numpy as np


def token_block_mass(q, k, T, scale, rows=None):
    """Softmax mass of each query of query block i on each key block j <= i.

    q [S, D], k [S, D] (one head; S a multiple of T).  Returns a dict
    i -> array [T, i + 1] for each i in `rows` (default: every block).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    nB = q.shape[0] // T
    rows = range(nB) if rows is None else rows
    out = {}
    for i in rows:
        n = (i + 1) * T
        s = scale * (q[i * T:n] @ k[:n].T)                     # [T, n]
        visible = np.arange(n)[None, :] <= (i * T + np.arange(T))[:, None]
        s = np.where(visible, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out[i] = p.reshape(T, i + 1, T).sum(axis=2)
    return out


def retention(q, k, mask, T, scale, rows=None):
    """Retention of every query of the given query blocks under block mask
    `mask` [nB, nB] (bool; entries j > i are ignored).  Returns a dict
    i -> array [T]."""
    mask = np.asarray(mask, dtype=bool)
    mass = token_block_mass(q, k, T, scale, rows)
    return {i: m[:, mask[i, :i + 1]].sum(axis=1) for i, m in mass.items()}


def ideal_rows(q, k, T, scale, counts, rows):
    """The ideal block set of each query block i in `rows` at counts[i]
    blocks (clipped to the i + 1 visible ones): ascending block indices, and
    the retention of each of its T queries.  Returns a dict i -> (blocks,
    retention [T])."""
    mass = token_block_mass(q, k, T, scale, rows)
    out = {}
    for i, m in mass.items():
        c = int(min(max(counts[i], 0), i + 1))
        mean = m.mean(axis=0)
        order = np.lexsort((np.arange(i + 1), -mean))
        keep = np.sort(order[:c])
        out[i] = (keep, m[:, keep].sum(axis=1))
    return out


def index_mass(q, kseq, idx, scale):
    """Decode counterpart of retention: the share of one query's softmax mass
    over every cached key, softmax_j(scale * q . k_j) for j < N, that falls on
    the keys listed in idx (negative entries are empty slots; a key listed
    twice counts once).  q [D], kseq [N, D]."""
    q = np.asarray(q, dtype=np.float64)
    kseq = np.asarray(kseq, dtype=np.float64)
    s = scale * (kseq @ q)
    p = np.exp(s - s.max())
    p /= p.sum()
    idx = np.unique(np.asarray(idx, dtype=np.int64))
    return float(p[idx[idx >= 0]].sum())

"""fp64 exact top-k (test infrastructure only).

Kascade post, "What Kascade got right: anchor-layer Top-k reuse": an anchor
layer computes the exact Top-k key indices; "Head-aware is the key to
accuracy": this is done per attention head.  Reading taken: the score is the
raw dot product q.k over every cached key, ties go to the lower key index, and
the index set is returned sorted ascending (so that any consumer reads keys in
cache order).

topk_pooled is the GQA-shared counterpart: one index set per KV head, the
head-aware choice above traded for G query heads sharing every index (the
post argues for per-head sets; the shared one cuts reads by G).  Reading
taken: a key's pooled score is the maximum of its G query heads' raw scores
(kept if any head of the group rates it).
"""

import numpy as np


def topk(scores, k):
    """Exact top-k of one score row.

    Returns (idx, kth): idx = ascending indices of the k largest scores, where
    a stable sort on (-score, index) decides ties; kth = the k-th largest
    score.  Requires 1 <= k <= len(scores).
    """
    s = np.asarray(scores, dtype=np.float64)
    if not 1 <= k <= s.size:
        raise ValueError("k out of range")
    order = np.lexsort((np.arange(s.size), -s))
    keep = order[:k]
    return np.sort(keep), s[order[k - 1]]


def near_kth_mask(scores, kth, band):
    """True where |score - kth| <= band: entries that may flip between two
    correct top-k sets computed at different precisions."""
    s = np.asarray(scores, dtype=np.float64)
    return np.abs(s - kth) <= band


def topk_pooled(scores, k):
    """Exact top-k of the per-key maximum over the rows of `scores` [G, N]
    (the G query heads of one KV head).  Returns (idx, kth) as topk."""
    s = np.asarray(scores, dtype=np.float64)
    return topk(s.max(axis=0), k)

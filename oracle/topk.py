"""fp64 exact top-k of the anchor layer (test infrastructure only).

Kascade post, "What Kascade got right: anchor-layer Top-k reuse": an anchor
layer scores every cached key, keeps the exact Top-k key indices, and later
layers attend only there; "Head-aware is the key to accuracy": this is done
per attention head.  Readings taken: the score of cached token j for query
head h is the raw dot product q_h . k_j of the KV head that h reads
(consecutive query heads share a KV head), ties go to the lower key index,
and the index set is returned sorted ascending (so that any consumer reads
keys in cache order).

topk_pooled is the GQA-shared counterpart: one index set per KV head, the
head-aware choice above traded for G query heads sharing every index (the
post argues for per-head sets; the shared one cuts reads by G).  Reading
taken: a key's pooled score is the maximum of its G query heads' raw scores
(kept if any head of the group rates it).  union_sets is the other shared
form: the union of the G heads' own sets, which keeps every head's own
top-k and shares the K/V reads of keys that several heads chose.

Parity status: every function here is pinned in tests/test_oracle_facts.py
(closed forms, brute force, torch library routines).
"""

import numpy as np


def kv_head(h, Hq, Hkv):
    """KV head read by query head h when Hq query heads share Hkv KV heads:
    each run of G = Hq / Hkv consecutive query heads reads one KV head."""
    if Hq % Hkv != 0 or not 0 <= h < Hq:
        raise ValueError("bad head mapping")
    return h // (Hq // Hkv)


def anchor_scores(q, kseq):
    """Raw anchor-layer scores of one query head over one sequence's keys.

    q [D] (the query of head h), kseq [N, D] (the keys of the KV head h
    reads, in token order).  Returns s [N] with s_j = sum_d q_d kseq[j, d],
    in float64, unscaled.
    """
    q = np.asarray(q, dtype=np.float64)
    kseq = np.asarray(kseq, dtype=np.float64)
    return kseq @ q


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


def anchor_topk(q, kseq, k):
    """The anchor layer's index set of one query head: the exact top-k of its
    raw scores over every cached key.  Returns (idx ascending, kth)."""
    return topk(anchor_scores(q, kseq), k)


def topk_pooled(scores, k):
    """Exact top-k of the per-key maximum over the rows of `scores` [G, N]
    (the G query heads of one KV head).  Returns (idx, kth) as topk."""
    s = np.asarray(scores, dtype=np.float64)
    return topk(s.max(axis=0), k)


def union_sets(sets):
    """Union of the index sets of one KV head's query heads, ascending.
    Negative entries are empty slots and are dropped."""
    keep = set()
    for s in sets:
        keep.update(int(x) for x in np.asarray(s).ravel() if x >= 0)
    return np.array(sorted(keep), dtype=np.int64)


def set_recall(own, shared):
    """Share of a head's own index set (empty slots dropped) that a shared
    set contains: |own & shared| / |own|."""
    own = {int(x) for x in np.asarray(own).ravel() if x >= 0}
    shared = {int(x) for x in np.asarray(shared).ravel() if x >= 0}
    if not own:
        raise ValueError("empty own set")
    return len(own & shared) / len(own)

"""fp64 block statistics and the two-branch block selector (test infrastructure only).

Source: "RBS-Attention: Radius-Bounded Sparse Prefill for Long-Context LLMs"
(yunkai-blog post).
  * Overview: a block centroid can average away a single highly relevant key
    ("mean dilution"), so a centroid-only selector drops that block.
  * "Key technical points" 1: a centroid base branch scores the average
    relevance of a key block; a rescue branch uses the maximum key-block
    radius to flag blocks whose mean score is low but that may hide a highly
    relevant token.
  * "Key technical points" 2: each branch is thresholded on its own and the
    two masks are merged; block-sparse FlashAttention then runs unchanged.
The pages print no formulas.  Readings taken here (listed with reasons in the
design notes): the centroid c_b is the arithmetic mean of the block's keys;
the radius r_b is the largest Euclidean distance from a key of the block to
c_b; the per-block query is the mean of the query block's rows; the rescue
score is the Cauchy-Schwarz upper bound q.c_b + ||q|| r_b; a "threshold" keeps
the top max(1, ceil(p * n_i)) of the n_i = i + 1 causally visible blocks of
query block i, ties going to the lower block index; the masks merge by union,
plus forced sink/band blocks, clipped to j <= i.
"""

import math

import numpy as np


def block_stats(k, T):
    """Centroid and radius of every key block of one (batch, KV head).

    k [S, D] with S % T == 0.  Returns c [nB, D] (mean key of each block) and
    r [nB] (max over the block's keys of ||k - c||_2).  Causality is ignored:
    the statistics describe the whole block.
    """
    k = np.asarray(k, dtype=np.float64)
    S, D = k.shape
    nB = S // T
    c = np.zeros((nB, D), dtype=np.float64)
    r = np.zeros(nB, dtype=np.float64)
    for j in range(nB):
        blk = k[j * T:(j + 1) * T]
        c[j] = blk.mean(axis=0)
        r[j] = np.linalg.norm(blk - c[j], axis=1).max()
    return c, r


def pool_queries(q, T):
    """Mean query of every query block of one (batch, query head): q [S, D] ->
    [nB, D].  The query block size equals the key block size."""
    q = np.asarray(q, dtype=np.float64)
    S, D = q.shape
    return q.reshape(S // T, T, D).mean(axis=1)


def k_of(p, n):
    """Blocks a branch keeps out of n visible ones: max(1, ceil(p * n)),
    capped at n; a negative p switches the branch off (keeps none).  The
    product is formed in IEEE double, as the library does."""
    if p < 0:
        return 0
    return min(n, max(1, math.ceil(float(p) * float(n))))


def visible_count(nB):
    """Causally visible (i, j) block pairs, j <= i, of one head."""
    return nB * (nB + 1) // 2


def _top(scores, kk):
    """Indices of the kk largest scores, ties to the lower index (a stable sort
    on (-score, index)), plus the value of the last one kept (nan if kk = 0)."""
    order = np.lexsort((np.arange(scores.size), -scores))
    keep = order[:kk]
    tau = scores[keep[-1]] if kk > 0 else math.nan
    return keep, tau


def select_blocks(qbar, c, r, p_c, p_r, band_blocks=0, sink_blocks=0):
    """Two-branch block selection for one (batch, query head).

    qbar [nB, D] pooled queries of this head; c [nB, D], r [nB] block stats of
    its KV head.  For query block i and visible key block j <= i:
      Sc[i, j] = qbar_i . c_j                      (centroid base branch)
      Sr[i, j] = Sc[i, j] + ||qbar_i|| * r_j       (radius rescue bound)
    C_i = top k_of(p_c, i+1) blocks by Sc, R_i = top k_of(p_r, i+1) by Sr,
    F_i = {j < sink_blocks} U {i - band_blocks < j <= i},
    M_i = (C_i U R_i U F_i) restricted to j <= i.
    Returns a dict of bool masks C, R, M [nB, nB], scores Sc, Sr [nB, nB]
    (nan above the diagonal), thresholds tau_c, tau_r [nB] (score of the last
    kept entry of each branch) and kept counts k_c, k_r [nB].
    """
    qbar = np.asarray(qbar, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    nB = qbar.shape[0]
    Sc = np.full((nB, nB), np.nan)
    Sr = np.full((nB, nB), np.nan)
    C = np.zeros((nB, nB), dtype=bool)
    R = np.zeros((nB, nB), dtype=bool)
    M = np.zeros((nB, nB), dtype=bool)
    tau_c = np.full(nB, np.nan)
    tau_r = np.full(nB, np.nan)
    kc = np.zeros(nB, dtype=np.int64)
    kr = np.zeros(nB, dtype=np.int64)
    for i in range(nB):
        n = i + 1
        sc = c[:n] @ qbar[i]
        sr = sc + np.linalg.norm(qbar[i]) * r[:n]
        Sc[i, :n] = sc
        Sr[i, :n] = sr
        kc[i] = k_of(p_c, n)
        kr[i] = k_of(p_r, n)
        keep_c, tau_c[i] = _top(sc, kc[i])
        keep_r, tau_r[i] = _top(sr, kr[i])
        C[i, keep_c] = True
        R[i, keep_r] = True
        M[i] = C[i] | R[i]
        M[i, :min(sink_blocks, n)] = True
        if band_blocks > 0:
            M[i, max(0, i - band_blocks + 1):n] = True
    return {"Sc": Sc, "Sr": Sr, "C": C, "R": R, "M": M,
            "tau_c": tau_c, "tau_r": tau_r, "k_c": kc, "k_r": kr}

"""Comparison helpers shared by the GPU parity tests (test code only)."""

import numpy as np

BAND = 1e-3      # near-threshold band for masks and top-k sets
TOL_BF16 = 2e-2  # max-abs output tolerance, bf16 inputs
TOL_F32 = 1e-4   # max-abs output tolerance, fp32 inputs
# log-sum-exp tolerance (natural log).  Scores are exact fp32 products of the
# inputs and the row sum adds the same (bf16-rounded, for bf16 inputs)
# probabilities that weight the values, so the LSE error is a few ulps of the
# sum: these bounds leave an order of magnitude of room, and a constant bias
# of 0.01 (bf16) or 1e-4 (fp32) nats fails them.
LSE_TOL_BF16 = 1e-2
LSE_TOL_F32 = 1e-4


def lists_to_mask(block_idx, block_cnt, nB):
    """GPU block lists -> bool [nB, nB] mask of one head (numpy inputs)."""
    m = np.zeros((nB, nB), dtype=bool)
    for i in range(nB):
        c = int(block_cnt[i])
        m[i, block_idx[i, :c]] = True
    return m


def bits_to_mask(words, nB):
    """uint32 bitmask words [nB, W] (as int32) -> bool [nB, nB]."""
    w = np.asarray(words).astype(np.int64) & 0xFFFFFFFF
    m = np.zeros((nB, nB), dtype=bool)
    for j in range(nB):
        m[:, j] = (w[:, j // 32] >> (j % 32)) & 1
    return m


def mask_diff_excused(gpu_mask, sel):
    """Entries where the GPU mask differs from the oracle's merged mask.

    Returns (n_diff, n_excused): a differing entry is excused when its oracle
    centroid score is within BAND of the centroid threshold or its rescue
    score is within BAND of the rescue threshold (two correct selections at
    different precisions may disagree there)."""
    diff = gpu_mask != sel["M"]
    ii, jj = np.nonzero(diff)
    exc = 0
    for i, j in zip(ii, jj):
        near_c = abs(sel["Sc"][i, j] - sel["tau_c"][i]) <= BAND if sel["k_c"][i] > 0 else False
        near_r = abs(sel["Sr"][i, j] - sel["tau_r"][i]) <= BAND if sel["k_r"][i] > 0 else False
        exc += int(near_c or near_r)
    return int(diff.sum()), exc


def topk_diff_excused(gpu_idx, oracle_idx, scores, kth):
    """Symmetric difference of two top-k sets; excused where the oracle score is
    within BAND of the oracle k-th value.  Returns (n_diff, n_excused)."""
    a, b = set(int(x) for x in gpu_idx if x >= 0), set(int(x) for x in oracle_idx)
    sd = a ^ b
    exc = sum(1 for j in sd if abs(scores[j] - kth) <= BAND)
    return len(sd), exc

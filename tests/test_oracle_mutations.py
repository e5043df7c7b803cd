"""Planted mistakes in the oracle must fail at least one pin (CPU only).

Each case swaps one oracle function, inside the pin module's namespace only,
for a copy with a plausible bug (a dropped term, a flipped sign, an off-by-one
index, a transposed operand, a wrong tie rule) and runs the pins that should
catch it.  Nothing here touches the GPU or the HIP library.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import attention as att
from oracle import blocks as blk
from oracle import quality as qual
from tests import test_oracle_facts as pins


def _rescue_sign_flipped(qbar, c, r, p_c, p_r, band_blocks=0, sink_blocks=0):
    return blk.select_blocks(qbar, c, -np.asarray(r), p_c, p_r, band_blocks, sink_blocks)


def _radius_is_mean_distance(k, T):
    c, _ = blk.block_stats(k, T)
    k = np.asarray(k, dtype=np.float64)
    r = np.array([np.linalg.norm(k[j * T:(j + 1) * T] - c[j], axis=1).mean() for j in range(c.shape[0])])
    return c, r


def _dense_off_by_one(q, k, v, scale, causal=True):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    o = np.zeros((q.shape[0], v.shape[1])); lse = np.zeros(q.shape[0])
    for t in range(q.shape[0]):
        n = max(1, t) if causal else k.shape[0]
        o[t], lse[t] = att._softmax_row(scale * (k[:n] @ q[t]), v[:n])
    return o, lse


def _topk_ties_high(scores, k):
    s = np.asarray(scores, dtype=np.float64)
    order = np.lexsort((-np.arange(s.size), -s))
    return np.sort(order[:k]), s[order[k - 1]]


def _combine_drops_l(parts):
    return oracle.lse_combine([(m, 1.0 if l > 0 else 0.0, o) for m, l, o in parts])


def _gather_ignores_table(pool, page_table, seq_len, g):
    return oracle.gather_pages(pool, np.arange(len(page_table)), seq_len, g)


def _masked_transposed(q, k, v, mask, T, scale):
    return att.masked_attention(q, k, v, np.asarray(mask).T, T, scale)


def _segments_not_rounded(mode, n, chunk_start=0, chunk_len=2048, local_len=1024, n_sink=4, page=16):
    return oracle.build_segments(mode, n, chunk_start, chunk_len, local_len, n_sink, page=1)


def _neighbourhood_one_sided(mode, n, chunk_start=0, chunk_len=2048, local_len=1024, n_sink=4,
                             page=16, min_nb=0):
    # widens the focus chunk after it, not before it
    return oracle.build_segments(mode, n, chunk_start, chunk_len + min_nb, local_len, n_sink, page)


def _pooled_by_mean(scores, k):
    return oracle.topk(np.asarray(scores, dtype=np.float64).mean(axis=0), k)


def _pool_uses_first_row(q, T):
    q = np.asarray(q, dtype=np.float64)
    return q[::T].copy()


def _mass_without_causality(q, k, T, scale, rows=None):
    q, k = np.asarray(q, dtype=np.float64), np.asarray(k, dtype=np.float64)
    rows = range(q.shape[0] // T) if rows is None else rows
    out = {}
    for i in rows:
        s = scale * (q[i * T:(i + 1) * T] @ k[:(i + 1) * T].T)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out[i] = p.reshape(T, i + 1, T).sum(axis=2)
    return out


def _retention_of_complement(q, k, mask, T, scale, rows=None):
    mass = qual.token_block_mass(q, k, T, scale, rows)
    mask = np.asarray(mask, dtype=bool)
    return {i: m[:, ~mask[i, :i + 1]].sum(axis=1) for i, m in mass.items()}


def _ideal_keeps_least(q, k, T, scale, counts, rows):
    mass = qual.token_block_mass(q, k, T, scale, rows)
    out = {}
    for i, m in mass.items():
        keep = np.sort(np.argsort(m.mean(axis=0), kind="stable")[:counts[i]])
        out[i] = (keep, m[:, keep].sum(axis=1))
    return out


def _kv_head_interleaved(h, Hq, Hkv):
    return h % Hkv


def _scores_drop_last_coordinate(q, kseq):
    q = np.asarray(q, dtype=np.float64)
    kseq = np.asarray(kseq, dtype=np.float64)
    return kseq[:, :-1] @ q[:-1]


def _scores_sign_flipped(q, kseq):
    return -(np.asarray(kseq, dtype=np.float64) @ np.asarray(q, dtype=np.float64))


def _union_keeps_intersection(sets):
    keep = None
    for s in sets:
        x = {int(v) for v in np.asarray(s).ravel() if v >= 0}
        keep = x if keep is None else keep & x
    return np.array(sorted(keep), dtype=np.int64)


def _recall_over_shared(own, shared):
    own = {int(x) for x in np.asarray(own).ravel() if x >= 0}
    shared = {int(x) for x in np.asarray(shared).ravel() if x >= 0}
    return len(own & shared) / len(shared)


def _mass_renormalised_over_set(q, kseq, idx, scale):
    q, kseq = np.asarray(q, dtype=np.float64), np.asarray(kseq, dtype=np.float64)
    idx = np.unique(np.asarray(idx, dtype=np.int64))
    idx = idx[idx >= 0]
    s = scale * (kseq[idx] @ q)
    p = np.exp(s - s.max())
    return float((p / p.sum()).sum())


CASES = [
    ("select_blocks", _rescue_sign_flipped,
     [pins.test_F4_planted_spike_dropped_by_centroid_recovered_by_rescue]),
    ("block_stats", _radius_is_mean_distance,
     [lambda: pins.test_F3_rescue_bound_never_below_block_max(8, 8)]),
    ("dense_attention", _dense_off_by_one,
     [lambda: pins.test_F1_all_blocks_mask_is_dense_causal(8, 4, 2)]),
    ("topk", _topk_ties_high, [pins.test_F6_topk_special_cases_and_brute_force]),
    ("lse_combine", _combine_drops_l, [pins.test_F9_lse_combine_partition_invariant]),
    ("gather_pages", _gather_ignores_table, [pins.test_F10_paged_gather_identity_vs_shuffled]),
    ("masked_attention", _masked_transposed, [pins.test_masked_attention_equals_sdpa_with_explicit_mask]),
    ("build_segments", _segments_not_rounded, [pins.test_F8_golden_focus_segments]),
    ("build_segments", _neighbourhood_one_sided,
     [lambda: pins.test_F8_focus_minimum_neighbourhood(5000, 100)]),
    ("pool_queries", _pool_uses_first_row, [pins.test_F5_pool_queries_block_means]),
    ("topk_pooled", _pooled_by_mean, [pins.test_topk_pooled_closed_forms_and_brute_force]),
    ("token_block_mass", _mass_without_causality,
     [pins.test_Q2_block_mass_brute_force_and_library_softmax]),
    ("retention", _retention_of_complement,
     [pins.test_Q1_full_mask_retains_everything_and_complement_sums_to_one]),
    ("ideal_rows", _ideal_keeps_least, [pins.test_Q3_ideal_rows_brute_force_over_block_subsets]),
    ("kv_head", _kv_head_interleaved, [pins.test_kv_head_matches_library_gqa_attention]),
    ("anchor_scores", _scores_drop_last_coordinate,
     [pins.test_anchor_scores_closed_forms_brute_force_and_library_softmax]),
    ("anchor_scores", _scores_sign_flipped,
     [pins.test_anchor_scores_closed_forms_brute_force_and_library_softmax]),
    ("union_sets", _union_keeps_intersection, [pins.test_union_sets_brute_force_and_closed_forms]),
    ("set_recall", _recall_over_shared, [pins.test_set_recall_closed_forms]),
    ("index_mass", _mass_renormalised_over_set,
     [pins.test_index_mass_full_set_complement_and_library_weights]),
]


@pytest.mark.parametrize("name,mutant,catchers", CASES, ids=[c[1].__name__.strip("_") for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, catchers):
    monkeypatch.setattr(pins, name, mutant)
    caught = False
    for fn in catchers:
        try:
            fn()
        except AssertionError:
            caught = True
    assert caught, f"no pin caught a planted mistake in {name}"

"""Pins of the fp64 oracle against facts fixed by the mathematics and by the
source pages' definitions (runs on the CPU, no GPU, no HIP library).

Each test names the fact it checks.  A pin never re-types the oracle's own
formula: it uses a closed form, a brute-force enumeration, a library routine
(torch's CPU scaled_dot_product_attention, numpy sort / argpartition) or an
invariant that a dropped term, a wrong sign or index or a transposed operand
would break.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (anchor_scores, anchor_topk, block_stats, build_segments, dense_attention,
                    gather_pages, ideal_rows, index_attention, index_mass, kv_head, lse_combine,
                    masked_attention, pool_queries, retention, segment_attention, select_blocks,
                    set_recall, token_block_mass, topk, topk_pooled, union_sets)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _sdpa(q, k, v, scale, causal):
    """torch CPU float64 scaled_dot_product_attention on one head."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), is_causal=causal, scale=scale)
    return o[0, 0].numpy()


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- F1 -------
@pytest.mark.parametrize("S,D,T", [(8, 4, 2), (256, 64, 64), (320, 32, 64)])
def test_F1_all_blocks_mask_is_dense_causal(S, D, T):
    rng = _rng(S + D)
    q, k, v = (rng.standard_normal((S, D)) for _ in range(3))
    scale = 1 / math.sqrt(D)
    nB = S // T
    full = np.tril(np.ones((nB, nB), dtype=bool))
    om, lm = masked_attention(q, k, v, full, T, scale)
    od, ld = dense_attention(q, k, v, scale, causal=True)
    assert np.abs(om - od).max() <= 1e-12
    assert np.abs(lm - ld).max() <= 1e-12
    ref = _sdpa(q, k, v, scale, causal=True)
    assert np.abs(od - ref).max() <= 1e-12
    # the selector with p_c = 1 keeps every visible block
    c, r = block_stats(k, T)
    sel = select_blocks(pool_queries(q, T), c, r, 1.0, 0.1)
    assert (sel["M"] == full).all()


def test_F1_lse_matches_logsumexp():
    rng = _rng(3)
    q, k, v = (rng.standard_normal((16, 8)) for _ in range(3))
    _, lse = dense_attention(q, k, v, 0.5, causal=True)
    for t in range(16):
        ref = torch.logsumexp(torch.from_numpy(0.5 * (k[:t + 1] @ q[t])), 0).item()
        assert abs(lse[t] - ref) <= 1e-12


# ---------------------------------------------------------------- F2 -------
def test_F2_zero_query_gives_mean_of_visible_values():
    rng = _rng(5)
    S, D = 64, 16
    k, v = rng.standard_normal((S, D)), rng.standard_normal((S, D))
    o, lse = dense_attention(np.zeros((S, D)), k, v, 0.3, causal=True)
    for t in range(S):
        assert np.abs(o[t] - v[:t + 1].sum(0) / (t + 1)).max() <= 1e-12
        assert abs(lse[t] - math.log(t + 1)) <= 1e-12


def test_F2_first_row_and_dominant_key():
    rng = _rng(6)
    S, D = 32, 8
    q, k, v = (rng.standard_normal((S, D)) for _ in range(3))
    o, _ = dense_attention(q, k, v, 1.0, causal=True)
    assert np.abs(o[0] - v[0]).max() <= 1e-15
    # one key with a +50 logit margin over all others takes all the weight
    qq = np.zeros(D); qq[0] = 1.0
    kk = np.zeros((S, D)); kk[17, 0] = 50.0
    oo, _ = index_attention(qq, kk, v, np.arange(S), 1.0)
    # every other weight is below e^-50, so the error is below 2 S e^-50 max|v|
    assert np.abs(oo - v[17]).max() <= 2 * S * math.exp(-50) * np.abs(v).max()


def test_F2_golden_two_key_softmax():
    g = _gold("two_key_softmax.json")
    o, lse = index_attention(g["q"], g["k"], g["v"], [0, 1], g["scale"])
    assert np.abs(o - np.array(g["o"])).max() <= 1e-15
    assert abs(lse - g["lse"]) <= 1e-15


# ---------------------------------------------------------------- F3 -------
@pytest.mark.parametrize("D", [2, 4, 8, 64])
@pytest.mark.parametrize("T", [1, 2, 8, 64])
def test_F3_rescue_bound_never_below_block_max(D, T):
    rng = _rng(100 * D + T)
    for trial in range(10000 // (D * T) + 20):
        keys = rng.standard_normal((T, D)) * rng.uniform(0.1, 3.0)
        queries = rng.standard_normal((T, D))
        c, r = block_stats(keys, T)
        for qv in (queries[0], pool_queries(queries, T)[0]):
            sc = float(qv @ c[0])
            sr = sc + np.linalg.norm(qv) * r[0]
            true_max = (keys @ qv).max()
            assert sr >= true_max - 1e-12
            if T == 1:
                assert abs(sr - true_max) <= 1e-12


def test_F3_bound_is_tight_when_farthest_key_lies_along_query():
    # keys c + u and c - u with u parallel to q: max q.k = q.c + ||q|| ||u||
    D = 6
    rng = _rng(9)
    cvec = rng.standard_normal(D)
    qv = rng.standard_normal(D)
    u = 0.7 * qv / np.linalg.norm(qv)
    keys = np.stack([cvec + u, cvec - u])
    c, r = block_stats(keys, 2)
    sr = qv @ c[0] + np.linalg.norm(qv) * r[0]
    assert abs(sr - (keys @ qv).max()) <= 1e-12


# ---------------------------------------------------------------- F4 -------
def _spike_fixture(seed=0):
    """One query block of 8 queries all equal to 3 e1, 8 visible key blocks."""
    D = T = 8
    rng = _rng(seed)
    e = np.eye(D)
    blocks = []
    for j in range(8):
        if j in (1, 4):                   # decoys: e1 + small noise orthogonal to e1
            nz = 0.05 * rng.standard_normal((T, D)); nz[:, 0] = 0
            blocks.append(e[0] + nz)
        elif j == 6:                      # spike block: one key 6 e1, seven keys e2..e8
            blocks.append(np.vstack([6 * e[0], e[1:]]))
        else:
            blocks.append(0.1 * rng.standard_normal((T, D)))
    k = np.vstack(blocks)
    q = np.tile(3 * e[0], (8 * T, 1))
    return q, k, T


def test_F4_planted_spike_dropped_by_centroid_recovered_by_rescue():
    g = _gold("planted_spike.json")
    q, k, T = _spike_fixture()
    c, r = block_stats(k, T)
    qbar = pool_queries(q, T)
    assert abs(r[6] - g["spike_r"]) <= 1e-12
    sel = select_blocks(qbar, c, r, 0.25, 0.10)
    i = 7
    assert abs(sel["Sc"][i, 6] - g["spike_Sc"]) <= 1e-12
    assert abs(sel["Sr"][i, 6] - g["spike_Sr"]) <= 1e-12
    assert abs(sel["Sc"][i, 1] - g["decoy_Sc"]) <= 1e-12
    assert (k[6 * T:7 * T] @ qbar[i]).max() == g["spike_true_max"]
    assert sel["k_c"][i] == 2 and sel["k_r"][i] == 1
    assert set(np.flatnonzero(sel["C"][i])) == {1, 4}       # centroid branch: decoys only
    assert set(np.flatnonzero(sel["R"][i])) == {6}          # rescue branch: the spike block
    assert set(np.flatnonzero(sel["M"][i])) == {1, 4, 6}


# ---------------------------------------------------------------- F5 -------
def test_F5_block_stat_closed_forms():
    rng = _rng(11)
    key = rng.integers(-64, 64, 16) / 8.0     # dyadic: the block sum is exact
    c, r = block_stats(np.tile(key, (8, 1)), 8)
    assert np.abs(c[0] - key).max() <= 1e-15 and r[0] == 0.0
    cen, u = rng.standard_normal(16), rng.standard_normal(16)
    c, r = block_stats(np.stack([cen + u, cen - u]), 2)
    assert np.abs(c[0] - cen).max() <= 1e-14
    assert abs(r[0] - np.linalg.norm(u)) <= 1e-14
    # blocks are independent and ordered: block j sees rows j*T..j*T+T-1
    ks = np.concatenate([np.full((4, 3), j, dtype=np.float64) for j in range(5)])
    c, r = block_stats(ks, 4)
    assert (c[:, 0] == np.arange(5)).all() and (r == 0).all()


def test_F5_pool_queries_block_means():
    q = np.arange(24, dtype=np.float64).reshape(6, 4)
    p = pool_queries(q, 3)
    assert (p[0] == q[1]).all() and (p[1] == q[4]).all()  # mean of an arithmetic run is its middle


# ---------------------------------------------------------------- F6 -------
def _rank_topk(s, k):
    """Brute force: keep j iff fewer than k entries beat it, where i beats j
    when s_i > s_j or (s_i == s_j and i < j)."""
    n = len(s)
    keep = [j for j in range(n)
            if sum(1 for i in range(n) if s[i] > s[j] or (s[i] == s[j] and i < j)) < k]
    return np.array(keep)


def test_F6_topk_special_cases_and_brute_force():
    rng = _rng(12)
    s = rng.standard_normal(50)
    idx, kth = topk(s, 50)
    assert (idx == np.arange(50)).all() and kth == s.min()
    idx, kth = topk(s, 1)
    assert idx.tolist() == [int(np.argmax(s))] and kth == s.max()
    for k in (3, 7, 20):
        idx, kth = topk(s, k)
        assert (idx == np.sort(np.argpartition(-s, k - 1)[:k])).all()
        assert (idx == _rank_topk(s, k)).all()
        assert kth == np.sort(s)[::-1][k - 1]
    # duplicated scores: lower indices win
    d = np.array([1.0, 5.0, 3.0, 5.0, 3.0, 3.0, 0.0])
    assert topk(d, 3)[0].tolist() == [1, 2, 3]
    assert topk(d, 4)[0].tolist() == [1, 2, 3, 4]
    for k in range(1, 8):
        assert (topk(d, k)[0] == _rank_topk(d, k)).all()
    with pytest.raises(ValueError):
        topk(d, 0)


def test_F6_selector_branches_match_brute_force_rank():
    rng = _rng(13)
    nB, D, T = 12, 5, 3
    q = rng.standard_normal((nB * T, D))
    k = rng.standard_normal((nB * T, D))
    c, r = block_stats(k, T)
    qbar = pool_queries(q, T)
    sel = select_blocks(qbar, c, r, 0.3, 0.2, band_blocks=2, sink_blocks=1)
    for i in range(nB):
        n = i + 1
        sc = np.array([qbar[i] @ c[j] for j in range(n)])
        sr = sc + math.sqrt(qbar[i] @ qbar[i]) * r[:n]
        kc = max(1, math.ceil(0.3 * n)); kr = max(1, math.ceil(0.2 * n))
        assert set(np.flatnonzero(sel["C"][i])) == set(_rank_topk(sc, kc).tolist())
        assert set(np.flatnonzero(sel["R"][i])) == set(_rank_topk(sr, kr).tolist())
        forced = {0} | {j for j in range(max(0, i - 1), n)}
        want = set(_rank_topk(sc, kc).tolist()) | set(_rank_topk(sr, kr).tolist()) | forced
        assert set(np.flatnonzero(sel["M"][i])) == want
        assert not sel["M"][i, n:].any()


def test_F6_k_of_closed_values():
    assert oracle.k_of(0.25, 16) == 4
    assert oracle.k_of(0.25, 1) == 1
    assert oracle.k_of(0.1, 10) == 1
    assert oracle.k_of(0.1, 11) == 2
    assert oracle.k_of(0.0, 9) == 1
    assert oracle.k_of(1.5, 9) == 9
    assert oracle.k_of(-1.0, 9) == 0


# ---------------------------------------------------------------- F7 -------
def test_F7_index_attention_full_index_set_is_dense_decode():
    rng = _rng(14)
    N, D = 300, 32
    q = rng.standard_normal(D)
    k, v = rng.standard_normal((N, D)), rng.standard_normal((N, D))
    o, lse = index_attention(q, k, v, np.arange(N), 0.2)
    ref = _sdpa(q[None], k, v, 0.2, causal=False)[0]
    assert np.abs(o - ref).max() <= 1e-12
    assert abs(lse - torch.logsumexp(torch.from_numpy(0.2 * (k @ q)), 0).item()) <= 1e-12
    # order of the index list does not matter; -1 slots are skipped
    perm = rng.permutation(N)
    o2, _ = index_attention(q, k, v, np.concatenate([perm, [-1, -1]]), 0.2)
    assert np.abs(o2 - o).max() <= 1e-12


# ---------------------------------------------------------------- F8 -------
def test_F8_segment_modes():
    rng = _rng(15)
    n, D = 3000, 16
    q = rng.standard_normal(D)
    k, v = rng.standard_normal((n, D)), rng.standard_normal((n, D))
    og, _ = segment_attention(q, k, v, build_segments(oracle.SEG_GLOBAL, n), 0.25)
    ref = _sdpa(q[None], k, v, 0.25, causal=False)[0]
    assert np.abs(og - ref).max() <= 1e-12
    loc = build_segments(oracle.SEG_LOCAL, 3008, local_len=1024)
    assert loc == [(3008 - 1024, 3008)]
    ol, _ = segment_attention(q, k, v, build_segments(oracle.SEG_LOCAL, n, local_len=1024), 0.25)
    ref_l = _sdpa(q[None], k[n - 1024 - 8:], v[n - 1024 - 8:], 0.25, causal=False)[0]  # 3000-1024=1976 -> 1968
    assert np.abs(ol - ref_l).max() <= 1e-12
    st = build_segments(oracle.SEG_STREAMING, n, local_len=1024, n_sink=4)
    assert st == [(0, 4), (n - 1024, n)]


@pytest.mark.parametrize("start", [0, 1, 15, 16, 17, 1000, 2048 * 7 + 3, 100000 - 2048])
def test_F8_focus_ranges_page_aligned_and_tight(start):
    n, L, P = 100000, 2048, 16
    rs = build_segments(oracle.SEG_FOCUS, n, chunk_start=start, chunk_len=L, local_len=1024, page=P)
    covered = np.zeros(n, dtype=bool)
    for a, b in rs:
        assert a % P == 0 and (b % P == 0 or b == n)
        covered[a:b] = True
    assert covered[start:start + L].all() and covered[n - 1024:].all()
    a0 = (start // P) * P
    assert start - a0 <= P - 1
    chunk = [r for r in rs if r[0] <= start < r[1]][0]
    if chunk[1] < n - 1024:
        assert chunk[1] - (start + L) <= P - 1


@pytest.mark.parametrize("start,m", [(5000, 0), (5000, 1), (5000, 100), (7, 300), (0, 64),
                                     (100000 - 2048, 500), (20000, 200000)])
def test_F8_focus_minimum_neighbourhood(start, m):
    """The widened focus range covers [start - m, start + L + m) clipped to
    [0, n), is page-aligned, adds under a page per side beyond it, and m = 0
    gives the plain focus ranges."""
    n, L, P = 100000, 2048, 16
    rs = build_segments(oracle.SEG_FOCUS, n, chunk_start=start, chunk_len=L, local_len=1024,
                        page=P, min_nb=m)
    if m == 0:
        assert rs == build_segments(oracle.SEG_FOCUS, n, start, L, 1024, page=P)
    lo, hi = max(0, start - m), min(n, start + L + m)
    covered = np.zeros(n, dtype=bool)
    for a, b in rs:
        assert a % P == 0 and (b % P == 0 or b == n)
        covered[a:b] = True
    assert covered[lo:hi].all() and covered[n - 1024:].all()
    first = rs[0]
    if first[0] <= lo < first[1]:
        assert lo - first[0] <= P - 1
    chunk = [r for r in rs if r[0] <= lo < r[1]][0]
    if chunk[1] < n - 1024:
        assert chunk[1] - hi <= P - 1
    # ranges stay merged and sorted; the other modes ignore the option
    assert all(rs[x][1] < rs[x + 1][0] for x in range(len(rs) - 1))
    for mode in (oracle.SEG_GLOBAL, oracle.SEG_LOCAL, oracle.SEG_STREAMING):
        assert build_segments(mode, n, start, L, 1024, page=P, min_nb=m) == \
            build_segments(mode, n, start, L, 1024, page=P)


def test_F8_golden_focus_segments():
    g = _gold("focus_segments.json")
    rs = build_segments(oracle.SEG_FOCUS, g["n"], g["chunk_start"], g["chunk_len"],
                        g["local_len"], page=g["page"])
    assert [list(r) for r in rs] == g["ranges"]


# ---------------------------------------------------------------- F9 -------
def test_F9_lse_combine_partition_invariant():
    rng = _rng(16)
    N, D = 200, 8
    q = rng.standard_normal(D) * 2
    k, v = rng.standard_normal((N, D)), rng.standard_normal((N, D))
    o_ref, lse_ref = index_attention(q, k, v, np.arange(N), 1.0)
    for trial in range(10):
        perm = rng.permutation(N)
        cuts = np.sort(rng.choice(np.arange(1, N), size=rng.integers(1, 9), replace=False))
        parts = [oracle.attention_partial(q, k, v, s, 1.0) for s in np.split(perm, cuts)]
        parts.append(oracle.attention_partial(q, k, v, np.zeros(0, dtype=int), 1.0))  # empty split
        o, lse = lse_combine(parts)
        assert np.abs(o - o_ref).max() <= 1e-12 and abs(lse - lse_ref) <= 1e-12


def test_F9_golden_lse_combine():
    g = _gold("lse_combine.json")
    o, lse = lse_combine([(m, l, np.array(o)) for m, l, o in g["parts"]])
    assert np.abs(o - np.array(g["o"])).max() <= 1e-15 and abs(lse - g["lse"]) <= 1e-15


# ---------------------------------------------------------------- F10 ------
def test_F10_paged_gather_identity_vs_shuffled():
    rng = _rng(17)
    P, Hkv, D, n_pages = 16, 3, 8, 40
    seq = rng.standard_normal((n_pages * P, Hkv, D))
    ident = seq.reshape(n_pages, P, Hkv, D).transpose(0, 2, 1, 3).copy()
    perm = rng.permutation(n_pages)
    shuf = np.zeros_like(ident)
    shuf[perm] = ident                 # logical page p is stored at physical perm[p]
    for g in range(Hkv):
        for n in (1, 17, 300, n_pages * P):
            a = gather_pages(ident, np.arange(n_pages), n, g)
            b = gather_pages(shuf, perm, n, g)
            assert (a == b).all() and (a == seq[:n, g]).all()


# ---------------------------------------------------------------- F11 ------
def test_F11_density_bookkeeping():
    rng = _rng(18)
    nB, T, D = 20, 4, 6
    q, k = rng.standard_normal((nB * T, D)), rng.standard_normal((nB * T, D))
    c, r = block_stats(k, T)
    sel = select_blocks(pool_queries(q, T), c, r, 0.2, 0.08)
    M = sel["M"]
    executed = sum(int(M[i, j]) for i in range(nB) for j in range(nB))
    assert executed == int(M.sum())
    assert oracle.visible_count(nB) == sum(i + 1 for i in range(nB))
    assert not np.triu(M, 1).any()
    # every row keeps at least one visible block
    assert (M.sum(1) >= 1).all()


# ---------------------------------------------------------------- F12 ------
def test_F12_causality():
    rng = _rng(19)
    S, D, T = 96, 8, 16
    q, k, v = (rng.standard_normal((S, D)) for _ in range(3))
    mask = rng.random((S // T, S // T)) < 0.5
    np.fill_diagonal(mask, True)
    o1, _ = masked_attention(q, k, v, mask, T, 0.4)
    t = 37
    k2, v2 = k.copy(), v.copy()
    k2[t + 1:] = rng.standard_normal((S - t - 1, D))
    v2[t + 1:] = rng.standard_normal((S - t - 1, D))
    o2, _ = masked_attention(q, k2, v2, mask, T, 0.4)
    assert (o1[:t + 1] == o2[:t + 1]).all()
    assert np.abs(o1[t + 1:] - o2[t + 1:]).max() > 1e-3


def test_masked_attention_equals_sdpa_with_explicit_mask():
    """Block mask expanded to a token mask, run through the library routine."""
    rng = _rng(20)
    S, D, T = 128, 16, 16
    q, k, v = (rng.standard_normal((S, D)) for _ in range(3))
    mask = rng.random((S // T, S // T)) < 0.4
    np.fill_diagonal(mask, True)
    o, _ = masked_attention(q, k, v, mask, T, 0.25)
    tok = np.kron(mask, np.ones((T, T), dtype=bool)) & np.tril(np.ones((S, S), dtype=bool))
    t = lambda x: torch.from_numpy(x)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.from_numpy(tok)[None, None], scale=0.25)[0, 0].numpy()
    assert np.abs(o - ref).max() <= 1e-12


# ------------------------------------------------- forced-only (SSA) mask ---
@pytest.mark.parametrize("band,sink", [(8, 1), (2, 0), (1, 3), (40, 1)])
def test_forced_only_mask_is_window_plus_sink(band, sink):
    """Both branches off (p < 0): the mask is exactly the forced blocks (LoZA
    post, "2. ZigZag architecture": streaming sparse attention over a fixed
    window, here a band of key blocks plus sink blocks), and attention over it
    equals a token-level window-plus-sink mask run through the library routine."""
    rng = _rng(band * 7 + sink)
    S, D, T = 320, 16, 16
    nB = S // T
    q, k, v = (rng.standard_normal((S, D)) for _ in range(3))
    qbar = oracle.pool_queries(q, T)
    c, r = oracle.block_stats(k, T)
    sel = oracle.select_blocks(qbar, c, r, -1.0, -1.0, band, sink)
    i, j = np.meshgrid(np.arange(nB), np.arange(nB), indexing="ij")
    want = (j <= i) & ((j < sink) | (j > i - band))
    assert (sel["M"] == want).all() and not sel["C"].any() and not sel["R"].any()
    o, _ = masked_attention(q, k, v, sel["M"], T, 0.25)
    ti, tj = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    tok = (tj <= ti) & ((tj // T < sink) | (tj // T > ti // T - band))
    t = lambda x: torch.from_numpy(x)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.from_numpy(tok)[None, None], scale=0.25)[0, 0].numpy()
    assert np.abs(o - ref).max() <= 1e-12


# --------------------------------------------------- pooled (per-KV-head) top-k
def test_topk_pooled_closed_forms_and_brute_force():
    """G = 1 is plain top-k; a key that is the single best for one head only is
    kept; the result equals brute-force rank counting on the per-key max; ties
    go to the lower index; k = N keeps every key."""
    rng = _rng(31)
    G, N = 4, 300
    s = rng.standard_normal((G, N))
    for k in (1, 7, 64, N):
        idx, kth = topk_pooled(s[:1], k)
        ref_idx, ref_kth = oracle.topk(s[0], k)
        assert (idx == ref_idx).all() and kth == ref_kth
    star = s.copy()
    star[2, 123] = 50.0  # only head 2 rates key 123
    idx, kth = topk_pooled(star, 1)
    assert list(idx) == [123] and kth == 50.0
    m = s.max(axis=0)
    for k in (5, 40, 299):
        idx, kth = topk_pooled(s, k)
        rank = np.array([(m > m[j]).sum() + (m[:j] == m[j]).sum() for j in range(N)])
        assert list(idx) == list(np.flatnonzero(rank < k)) and kth == np.sort(m)[::-1][k - 1]
    tie = np.zeros((G, 10))
    tie[1, [3, 7]] = 1.0
    assert list(topk_pooled(tie, 3)[0]) == [0, 3, 7]
    assert list(topk_pooled(s, N)[0]) == list(range(N))


# ---- selector quality (RBS-Attention post, "Experimental data": actual
# retention, selectors compared at matched density)

def _mass_brute_force(q, k, T, scale, i):
    """Per-query softmax mass on each visible key block, with scalar loops
    and math.exp (no vectorised softmax)."""
    out = np.zeros((T, i + 1))
    for a in range(T):
        t = i * T + a
        s = [scale * float(np.dot(q[t], k[u])) for u in range(t + 1)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        tot = sum(w)
        for u in range(t + 1):
            out[a, u // T] += w[u] / tot
    return out


def test_Q1_full_mask_retains_everything_and_complement_sums_to_one():
    """Every visible block admitted -> retention 1 (the softmax sums to 1); a
    mask and its complement within the visible blocks split the mass."""
    rng = _rng(21)
    S, D, T = 48, 8, 4
    q, k = rng.standard_normal((S, D)), rng.standard_normal((S, D))
    nB = S // T
    full = np.tril(np.ones((nB, nB), dtype=bool))
    for i, r in retention(q, k, full, T, 0.5).items():
        assert np.abs(r - 1.0).max() < 1e-12
    half = full & (rng.random((nB, nB)) < 0.5)
    r1 = retention(q, k, half, T, 0.5)
    r2 = retention(q, k, full & ~half, T, 0.5)
    for i in range(nB):
        assert np.abs(r1[i] + r2[i] - 1.0).max() < 1e-12
        assert (r1[i] >= 0).all() and (r1[i] <= 1 + 1e-12).all()


def test_Q2_block_mass_brute_force_and_library_softmax():
    """Block masses equal scalar-loop softmax sums, and torch's causal softmax
    summed per block; a T = 1 diagonal-only mask keeps exactly each token's
    weight on itself."""
    rng = _rng(22)
    S, D, T, scale = 24, 6, 3, 0.7
    q, k = rng.standard_normal((S, D)), rng.standard_normal((S, D))
    mass = token_block_mass(q, k, T, scale)
    sc = torch.from_numpy(scale * q @ k.T)
    sc = sc.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), -math.inf)
    p = torch.softmax(sc, dim=1).numpy()
    for i in range(S // T):
        assert np.abs(mass[i] - _mass_brute_force(q, k, T, scale, i)).max() < 1e-12
        lib = p[i * T:(i + 1) * T, :(i + 1) * T].reshape(T, i + 1, T).sum(axis=2)
        assert np.abs(mass[i] - lib).max() < 1e-12
    diag = np.eye(S, dtype=bool)
    r = retention(q, k, diag, 1, scale)
    assert np.abs(np.array([r[t][0] for t in range(S)]) - np.diag(p)).max() < 1e-12


def test_Q3_ideal_rows_brute_force_over_block_subsets():
    """The ideal set at count c is the c-subset of visible blocks with the
    largest mean retention (checked against every subset)."""
    import itertools
    rng = _rng(23)
    S, D, T = 28, 5, 4
    q, k = 2 * rng.standard_normal((S, D)), rng.standard_normal((S, D))
    nB = S // T
    counts = {i: 1 + (i * 3) % (i + 1) for i in range(nB)}
    ideal = ideal_rows(q, k, T, 0.9, counts, range(nB))
    for i in range(nB):
        best, best_set = -1.0, None
        for sub in itertools.combinations(range(i + 1), counts[i]):
            m = np.zeros((nB, nB), dtype=bool)
            m[i, list(sub)] = True
            val = retention(q, k, m, T, 0.9, rows=[i])[i].mean()
            if val > best + 1e-12:
                best, best_set = val, sub
        blocks, ret = ideal[i]
        assert tuple(blocks) == best_set
        assert abs(ret.mean() - best) < 1e-12


# ---- anchor-layer scores and the GQA head mapping (Kascade post, "What
# Kascade got right": the anchor scores every cached key; "Head-aware is the
# key to accuracy": per attention head)

def test_kv_head_matches_library_gqa_attention():
    """Query heads attending through kv_head equal torch's grouped-query SDPA
    (enable_gqa: consecutive query heads share a KV head), which a mapping
    h % Hkv (interleaved heads) or any other grouping would break."""
    rng = _rng(41)
    Hq, Hkv, N, D = 8, 2, 11, 4
    q = rng.standard_normal((Hq, D))
    k = rng.standard_normal((Hkv, N, D))
    v = rng.standard_normal((Hkv, N, 3))
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None]
    lib = torch.nn.functional.scaled_dot_product_attention(
        t(q[:, None, :]), t(k), t(v), scale=0.5, enable_gqa=True)[0, :, 0].numpy()
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        o, _ = index_attention(q[h], k[g], v[g], np.arange(N), 0.5)
        assert np.abs(o - lib[h]).max() <= 1e-12
    assert [kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [kv_head(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]
    with pytest.raises(ValueError):
        kv_head(0, 6, 4)


def test_anchor_scores_closed_forms_brute_force_and_library_softmax():
    """Basis keys read the query's coordinates back; scores equal scalar
    math.fsum dot products; their softmax equals torch SDPA with identity
    values (the attention weights themselves), which a dropped coordinate, a
    flipped sign or a transposed operand would break."""
    rng = _rng(42)
    D, N = 6, 9
    q = rng.standard_normal(D)
    basis = np.zeros((N, D))
    for j in range(N):
        basis[j, j % D] = j + 1.0
    s = anchor_scores(q, basis)
    assert np.array_equal(s, np.array([(j + 1.0) * q[j % D] for j in range(N)]))
    K = rng.standard_normal((N, D))
    s = anchor_scores(q, K)
    for j in range(N):
        assert abs(s[j] - math.fsum(q[d] * K[j, d] for d in range(D))) <= 1e-14
    w = _sdpa(q[None], K, np.eye(N), 0.8, causal=False)[0]
    p = np.exp(0.8 * s - (0.8 * s).max())
    assert np.abs(p / p.sum() - w).max() <= 1e-13
    idx, kth = anchor_topk(q, K, 3)
    assert list(idx) == sorted(np.argsort(-s, kind="stable")[:3].tolist())
    assert kth == np.sort(s)[-3]


# ---- GQA-shared index sets (Kascade post, "Head-aware is the key to
# accuracy": per-head sets versus one set shared by a KV head's query heads)

def test_union_sets_brute_force_and_closed_forms():
    rng = _rng(43)
    sets = [np.sort(rng.choice(200, 30, replace=False)) for _ in range(4)]
    u = union_sets(sets)
    want = set()
    for x in sets:
        want |= set(x.tolist())
    assert u.tolist() == sorted(want)
    assert (np.diff(u) > 0).all()
    for x in sets:
        assert set(x.tolist()) <= set(u.tolist())
    assert union_sets([np.arange(5), np.arange(5, 9)]).tolist() == list(range(9))
    assert union_sets([np.arange(5), np.arange(5)]).tolist() == list(range(5))
    assert union_sets([np.array([3, -1, -1]), np.array([-1, 2, -1])]).tolist() == [2, 3]


def test_set_recall_closed_forms():
    assert set_recall(np.arange(10), np.arange(20)) == 1.0
    assert set_recall(np.arange(10), np.arange(10, 20)) == 0.0
    assert set_recall(np.arange(10), np.arange(5, 15)) == 0.5
    assert set_recall(np.array([0, 1, -1, -1]), np.array([1, 7])) == 0.5
    with pytest.raises(ValueError):
        set_recall(np.array([-1, -1]), np.arange(3))


def test_index_mass_full_set_complement_and_library_weights():
    """Every key listed -> mass 1; a set and its complement split the mass;
    the mass equals torch SDPA's attention weights (identity values) summed
    over the set; duplicates and empty slots do not count twice."""
    rng = _rng(44)
    N, D, scale = 40, 8, 0.6
    q, K = rng.standard_normal(D), rng.standard_normal((N, D))
    assert abs(index_mass(q, K, np.arange(N), scale) - 1.0) <= 1e-12
    sel = np.sort(rng.choice(N, 13, replace=False))
    rest = np.setdiff1d(np.arange(N), sel)
    assert abs(index_mass(q, K, sel, scale) + index_mass(q, K, rest, scale) - 1.0) <= 1e-12
    w = _sdpa(q[None], K, np.eye(N), scale, causal=False)[0]
    assert abs(index_mass(q, K, sel, scale) - w[sel].sum()) <= 1e-12
    dup = np.concatenate([sel, sel[:4], [-1, -1]])
    assert abs(index_mass(q, K, dup, scale) - w[sel].sum()) <= 1e-12

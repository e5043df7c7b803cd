"""GPU parity of the decode path (topk_indices, topk_indices_kv, sparse_decode_attn
in index, per-KV-head index, segment and all modes) against the fp64 oracle,
through the C ABI.

The paged pools are shuffled, sequences are ragged (one shorter than k, one
not a multiple of the page size), split counts vary (1, odd, automatic), and
every (head dim, group size) pair the kernels are built for is covered:
D = 64 and 128 with 1, 2, 4 and 8 query heads per KV head.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._parity import TOL_BF16, topk_diff_excused

pytestmark = pytest.mark.gpu

SHAPES = {
    # name: (B, N, Hq, Hkv, D, seq_lens, k)
    "gqa4_d128": (3, 8192, 8, 2, 128, [8192, 5003, 100], 256),
    "gqa8_d64": (2, 4096, 8, 1, 64, [4096, 2048 + 7], 128),
    # the other group sizes the kernels are built for: one query head per KV
    # head, and pairs
    "mha_d128": (2, 4096, 4, 4, 128, [4096, 1500], 64),
    "gqa2_d64": (2, 4096, 4, 2, 64, [3000, 4096], 128),
    # ... and the remaining (head dim, group size) pairs the kernels are built for
    "mha_d64": (2, 2048, 2, 2, 64, [2048, 999], 64),
    "gqa2_d128": (2, 2048, 4, 2, 128, [2048, 1040], 64),
    "gqa4_d64": (2, 2048, 8, 2, 64, [1500, 2048], 64),
    "gqa8_d128": (2, 2048, 16, 2, 128, [2048, 777], 64),
}

_cache = {}


def inputs(name):
    if name not in _cache:
        B, N, Hq, Hkv, D, sl, k = SHAPES[name]
        print(f"[decode case {name}] B={B} N={N} Hq={Hq} Hkv={Hkv} D={D} k={k}", flush=True)
        d = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=2, seq_lens=sl, seed=77,
                                    device="cpu")
        gpu = {"page_table": d["page_table"].cuda(), "seq_lens": d["seq_lens"].cuda(),
               "layers": [{x: t.cuda() for x, t in L.items()} for L in d["layers"]]}
        _cache[name] = (d, gpu)
    return _cache[name]


def seq_kv(d, layer, b, g, n=None):
    n = int(d["seq_lens"][b]) if n is None else n
    pt = d["page_table"][b].numpy()
    K = oracle.gather_pages(workloads.to_f64(d["layers"][layer]["k"]), pt, n, g)
    V = oracle.gather_pages(workloads.to_f64(d["layers"][layer]["v"]), pt, n, g)
    return K, V


@pytest.mark.parametrize("name", list(SHAPES))
def test_topk_parity(name):
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, sl, k = SHAPES[name]
    d, gpu = inputs(name)
    L0 = gpu["layers"][0]
    idx, kth = fsa.topk_indices(L0["q"], L0["k"], gpu["page_table"], gpu["seq_lens"], k,
                                max_seq_len=N)
    idx, kth = idx.cpu().numpy(), kth.cpu().numpy()
    q = workloads.to_f64(d["layers"][0]["q"])
    G = Hq // Hkv
    n_diff = n_exc = 0
    for b in range(B):
        n = sl[b]
        for h in range(Hq):
            row = idx[b, h]
            if n < k:
                assert (row[:n] == np.arange(n)).all() and (row[n:] == -1).all()
                assert np.isneginf(kth[b, h])
                continue
            assert (np.diff(row) > 0).all() and row.min() >= 0 and row.max() < n
            K, _ = seq_kv(d, 0, b, oracle.kv_head(h, Hq, Hkv))
            scores = oracle.anchor_scores(q[b, h], K)
            ref_idx, ref_kth = oracle.topk(scores, k)
            dd, ee = topk_diff_excused(row, ref_idx, scores, ref_kth)
            n_diff += dd
            n_exc += ee
            assert abs(kth[b, h] - ref_kth) <= 1e-3
    print(f"[{name}] top-k entries differing {n_diff}, excused near k-th value {n_exc}")
    assert n_diff == n_exc


def test_topk_k_equals_n_and_k_one():
    import free_sparse_attention_head_amd as fsa
    d, gpu = inputs("gqa4_d128")
    L0 = gpu["layers"][0]
    sl = torch.tensor([3000, 3000, 3000], dtype=torch.int32, device="cuda")
    idx, kth = fsa.topk_indices(L0["q"], L0["k"], gpu["page_table"], sl, 3000, max_seq_len=8192)
    assert (idx.cpu() == torch.arange(3000, dtype=torch.int32)).all()
    idx1, kth1 = fsa.topk_indices(L0["q"], L0["k"], gpu["page_table"], sl, 1, max_seq_len=8192)
    q = workloads.to_f64(d["layers"][0]["q"])
    for b in range(3):
        for h in range(8):
            K, _ = seq_kv(d, 0, b, oracle.kv_head(h, 8, 2), n=3000)
            s = oracle.anchor_scores(q[b, h], K)
            assert abs(kth[b, h].item() - s.min()) <= 1e-3
            assert abs(kth1[b, h].item() - s.max()) <= 1e-3
            am = int(idx1[b, h, 0])
            assert abs(s[am] - s.max()) <= 1e-3


def test_topk_ties_go_to_lower_index():
    """All keys of a sequence identical -> all scores equal (bit-identical on
    the GPU too) -> the k lowest indices, exactly."""
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D = 1, 2048, 4, 1, 128
    d = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=1, seed=3, device="cpu")
    kp = d["layers"][0]["k"].clone()
    kp[:] = kp[0, 0, 0]
    idx, kth = fsa.topk_indices(d["layers"][0]["q"].cuda(), kp.cuda(), d["page_table"].cuda(),
                                d["seq_lens"].cuda(), 100)
    assert (idx.cpu() == torch.arange(100, dtype=torch.int32)).all()
    # half the keys duplicated on the top: positions 1000..1099 get the best key
    kp2 = d["layers"][0]["k"].clone()
    q = d["layers"][0]["q"]
    best = q[0, 0].clone()
    pt = d["page_table"][0]
    for j in range(1000, 1200):
        kp2[pt[j // 16], 0, j % 16] = best
    idx2, _ = fsa.topk_indices(q.cuda(), kp2.cuda(), d["page_table"].cuda(), d["seq_lens"].cuda(), 150)
    assert (idx2.cpu()[0, 0] == torch.arange(1000, 1150, dtype=torch.int32)).all()


def test_topk_many_ties_uses_general_path_exactly():
    """More keys tie in the k-th key's histogram bin than the LDS candidate
    buffer holds (all keys identical, 20000 tokens): the row-rereading path
    must still return exactly the k lowest indices; a second sequence with
    a handful of distinct key values checks the same path against the oracle."""
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, k = 2, 20000, 4, 1, 128, 300
    d = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=1, seed=4, device="cpu")
    kp = d["layers"][0]["k"].clone()
    pt = d["page_table"]
    kp[pt[0].long()] = kp[0, 0, 0].clone()              # sequence 0: one key everywhere
    rng = np.random.default_rng(1)
    vals = kp[pt[1, 0].long(), 0, :3].clone()           # sequence 1: three distinct keys
    for j in range(N):
        kp[pt[1, j // 16], 0, j % 16] = vals[int(rng.integers(0, 3))]
    q = d["layers"][0]["q"]
    idx, kth = fsa.topk_indices(q.cuda(), kp.cuda(), pt.cuda(), d["seq_lens"].cuda(), k)
    idx = idx.cpu().numpy()
    assert (idx[0] == np.arange(k)).all()
    qq = workloads.to_f64(q)
    for h in range(Hq):
        K = oracle.gather_pages(workloads.to_f64(kp), pt[1].numpy(), N, 0)
        ref, _ = oracle.anchor_topk(qq[1, h], K, k)
        assert (idx[1, h] == ref).all()


def test_topk_ties_across_pruned_tiles():
    """Candidate pruning across tiles: the best key is planted in three tiles
    of a 20000-token row (50 copies each, in tiles 0, 5 and 9 of 2048
    tokens), so the k-th key (k = 120) is tied 150 times and its ties
    straddle tiles scored before and after the row's histogram fills up.  The
    index set must be exactly the oracle's (the 120 lowest tied positions),
    per query head and pooled per KV head."""
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, k = 1, 20000, 4, 1, 128, 120
    d = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=1, seed=5, device="cpu")
    kp = d["layers"][0]["k"].clone()
    pt = d["page_table"]
    q = d["layers"][0]["q"].clone()
    q[0, 1:] = q[0, 0]                      # one query for every head: one best key
    best = q[0, 0].clone()
    planted = [j for t in (0, 5, 9) for j in range(t * 2048 + 100, t * 2048 + 150)]
    for j in planted:
        kp[pt[0, j // 16], 0, j % 16] = best
    idx, kth = fsa.topk_indices(q.cuda(), kp.cuda(), pt.cuda(), d["seq_lens"].cuda(), k)
    idxp, _ = fsa.topk_indices_kv(q.cuda(), kp.cuda(), pt.cuda(), d["seq_lens"].cuda(), k)
    K = oracle.gather_pages(workloads.to_f64(kp), pt[0].numpy(), N, 0)
    qq = workloads.to_f64(q)
    ref, _ = oracle.anchor_topk(qq[0, 0], K, k)
    assert list(ref) == planted[:k]
    for h in range(Hq):
        assert (idx[0, h].cpu().numpy() == ref).all()
    assert (idxp[0, 0].cpu().numpy() == ref).all()


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("n_split", [0, 1, 3])
def test_index_decode_parity(name, n_split):
    """Kascade reuse layer: layer 1 attends at layer 0's per-head indices."""
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, sl, k = SHAPES[name]
    d, gpu = inputs(name)
    L0, L1 = gpu["layers"]
    idx, _ = fsa.topk_indices(L0["q"], L0["k"], gpu["page_table"], gpu["seq_lens"], k, max_seq_len=N)
    out, lse = fsa.sparse_decode_attn(L1["q"], L1["k"], L1["v"], gpu["page_table"], gpu["seq_lens"],
                                      mode=fsa.SEL_INDEX, idx=idx, n_split=n_split, max_seq_len=N)
    out, lse, idx = out.cpu(), lse.cpu(), idx.cpu().numpy()
    q1 = workloads.to_f64(d["layers"][1]["q"])
    G = Hq // Hkv
    scale = 1 / math.sqrt(D)
    for b in range(B):
        for h in range(Hq):
            K, V = seq_kv(d, 1, b, oracle.kv_head(h, Hq, Hkv))
            o, l = oracle.index_attention(q1[b, h], K, V, idx[b, h], scale)
            assert np.abs(out[b, h].double().numpy() - o).max() <= TOL_BF16
            assert abs(lse[b, h].item() - l) <= 1e-2


@pytest.mark.parametrize("mode", ["index", "index_kv"])
def test_listed_decode_spans_several_row_batches(mode):
    """One split of 2500 listed positions: the kernel resolves positions to
    pool rows 1024 at a time, so a split crosses three batches (the last one
    ragged).  The list also repeats some positions and holds out-of-range ones
    (skipped)."""
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, k = 2, 6000, 4, 2, 128, 2500
    print(f"[listed decode case {mode}] B={B} N={N} k={k} one split", flush=True)
    d = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=1, seq_lens=[6000, 4000], seed=41,
                                device="cpu")
    rows = Hq if mode == "index" else Hkv
    rng = np.random.default_rng(41)
    idx = rng.integers(0, N, size=(B, rows, k)).astype(np.int32)
    idx[:, :, :7] = -3          # out of range: skipped
    idx[:, :, 7:20] = idx[:, :, 20:33]   # repeated positions count twice
    L = d["layers"][0]
    sel = fsa.SEL_INDEX if mode == "index" else fsa.SEL_INDEX_KV
    out, lse = fsa.sparse_decode_attn(L["q"].cuda(), L["k"].cuda(), L["v"].cuda(),
                                      d["page_table"].cuda(), d["seq_lens"].cuda(), mode=sel,
                                      idx=torch.from_numpy(idx).cuda(), n_split=1)
    out, lse = out.cpu(), lse.cpu()
    q = workloads.to_f64(L["q"])
    G = Hq // Hkv
    for b in range(B):
        n = int(d["seq_lens"][b])
        for h in range(Hq):
            K, V = seq_kv(d, 0, b, oracle.kv_head(h, Hq, Hkv))
            ix = idx[b, h if mode == "index" else oracle.kv_head(h, Hq, Hkv)]
            ix = np.where(ix < n, ix, -1)
            o, l = oracle.index_attention(q[b, h], K, V, ix, 1 / math.sqrt(D))
            assert np.abs(out[b, h].double().numpy() - o).max() <= TOL_BF16
            assert abs(lse[b, h].item() - l) <= 1e-2


@pytest.mark.parametrize("name", list(SHAPES))
def test_topk_kv_parity(name):
    """One index set per KV head from the max over its query heads' scores."""
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, sl, k = SHAPES[name]
    d, gpu = inputs(name)
    L0 = gpu["layers"][0]
    idx, kth = fsa.topk_indices_kv(L0["q"], L0["k"], gpu["page_table"], gpu["seq_lens"], k,
                                   max_seq_len=N)
    assert idx.shape == (B, Hkv, k) and kth.shape == (B, Hkv)
    idx, kth = idx.cpu().numpy(), kth.cpu().numpy()
    q = workloads.to_f64(d["layers"][0]["q"])
    G = Hq // Hkv
    n_diff = n_exc = 0
    for b in range(B):
        n = sl[b]
        for g in range(Hkv):
            row = idx[b, g]
            if n < k:
                assert (row[:n] == np.arange(n)).all() and (row[n:] == -1).all()
                assert np.isneginf(kth[b, g])
                continue
            assert (np.diff(row) > 0).all() and row.min() >= 0 and row.max() < n
            K, _ = seq_kv(d, 0, b, g)
            heads = [h for h in range(Hq) if oracle.kv_head(h, Hq, Hkv) == g]
            scores = np.stack([oracle.anchor_scores(q[b, h], K) for h in heads], axis=1)  # [n, G]
            ref_idx, ref_kth = oracle.topk_pooled(scores.T, k)
            dd, ee = topk_diff_excused(row, ref_idx, scores.max(axis=1), ref_kth)
            n_diff += dd
            n_exc += ee
            assert abs(kth[b, g] - ref_kth) <= 1e-3
    print(f"[{name}] pooled top-k entries differing {n_diff}, excused near k-th value {n_exc}")
    assert n_diff == n_exc


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("n_split", [1, 3, 0])
def test_index_kv_decode_parity(name, n_split):
    """Reuse layer with one shared index set per KV head: every query head of
    the group attends at its KV head's indices."""
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, sl, k = SHAPES[name]
    d, gpu = inputs(name)
    L0, L1 = gpu["layers"]
    idx, _ = fsa.topk_indices_kv(L0["q"], L0["k"], gpu["page_table"], gpu["seq_lens"], k,
                                 max_seq_len=N)
    out, lse = fsa.sparse_decode_attn(L1["q"], L1["k"], L1["v"], gpu["page_table"], gpu["seq_lens"],
                                      mode=fsa.SEL_INDEX_KV, idx=idx, n_split=n_split,
                                      max_seq_len=N)
    out, lse, idx = out.cpu(), lse.cpu(), idx.cpu().numpy()
    q1 = workloads.to_f64(d["layers"][1]["q"])
    G = Hq // Hkv
    scale = 1 / math.sqrt(D)
    for b in range(B):
        for h in range(Hq):
            K, V = seq_kv(d, 1, b, oracle.kv_head(h, Hq, Hkv))
            o, l = oracle.index_attention(q1[b, h], K, V, idx[b, oracle.kv_head(h, Hq, Hkv)], scale)
            assert np.abs(out[b, h].double().numpy() - o).max() <= TOL_BF16
            assert abs(lse[b, h].item() - l) <= 1e-2


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("mode", ["all", "global", "focus", "local", "streaming"])
def test_segment_decode_parity(name, mode):
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, sl, k = SHAPES[name]
    d, gpu = inputs(name)
    L1 = gpu["layers"][1]
    G = Hq // Hkv
    scale = 1 / math.sqrt(D)
    ranges = []
    rng = np.random.default_rng(5)
    for b in range(B):
        n = sl[b]
        if mode in ("all", "global"):
            ranges.append(oracle.build_segments(oracle.SEG_GLOBAL, n))
        elif mode == "focus":
            s = int(rng.integers(0, max(1, n - 2048)))
            ranges.append(oracle.build_segments(oracle.SEG_FOCUS, n, s, 2048, 1024))
        elif mode == "local":
            ranges.append(oracle.build_segments(oracle.SEG_LOCAL, n, local_len=1024))
        else:
            ranges.append(oracle.build_segments(oracle.SEG_STREAMING, n, local_len=1024, n_sink=4))
    if mode == "all":
        out, lse = fsa.sparse_decode_attn(L1["q"], L1["k"], L1["v"], gpu["page_table"],
                                          gpu["seq_lens"], mode=fsa.SEL_ALL, max_seq_len=N)
    else:
        segs = torch.zeros((B, 4, 2), dtype=torch.int32)
        nseg = torch.zeros(B, dtype=torch.int32)
        for b, rs in enumerate(ranges):
            nseg[b] = len(rs)
            for x, (a, e) in enumerate(rs):
                segs[b, x, 0], segs[b, x, 1] = a, e
        out, lse = fsa.sparse_decode_attn(L1["q"], L1["k"], L1["v"], gpu["page_table"],
                                          gpu["seq_lens"], mode=fsa.SEL_SEGMENT, segments=segs.cuda(),
                                          n_seg=nseg.cuda(), n_split=5 if mode == "focus" else 0,
                                          max_seq_len=N)
    out, lse = out.cpu(), lse.cpu()
    q1 = workloads.to_f64(d["layers"][1]["q"])
    for b in range(B):
        for h in range(Hq):
            K, V = seq_kv(d, 1, b, oracle.kv_head(h, Hq, Hkv))
            o, l = oracle.segment_attention(q1[b, h], K, V, ranges[b], scale)
            assert np.abs(out[b, h].double().numpy() - o).max() <= TOL_BF16, (b, h)
            assert abs(lse[b, h].item() - l) <= 1e-2


def test_empty_segment_gives_zero_output():
    import free_sparse_attention_head_amd as fsa
    d, gpu = inputs("gqa4_d128")
    L1 = gpu["layers"][1]
    segs = torch.zeros((3, 1, 2), dtype=torch.int32, device="cuda")
    nseg = torch.zeros(3, dtype=torch.int32, device="cuda")
    out, lse = fsa.sparse_decode_attn(L1["q"], L1["k"], L1["v"], gpu["page_table"], gpu["seq_lens"],
                                      mode=fsa.SEL_SEGMENT, segments=segs, n_seg=nseg, max_seq_len=8192)
    assert (out.cpu() == 0).all() and torch.isinf(lse.cpu()).all()


@pytest.mark.parametrize("n_split", [0, 1, 3])
def test_empty_sequence_in_a_batch(n_split):
    """A sequence with no cached tokens beside a ragged one: its top-k slots
    are all -1 with kth -inf (scores -inf in the scored form), and index and
    all-token decode give o = 0, lse = -inf; the other sequence still matches
    the oracle."""
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, k = 2, 2048, 8, 2, 128, 64
    print(f"[decode case empty-seq] n_split={n_split}", flush=True)
    d = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=2, seq_lens=[0, 1500], seed=91,
                                device="cpu")
    pt, sl = d["page_table"].cuda(), d["seq_lens"].cuda()
    L0 = {x: t.cuda() for x, t in d["layers"][0].items()}
    L1 = {x: t.cuda() for x, t in d["layers"][1].items()}
    idx, kth = fsa.topk_indices(L0["q"], L0["k"], pt, sl, k, max_seq_len=N)
    idxs, sco, kths = fsa.topk_indices_scored(L0["q"], L0["k"], pt, sl, k, max_seq_len=N)
    assert (idx[0].cpu() == -1).all()
    assert (idxs[0].cpu() == -1).all() and (sco[0].cpu() == -math.inf).all()
    assert torch.equal(idx.cpu(), idxs.cpu())
    scale = 1.0 / math.sqrt(D)
    q0, q1 = workloads.to_f64(d["layers"][0]["q"]), workloads.to_f64(d["layers"][1]["q"])
    assert np.isneginf(kth[0].cpu().numpy()).all()
    for h in range(Hq):
        K0, _ = seq_kv(d, 0, 1, oracle.kv_head(h, Hq, Hkv))
        scores = oracle.anchor_scores(q0[1, h], K0)
        ref, ref_kth = oracle.topk(scores, k)
        n_diff, n_exc = topk_diff_excused(idx[1, h].cpu().numpy(), ref, scores, ref_kth)
        assert n_diff == n_exc
        assert abs(kth[1, h].item() - ref_kth) <= 1e-3
    out, lse = fsa.sparse_decode_attn(L1["q"], L1["k"], L1["v"], pt, sl, mode=fsa.SEL_INDEX,
                                      idx=idx, n_split=n_split, max_seq_len=N)
    outa, lsea = fsa.sparse_decode_attn(L1["q"], L1["k"], L1["v"], pt, sl, mode=fsa.SEL_ALL,
                                        n_split=n_split, max_seq_len=N)
    for o, l in ((out, lse), (outa, lsea)):
        assert (o[0].cpu() == 0).all() and (l[0].cpu() == -math.inf).all()
    for h in range(Hq):
        K1, V1 = seq_kv(d, 1, 1, oracle.kv_head(h, Hq, Hkv))
        ro, rl = oracle.index_attention(q1[1, h], K1, V1, idx[1, h].cpu().numpy(), scale)
        assert np.abs(out[1, h].float().cpu().numpy() - ro).max() <= TOL_BF16
        assert abs(lse[1, h].item() - rl) <= 1e-2
        ao, al = oracle.segment_attention(q1[1, h], K1, V1, [(0, 1500)], scale)
        assert np.abs(outa[1, h].float().cpu().numpy() - ao).max() <= TOL_BF16
        assert abs(lsea[1, h].item() - al) <= 1e-2


@pytest.mark.parametrize("n_split", [64, 4096])
def test_short_segments_with_many_splits(n_split):
    """A few hundred admitted tokens (three short segments, 600 in all) against
    many splits: a split takes at least 256 positions, so all but a few splits
    are empty and write empty partials, which the combine must skip.  The
    result equals the oracle's attention over the same ranges."""
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, sl, k = SHAPES["gqa4_d128"]
    print(f"[short segments] n_split={n_split}", flush=True)
    d, gpu = inputs("gqa4_d128")
    L1 = gpu["layers"][1]
    G = Hq // Hkv
    scale = 1 / math.sqrt(D)
    ranges = [[(0, 16), (1024, 1280), (4000, 4328)], [(32, 48), (2000, 2256), (4900, 5003)],
              [(0, 100)]]
    segs = torch.zeros((B, 3, 2), dtype=torch.int32)
    nseg = torch.zeros(B, dtype=torch.int32)
    for b, rs in enumerate(ranges):
        nseg[b] = len(rs)
        for x, (a, e) in enumerate(rs):
            segs[b, x, 0], segs[b, x, 1] = a, e
    out, lse = fsa.sparse_decode_attn(L1["q"], L1["k"], L1["v"], gpu["page_table"],
                                      gpu["seq_lens"], mode=fsa.SEL_SEGMENT, segments=segs.cuda(),
                                      n_seg=nseg.cuda(), n_split=n_split, max_seq_len=N)
    out, lse = out.cpu(), lse.cpu()
    q1 = workloads.to_f64(d["layers"][1]["q"])
    for b in range(B):
        for h in range(Hq):
            K, V = seq_kv(d, 1, b, oracle.kv_head(h, Hq, Hkv))
            o, l = oracle.segment_attention(q1[b, h], K, V, ranges[b], scale)
            assert np.abs(out[b, h].double().numpy() - o).max() <= TOL_BF16, (b, h)
            assert abs(lse[b, h].item() - l) <= 1e-2


@pytest.mark.parametrize("name", ["gqa4_d128", "gqa8_d64"])
def test_segment_decode_mixed_batch(name):
    """One batch whose sequences use different modes (drawn by seed: global,
    focus, local or streaming per sequence), with automatic splits."""
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, sl, k = SHAPES[name]
    d, gpu = inputs(name)
    L1 = gpu["layers"][1]
    G = Hq // Hkv
    scale = 1 / math.sqrt(D)
    rng = np.random.default_rng(21)
    kinds = ["global", "focus", "local", "streaming"]
    draw = [kinds[(b + int(rng.integers(0, 4))) % 4] for b in range(B)]
    print(f"[mixed batch {name}] modes {draw}", flush=True)
    ranges = []
    for b, mode in enumerate(draw):
        n = sl[b]
        if mode == "global":
            ranges.append(oracle.build_segments(oracle.SEG_GLOBAL, n))
        elif mode == "focus":
            s = int(rng.integers(0, max(1, n - 2048)))
            ranges.append(oracle.build_segments(oracle.SEG_FOCUS, n, s, 2048, 1024))
        elif mode == "local":
            ranges.append(oracle.build_segments(oracle.SEG_LOCAL, n, local_len=1024))
        else:
            ranges.append(oracle.build_segments(oracle.SEG_STREAMING, n, local_len=1024, n_sink=4))
    segs = torch.zeros((B, 4, 2), dtype=torch.int32)
    nseg = torch.zeros(B, dtype=torch.int32)
    for b, rs in enumerate(ranges):
        nseg[b] = len(rs)
        for x, (a, e) in enumerate(rs):
            segs[b, x, 0], segs[b, x, 1] = a, e
    out, lse = fsa.sparse_decode_attn(L1["q"], L1["k"], L1["v"], gpu["page_table"],
                                      gpu["seq_lens"], mode=fsa.SEL_SEGMENT, segments=segs.cuda(),
                                      n_seg=nseg.cuda(), max_seq_len=N)
    out, lse = out.cpu(), lse.cpu()
    q1 = workloads.to_f64(d["layers"][1]["q"])
    for b in range(B):
        for h in range(Hq):
            K, V = seq_kv(d, 1, b, oracle.kv_head(h, Hq, Hkv))
            o, l = oracle.segment_attention(q1[b, h], K, V, ranges[b], scale)
            assert np.abs(out[b, h].double().numpy() - o).max() <= TOL_BF16, (b, h)
            assert abs(lse[b, h].item() - l) <= 1e-2


@pytest.mark.parametrize("name", list(SHAPES))
def test_topk_union_kv_parity(name):
    """The union of each KV head's per-query-head top-k sets equals the
    oracle's union of the same sets exactly (ragged sequences leave -1 slots,
    which are dropped), and decode over the union matches the oracle's
    attention of every query head at that set."""
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, sl, k = SHAPES[name]
    d, gpu = inputs(name)
    L0, L1 = gpu["layers"]
    idx, _ = fsa.topk_indices(L0["q"], L0["k"], gpu["page_table"], gpu["seq_lens"], k, max_seq_len=N)
    uni, cnt = fsa.topk_union_kv(idx, Hkv)
    out, lse = fsa.sparse_decode_attn(L1["q"], L1["k"], L1["v"], gpu["page_table"], gpu["seq_lens"],
                                      mode=fsa.SEL_INDEX_KV, idx=uni, max_seq_len=N)
    idx, uni, cnt, out, lse = (t.cpu() for t in (idx, uni, cnt, out, lse))
    G = Hq // Hkv
    assert uni.shape == (B, Hkv, G * k)
    q1 = workloads.to_f64(d["layers"][1]["q"])
    scale = 1 / math.sqrt(D)
    sizes = []
    for b in range(B):
        for g in range(Hkv):
            heads = [h for h in range(Hq) if oracle.kv_head(h, Hq, Hkv) == g]
            ref = oracle.union_sets([idx[b, h].numpy() for h in heads])
            c = int(cnt[b, g])
            assert c == ref.size
            assert (uni[b, g, :c].numpy() == ref).all() and (uni[b, g, c:] == -1).all()
            sizes.append(c / (G * k))
            K, V = seq_kv(d, 1, b, g)
            for h in (heads[0], heads[-1]):
                o, l = oracle.index_attention(q1[b, h], K, V, ref, scale)
                assert np.abs(out[b, h].double().numpy() - o).max() <= TOL_BF16
                assert abs(lse[b, h].item() - l) <= 1e-2
    print(f"[{name}] union size / (G k) mean {np.mean(sizes):.3f}")


def test_topk_union_kv_unsorted_duplicates_and_empty_slots():
    """Any order, repeated entries within and across heads, and negative
    slots anywhere: the union is the sorted distinct non-negative entries."""
    import free_sparse_attention_head_amd as fsa
    rng = np.random.default_rng(9)
    B, Hq, Hkv, k = 3, 8, 2, 700       # G k = 2800: padded to 4096 in the sort
    idx = rng.integers(-3, 5000, size=(B, Hq, k)).astype(np.int32)
    idx[0, 1, :] = idx[0, 0, ::-1]      # one head repeats another's set reversed
    idx[1, 4:8, :] = -1                 # a KV head with every slot empty
    idx[2, :, :350] = 77                # heavy duplication
    uni, cnt = fsa.topk_union_kv(torch.from_numpy(idx).cuda(), Hkv)
    uni, cnt = uni.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            ref = oracle.union_sets([idx[b, h] for h in range(Hq) if oracle.kv_head(h, Hq, Hkv) == g])
            assert cnt[b, g] == ref.size
            assert (uni[b, g, :ref.size] == ref).all() and (uni[b, g, ref.size:] == -1).all()
    assert cnt[1, 1] == 0


def test_topk_union_kv_largest_sort():
    """G k = 16384 exactly (8 heads x 2048): the largest sort the kernel runs."""
    import free_sparse_attention_head_amd as fsa
    rng = np.random.default_rng(10)
    B, Hq, Hkv, k = 2, 8, 1, 2048
    idx = np.sort(rng.integers(0, 40000, size=(B, Hq, k)), axis=2).astype(np.int32)
    uni, cnt = fsa.topk_union_kv(torch.from_numpy(idx).cuda(), Hkv)
    uni, cnt = uni.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        ref = oracle.union_sets(list(idx[b]))
        assert cnt[b, 0] == ref.size and (uni[b, 0, :ref.size] == ref).all()
        assert (uni[b, 0, ref.size:] == -1).all()


def test_shared_set_accuracy_harness_matches_oracle():
    """The measurements behind the bench's per-head vs shared-set comparison:
    recall of each head's own top-k inside the pooled set (bench's
    shared_set_recall) against oracle.set_recall, and the softmax mass a set
    keeps, exp(lse_set - lse_dense) from two decode launches, against
    oracle.index_mass for per-head, pooled and union sets."""
    import bench
    import free_sparse_attention_head_amd as fsa
    name = "gqa4_d128"
    B, N, Hq, Hkv, D, sl, k = SHAPES[name]
    d, gpu = inputs(name)
    L0, L1 = gpu["layers"]
    pt, sls = gpu["page_table"], gpu["seq_lens"]
    own, _ = fsa.topk_indices(L0["q"], L0["k"], pt, sls, k, max_seq_len=N)
    pooled, _ = fsa.topk_indices_kv(L0["q"], L0["k"], pt, sls, k, max_seq_len=N)
    uni, _ = fsa.topk_union_kv(own, Hkv)
    G = Hq // Hkv
    rec = bench.shared_set_recall(own, pooled, G).cpu().numpy()
    args = (L1["q"], L1["k"], L1["v"], pt, sls)
    _, lse_d = fsa.sparse_decode_attn(*args, mode=fsa.SEL_ALL, max_seq_len=N)
    kept = {}
    for key, mode, ix in (("own", fsa.SEL_INDEX, own), ("pooled", fsa.SEL_INDEX_KV, pooled),
                          ("union", fsa.SEL_INDEX_KV, uni)):
        _, lse = fsa.sparse_decode_attn(*args, mode=mode, idx=ix, max_seq_len=N)
        kept[key] = torch.exp(lse - lse_d).cpu().numpy()
    own, pooled, uni = own.cpu().numpy(), pooled.cpu().numpy(), uni.cpu().numpy()
    q1 = workloads.to_f64(d["layers"][1]["q"])
    scale = 1 / math.sqrt(D)
    worst = 0.0
    for b in range(B):
        for h in range(Hq):
            g = oracle.kv_head(h, Hq, Hkv)
            if (own[b, h] >= 0).any():
                assert abs(rec[b, h] - oracle.set_recall(own[b, h], pooled[b, g])) <= 1e-6
            K, _ = seq_kv(d, 1, b, g)
            for key, ix in (("own", own[b, h]), ("pooled", pooled[b, g]), ("union", uni[b, g])):
                ref = oracle.index_mass(q1[b, h], K, ix, scale)
                worst = max(worst, abs(kept[key][b, h] - ref))
    print(f"[shared-set harness] mass kept max-abs difference GPU vs oracle {worst:.2e}")
    assert worst <= 2e-2


@pytest.mark.parametrize("name", list(SHAPES))
def test_topk_scores_and_scored_anchor_decode(name):
    """topk_indices_scored returns the same index sets as topk_indices and, for
    each kept key, its score (against the oracle's anchor scores; -inf in
    the empty slots of a short sequence); the anchor layer's attention at
    its own top-k from those scores, reading V only, equals index decode of
    the same layer bit for bit (the scores are the decode kernel's own dot
    products) and the oracle's attention at those indices."""
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D, sl, k = SHAPES[name]
    d, gpu = inputs(name)
    L0 = gpu["layers"][0]
    pt, sls = gpu["page_table"], gpu["seq_lens"]
    idx_ref, kth_ref = fsa.topk_indices(L0["q"], L0["k"], pt, sls, k, max_seq_len=N)
    idx, sco, kth = fsa.topk_indices_scored(L0["q"], L0["k"], pt, sls, k, max_seq_len=N)
    assert torch.equal(idx, idx_ref) and torch.equal(kth, kth_ref)
    args = (L0["q"], L0["k"], L0["v"], pt, sls)
    o_i, l_i = fsa.sparse_decode_attn(*args, mode=fsa.SEL_INDEX, idx=idx, max_seq_len=N)
    for ns in (0, 3):
        o_s, l_s = fsa.sparse_decode_attn(*args, mode=fsa.SEL_INDEX_SCORED, idx=idx, scores=sco,
                                          n_split=ns, max_seq_len=N)
        if ns == 0:
            assert torch.equal(o_s, o_i) and torch.equal(l_s, l_i)
    # keys are not read in scored mode: a pool of zeros in their place changes nothing
    o_z, l_z = fsa.sparse_decode_attn(L0["q"], torch.zeros_like(L0["k"]), L0["v"], pt, sls,
                                      mode=fsa.SEL_INDEX_SCORED, idx=idx, scores=sco, max_seq_len=N)
    assert torch.equal(o_z, o_i) and torch.equal(l_z, l_i)
    idx, sco, o_i, l_i = idx.cpu().numpy(), sco.cpu().numpy(), o_i.cpu(), l_i.cpu()
    q = workloads.to_f64(d["layers"][0]["q"])
    scale = 1 / math.sqrt(D)
    for b in range(B):
        n = sl[b]
        for h in range(Hq):
            K, V = seq_kv(d, 0, b, oracle.kv_head(h, Hq, Hkv))
            s = oracle.anchor_scores(q[b, h], K)
            valid = idx[b, h] >= 0
            assert np.abs(sco[b, h][valid] - s[idx[b, h][valid]]).max() <= 1e-3
            assert np.isneginf(sco[b, h][~valid]).all()
            assert valid.sum() == min(n, k)
            o, l = oracle.index_attention(q[b, h], K, V, idx[b, h], scale)
            assert np.abs(o_i[b, h].double().numpy() - o).max() <= TOL_BF16
            assert abs(l_i[b, h].item() - l) <= 1e-2

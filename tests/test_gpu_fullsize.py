"""GPU parity at the full benchmark sizes, in the launch configuration bench.py
times, checked on sampled outputs that the fp64 oracle computes one by one.

  * 32K sparse prefill: B=1, S=32768, 32 query / 8 KV heads, D=128, bf16,
    block 64, low-rank keys with 1% planted spikes, selector tuned to 10%
    density.
  * 128K sparse prefill: B=1, S=131072, 32 / 4 heads, block 128, diagonal
    band of 8 blocks + sink block, densities 3 / 6 / 12%.
  * 128K Kascade decode group: B=32, N=131072, 32 / 8 heads, k=2048, 4 layers
    (anchor top-k, indices reused by layers 1-3), shuffled 16-token pages; and
    its per-KV-head variant (pooled top-k, shared indices).
  * 1M segment decode: B=4, N=2^20, global / focus / local / streaming masks;
    and the scored top-k with the anchor's attention over the same 1M pool
    shape, ragged lengths.

Sampled rows: block statistics and selector rows against the oracle
(bit-exact up to near-threshold entries), attention outputs against the
oracle evaluated on the GPU's own mask or indices (2e-2 max-abs, bf16) and
log-sum-exps within 1e-2.  Decode keys and values reach the oracle through
its own paged gather: the pages a sequence uses are copied to the host whole,
in page-id order, and oracle.gather_pages reads them through the sequence's
page table (remapped to that copy).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._parity import (BAND, LSE_TOL_BF16, TOL_BF16, lists_to_mask, mask_diff_excused,
                           topk_diff_excused)

pytestmark = pytest.mark.gpu


def _fsa():
    import free_sparse_attention_head_amd as fsa
    return fsa


def _tune(fsa, q, c, r, T, target, band, sink, visible):
    """Bisect p_c (p_r = 0.4 p_c) to the target density, as the benchmark does."""
    lo, hi, out = 0.0, 1.0, None
    for _ in range(30):
        pc = 0.5 * (lo + hi)
        out = fsa.select_blocks(q, c, r, T, pc, 0.4 * pc, band, sink, out=out)
        dens = out["block_cnt"].sum().item() / visible
        if abs(dens - target) <= 0.0025:
            return pc, dens, out
        lo, hi = (pc, hi) if dens < target else (lo, pc)
    return pc, dens, out


def _check_prefill(name, S, Hq, Hkv, T, band, sink, density, seed, n_rows=6, n_tok=3):
    fsa = _fsa()
    print(f"[fullsize {name}] S={S} Hq={Hq} Hkv={Hkv} T={T} density={density}", flush=True)
    D, G, nB = 128, Hq // Hkv, S // T
    inp = workloads.prefill_inputs(1, S, Hq, Hkv, D, T, model="lowrank", seed=seed, device="cuda")
    q, k, v = inp["q"], inp["k"], inp["v"]
    c, r = fsa.block_stats(k, T)
    visible = Hq * nB * (nB + 1) // 2
    pc, dens, sel = _tune(fsa, q, c, r, T, density, band, sink, visible)
    assert abs(dens - density) <= 0.0025
    o, lse = fsa.sparse_prefill_attn(q, k, v, T, sel["block_idx"], sel["block_cnt"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    scale = 1 / math.sqrt(D)
    n_diff = n_exc = 0
    worst_lse = 0.0
    for g in rng.choice(Hkv, size=min(2, Hkv), replace=False):
        kk = workloads.to_f64(k[0, :, g])
        vv = workloads.to_f64(v[0, :, g])
        c_ref, r_ref = oracle.block_stats(kk, T)
        assert np.abs(c[0, g].double().cpu().numpy() - c_ref).max() <= 1e-5
        assert np.abs(r[0, g].double().cpu().numpy() - r_ref).max() <= 1e-4 * r_ref.max()
        heads = [h for h in range(Hq) if oracle.kv_head(h, Hq, Hkv) == g]
        for h in rng.choice(heads, size=2, replace=False):
            qh = workloads.to_f64(q[0, :, h])
            qbar = oracle.pool_queries(qh, T)
            cnt = sel["block_cnt"][0, h].cpu().numpy()
            lst = sel["block_idx"][0, h].cpu().numpy()
            rows = np.unique(np.concatenate([[0, nB - 1], rng.integers(0, nB, n_rows)]))
            for i in rows:
                # one selector row: the oracle's own selection restricted to row i
                ref = oracle.select_blocks(qbar[:i + 1], c_ref[:i + 1], r_ref[:i + 1], pc, 0.4 * pc,
                                           band, sink)
                li = lst[i, :cnt[i]]
                assert (np.diff(li) > 0).all() and li.min() >= 0 and li.max() <= i
                gm = np.zeros((i + 1, i + 1), dtype=bool)
                gm[i, li] = True
                one = {x: y[i:i + 1] for x, y in ref.items()}
                d_, e_ = mask_diff_excused(gm[i:i + 1], one)
                n_diff, n_exc = n_diff + d_, n_exc + e_
                # attention rows of this query block, on the GPU's mask
                m = np.zeros((nB, nB), dtype=bool)
                m[i, li] = True
                toks = i * T + np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, n_tok)]))
                o_ref, l_ref = oracle.masked_attention_rows(qh, kk, vv, m, T, scale, toks)
                got = o[0, toks, h].double().cpu().numpy()
                assert np.abs(got - o_ref).max() <= TOL_BF16, (g, h, i)
                err = np.abs(lse[0, h, toks].double().cpu().numpy() - l_ref).max()
                worst_lse = max(worst_lse, err)
                assert err <= LSE_TOL_BF16, (g, h, i, err)
    print(f"[fullsize {name}] density {dens:.4f}; sampled mask entries differing {n_diff}, "
          f"excused {n_exc}; worst lse error {worst_lse:.2e}", flush=True)
    assert n_diff == n_exc


def test_prefill_32k_block64_density10():
    _check_prefill("prefill32k", 32768, 32, 8, 64, 0, 0, 0.10, seed=1001)


@pytest.mark.parametrize("density", [0.03, 0.06, 0.12])
def test_prefill_128k_block128(density):
    _check_prefill(f"prefill128k-{density}", 131072, 32, 4, 128, 8, 1, density, seed=1002)


def _seq_kv(pool, page_table_row, n, g, start=0):
    """K or V of tokens [start, start + n) of one sequence and KV head (start
    page-aligned), through the oracle's paged gather: the pages the range uses
    are copied to the host whole, in page-id order, and oracle.gather_pages
    reads them through the range's page-table entries remapped to that copy."""
    assert start % 16 == 0
    ids = page_table_row[start // 16: (start + n + 15) // 16].long()
    uniq, inv = torch.unique(ids, sorted=True, return_inverse=True)
    sub = workloads.to_f64(pool[uniq, g:g + 1])          # [pages, 1, 16, D]
    return oracle.gather_pages(sub, inv.cpu().numpy(), n, 0)


def test_kascade_decode_128k_group():
    fsa = _fsa()
    B, N, Hq, Hkv, D, k, L = 32, 131072, 32, 8, 128, 2048, 4
    print(f"[fullsize kascade] B={B} N={N} k={k} layers={L}", flush=True)
    d = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=L, seed=1003, device="cuda")
    pt, sl = d["page_table"], d["seq_lens"]
    idx, kth = fsa.topk_indices(d["layers"][0]["q"], d["layers"][0]["k"], pt, sl, k)
    outs = [fsa.sparse_decode_attn(d["layers"][li]["q"], d["layers"][li]["k"], d["layers"][li]["v"],
                                   pt, sl, mode=fsa.SEL_INDEX, idx=idx)[0] for li in range(L)]
    torch.cuda.synchronize()
    idx_h, kth_h = idx.cpu().numpy(), kth.cpu().numpy()
    rng = np.random.default_rng(3)
    n_diff = n_exc = 0
    for b in rng.choice(B, size=3, replace=False):
        for h in rng.choice(Hq, size=3, replace=False):
            g = oracle.kv_head(h, Hq, Hkv)
            K0 = _seq_kv(d["layers"][0]["k"], pt[b], N, g)
            s = oracle.anchor_scores(workloads.to_f64(d["layers"][0]["q"][b, h]), K0)
            ref_idx, ref_kth = oracle.topk(s, k)
            row = idx_h[b, h]
            assert (np.diff(row) > 0).all()
            dd, ee = topk_diff_excused(row, ref_idx, s, ref_kth)
            n_diff, n_exc = n_diff + dd, n_exc + ee
            assert abs(kth_h[b, h] - ref_kth) <= BAND
            for li in range(L):
                Kl = K0 if li == 0 else _seq_kv(d["layers"][li]["k"], pt[b], N, g)
                Vl = _seq_kv(d["layers"][li]["v"], pt[b], N, g)
                o_ref, _ = oracle.index_attention(workloads.to_f64(d["layers"][li]["q"][b, h]), Kl, Vl,
                                                  row, 1 / math.sqrt(D))
                assert np.abs(outs[li][b, h].double().cpu().numpy() - o_ref).max() <= TOL_BF16
    print(f"[fullsize kascade] top-k entries differing {n_diff}, excused {n_exc}", flush=True)
    assert n_diff == n_exc


def test_kascade_kv_shared_decode_128k_group():
    """The per-KV-head variant at the benchmark size: one pooled top-k per KV
    head, four layers attending at it with the group's query heads sharing
    every read."""
    fsa = _fsa()
    B, N, Hq, Hkv, D, k, L = 32, 131072, 32, 8, 128, 2048, 4
    print(f"[fullsize kascade-kv] B={B} N={N} k={k} layers={L}", flush=True)
    d = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=L, seed=1003, device="cuda")
    pt, sl = d["page_table"], d["seq_lens"]
    idx, kth = fsa.topk_indices_kv(d["layers"][0]["q"], d["layers"][0]["k"], pt, sl, k)
    outs = [fsa.sparse_decode_attn(d["layers"][li]["q"], d["layers"][li]["k"], d["layers"][li]["v"],
                                   pt, sl, mode=fsa.SEL_INDEX_KV, idx=idx)[0] for li in range(L)]
    torch.cuda.synchronize()
    idx_h, kth_h = idx.cpu().numpy(), kth.cpu().numpy()
    rng = np.random.default_rng(5)
    n_diff = n_exc = 0
    for b in rng.choice(B, size=3, replace=False):
        for g in rng.choice(Hkv, size=2, replace=False):
            heads = [h for h in range(Hq) if oracle.kv_head(h, Hq, Hkv) == g]
            K0 = _seq_kv(d["layers"][0]["k"], pt[b], N, g)
            s = np.stack([oracle.anchor_scores(workloads.to_f64(d["layers"][0]["q"][b, h]), K0)
                          for h in heads], axis=1)         # [N, G]
            ref_idx, ref_kth = oracle.topk_pooled(s.T, k)
            row = idx_h[b, g]
            assert (np.diff(row) > 0).all()
            dd, ee = topk_diff_excused(row, ref_idx, s.max(axis=1), ref_kth)
            n_diff, n_exc = n_diff + dd, n_exc + ee
            assert abs(kth_h[b, g] - ref_kth) <= BAND
            for li in range(L):
                Kl = K0 if li == 0 else _seq_kv(d["layers"][li]["k"], pt[b], N, g)
                Vl = _seq_kv(d["layers"][li]["v"], pt[b], N, g)
                for h in (heads[0], heads[-1]):
                    o_ref, _ = oracle.index_attention(workloads.to_f64(d["layers"][li]["q"][b, h]),
                                                      Kl, Vl, row, 1 / math.sqrt(D))
                    assert np.abs(outs[li][b, h].double().cpu().numpy() - o_ref).max() <= TOL_BF16
    print(f"[fullsize kascade-kv] pooled top-k entries differing {n_diff}, excused {n_exc}", flush=True)
    assert n_diff == n_exc


def test_scored_topk_1m_context():
    """Top-k at a 1M-token context (the segment workload's pool shape: B=4,
    2^20 tokens, 32 / 8 heads, shuffled pages), ragged lengths (2^20, a
    length not a multiple of the page, and exactly k), in the scored form the
    anchor layer uses, and the anchor's V-only attention from those scores:
    about 500 score tiles per row and the longest candidate streams the
    select kernel reads."""
    fsa = _fsa()
    B, N, Hq, Hkv, D, k = 4, 1 << 20, 32, 8, 128, 2048
    lens = [N, N - 12345, 700003, k]
    print(f"[fullsize topk-1m] B={B} N={N} k={k} seq_lens={lens}", flush=True)
    d = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=1, seq_lens=lens, seed=1005, device="cuda")
    pt, sl = d["page_table"], d["seq_lens"]
    Lr = d["layers"][0]
    idx, sco, kth = fsa.topk_indices_scored(Lr["q"], Lr["k"], pt, sl, k)
    out, _ = fsa.sparse_decode_attn(Lr["q"], Lr["k"], Lr["v"], pt, sl, mode=fsa.SEL_INDEX_SCORED,
                                    idx=idx, scores=sco)
    torch.cuda.synchronize()
    idx_h, sco_h, kth_h = idx.cpu().numpy(), sco.cpu().numpy(), kth.cpu().numpy()
    assert (idx_h[3] == np.arange(k)).all()               # n == k: every key, in order
    rng = np.random.default_rng(6)
    n_diff = n_exc = 0
    for b in (0, 1, 2):
        for h in rng.choice(Hq, size=2, replace=False):
            g = oracle.kv_head(h, Hq, Hkv)
            n = lens[b]
            K = _seq_kv(Lr["k"], pt[b], n, g)
            qh = workloads.to_f64(Lr["q"][b, h])
            s = oracle.anchor_scores(qh, K)
            ref_idx, ref_kth = oracle.topk(s, k)
            row = idx_h[b, h]
            assert (np.diff(row) > 0).all() and row.min() >= 0 and row.max() < n
            dd, ee = topk_diff_excused(row, ref_idx, s, ref_kth)
            n_diff, n_exc = n_diff + dd, n_exc + ee
            assert abs(kth_h[b, h] - ref_kth) <= BAND
            assert np.abs(sco_h[b, h] - s[row]).max() <= 1e-3      # each kept key's own score
            V = _seq_kv(Lr["v"], pt[b], n, g)
            o_ref, _ = oracle.index_attention(qh, K, V, row, 1 / math.sqrt(D))
            assert np.abs(out[b, h].double().cpu().numpy() - o_ref).max() <= TOL_BF16, (b, h)
    print(f"[fullsize topk-1m] top-k entries differing {n_diff}, excused {n_exc}", flush=True)
    assert n_diff == n_exc


def test_segment_decode_1m_all_modes():
    fsa = _fsa()
    B, N, Hq, Hkv, D = 4, 1 << 20, 32, 8, 128
    print(f"[fullsize segment] B={B} N={N}", flush=True)
    d = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=1, seed=1004, device="cuda")
    pt, sl = d["page_table"], d["seq_lens"]
    Lr = d["layers"][0]
    rng = np.random.default_rng(4)
    modes = {"global": fsa.SEG_GLOBAL, "focus": fsa.SEG_FOCUS, "local": fsa.SEG_LOCAL,
             "streaming": fsa.SEG_STREAMING}
    for name, code in modes.items():
        ranges, segs, nseg = [], torch.zeros((B, 2, 2), dtype=torch.int32), torch.zeros(B, dtype=torch.int32)
        for b in range(B):
            st = int(rng.integers(0, N - 2048))
            rs = fsa.build_segments(code, N, chunk_start=st, chunk_len=2048, local_len=1024, n_sink=4)
            ranges.append(rs)
            nseg[b] = len(rs)
            for x, (a, e) in enumerate(rs):
                segs[b, x, 0], segs[b, x, 1] = a, e
        out, lse = fsa.sparse_decode_attn(Lr["q"], Lr["k"], Lr["v"], pt, sl, mode=fsa.SEL_SEGMENT,
                                          segments=segs.cuda(), n_seg=nseg.cuda())
        torch.cuda.synchronize()
        for b in rng.choice(B, size=2, replace=False):
            for h in rng.choice(Hq, size=2, replace=False):
                g = oracle.kv_head(h, Hq, Hkv)
                qh = workloads.to_f64(Lr["q"][b, h])
                if name == "global":
                    K = _seq_kv(Lr["k"], pt[b], N, g)
                    V = _seq_kv(Lr["v"], pt[b], N, g)
                    o_ref, l_ref = oracle.segment_attention(qh, K, V, ranges[b], 1 / math.sqrt(D))
                else:
                    # each range starts on a page boundary (rounded outward, or
                    # token 0 / N - 1024): gather the ranges alone and attend
                    # over all of their tokens
                    K = np.concatenate([_seq_kv(Lr["k"], pt[b], e - a, g, start=a) for a, e in ranges[b]])
                    V = np.concatenate([_seq_kv(Lr["v"], pt[b], e - a, g, start=a) for a, e in ranges[b]])
                    o_ref, l_ref = oracle.index_attention(qh, K, V, np.arange(K.shape[0]),
                                                          1 / math.sqrt(D))
                assert np.abs(out[b, h].double().cpu().numpy() - o_ref).max() <= TOL_BF16, (name, b, h)
                assert abs(lse[b, h].item() - l_ref) <= LSE_TOL_BF16
        print(f"[fullsize segment] mode {name} ok", flush=True)

"""GPU parity of the prefill path (block_stats, select_blocks, sparse_prefill_attn)
against the fp64 oracle, through the C ABI.

Sizes are small enough for the oracle to finish in seconds but span several
MFMA tiles, several 32-bit mask words with a ragged tail (nB = 40), both block
sizes, both head dims, GQA groups, batch > 1, forced band/sink blocks, a
switched-off branch, both branches off (forced blocks only), and fp32 as well
as bf16 inputs at every head-dim / block-size pair.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests._parity import (LSE_TOL_BF16, LSE_TOL_F32, TOL_BF16, TOL_F32, bits_to_mask,
                           lists_to_mask, mask_diff_excused)

pytestmark = pytest.mark.gpu

CASES = {
    # name: (B, S, Hq, Hkv, D, T, dtype, model, n_spikes, p_c, p_r, band, sink)
    "cfg0_tiny_fp32": (1, 1024, 2, 2, 64, 64, torch.float32, "iid", 4, 0.25, 0.10, 0, 0),
    "bf16_T64_ragged": (1, 2560, 8, 2, 128, 64, torch.bfloat16, "lowrank", 26, 0.15, 0.06, 0, 0),
    "bf16_T128_band_sink_B2": (2, 2048, 4, 1, 128, 128, torch.bfloat16, "lowrank", 20, 0.10, 0.04, 4, 1),
    "bf16_D64_T128_rescue_off": (1, 1536, 2, 2, 64, 128, torch.bfloat16, "iid", 4, 0.30, -1.0, 0, 0),
    "fp32_D128_T128": (1, 1024, 4, 2, 128, 128, torch.float32, "lowrank", 10, 0.25, 0.10, 1, 0),
    "bf16_D64_T64_G4": (1, 1024, 8, 2, 64, 64, torch.bfloat16, "lowrank", 10, 0.2, 0.08, 2, 1),
    # the other fp32 head-dim / block-size pairs
    "fp32_D128_T64": (1, 1536, 4, 4, 128, 64, torch.float32, "lowrank", 8, 0.2, 0.08, 1, 1),
    "fp32_D64_T128_G2": (2, 1024, 4, 2, 64, 128, torch.float32, "iid", 6, 0.3, 0.1, 0, 0),
    # both branches off: the forced band + sink only (a fixed-window mask)
    "bf16_forced_only_band8_sink1": (1, 4096, 4, 2, 128, 128, torch.bfloat16, "lowrank", 10,
                                     -1.0, -1.0, 8, 1),
}


def _run(name):
    B, S, Hq, Hkv, D, T, dt, model, nsp, pc, pr, band, sink = CASES[name]
    print(f"[prefill case {name}] B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} T={T} {dt}", flush=True)
    import free_sparse_attention_head_amd as fsa
    inp = workloads.prefill_inputs(B, S, Hq, Hkv, D, T, dtype=dt, model=model, n_spikes=nsp,
                                   seed=1000 + len(name), device="cpu")
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    c, r = fsa.block_stats(k, T)
    sel = fsa.select_blocks(q, c, r, T, pc, pr, band, sink, want_scores=True)
    o_sp, lse_sp = fsa.sparse_prefill_attn(q, k, v, T, sel["block_idx"], sel["block_cnt"])
    o_dn, lse_dn = fsa.sparse_prefill_attn(q, k, v, T)
    torch.cuda.synchronize()
    host = lambda t: None if t is None else t.cpu()
    res = {x: host(y) for x, y in dict(c=c, r=r, o_sp=o_sp, lse_sp=lse_sp, o_dn=o_dn, lse_dn=lse_dn,
                                     **sel).items()}
    res["inp"] = inp
    return res


_cache = {}


def run(name):
    if name not in _cache:
        _cache[name] = _run(name)
    return _cache[name]


@pytest.mark.parametrize("name", list(CASES))
def test_block_stats_parity(name):
    B, S, Hq, Hkv, D, T = CASES[name][:6]
    res = run(name)
    k = workloads.to_f64(res["inp"]["k"])
    for b in range(B):
        for g in range(Hkv):
            c, r = oracle.block_stats(k[b, :, g], T)
            assert np.abs(res["c"][b, g].double().numpy() - c).max() <= 1e-5
            assert np.abs(res["r"][b, g].double().numpy() - r).max() <= 1e-4 * max(1.0, r.max())


@pytest.mark.parametrize("name", list(CASES))
def test_select_blocks_parity(name):
    B, S, Hq, Hkv, D, T, dt, model, nsp, pc, pr, band, sink = CASES[name]
    res = run(name)
    nB = S // T
    q = workloads.to_f64(res["inp"]["q"])
    k = workloads.to_f64(res["inp"]["k"])
    n_diff = n_exc = 0
    for b in range(B):
        for g in range(Hkv):
            c, r = oracle.block_stats(k[b, :, g], T)
            for h in [x for x in range(Hq) if oracle.kv_head(x, Hq, Hkv) == g]:
                ref = oracle.select_blocks(oracle.pool_queries(q[b, :, h], T), c, r, pc, pr,
                                           band, sink)
                cnt = res["block_cnt"][b, h].numpy()
                lst = res["block_idx"][b, h].numpy()
                gm = lists_to_mask(lst, cnt, nB)
                # lists ascending, unique, causal; bitmask agrees with lists
                for i in range(nB):
                    li = lst[i, :cnt[i]]
                    assert (np.diff(li) > 0).all() and li.min() >= 0 and li.max() <= i
                assert (bits_to_mask(res["mask"][b, h].numpy(), nB) == gm).all()
                # GPU scores track the oracle's
                tri = np.tril(np.ones((nB, nB), dtype=bool))
                assert np.abs(res["score_c"][b, h].double().numpy()[tri] - ref["Sc"][tri]).max() <= 1e-4
                assert np.abs(res["score_r"][b, h].double().numpy()[tri] - ref["Sr"][tri]).max() <= 1e-3
                d, e = mask_diff_excused(gm, ref)
                n_diff += d
                n_exc += e
    print(f"[{name}] mask entries differing {n_diff}, excused near threshold {n_exc}")
    assert n_diff == n_exc


@pytest.mark.parametrize("name", list(CASES))
def test_sparse_prefill_attn_parity(name):
    B, S, Hq, Hkv, D, T, dt = CASES[name][:7]
    res = run(name)
    nB = S // T
    tol = TOL_F32 if dt == torch.float32 else TOL_BF16
    ltol = LSE_TOL_F32 if dt == torch.float32 else LSE_TOL_BF16
    q, k, v = (workloads.to_f64(res["inp"][x]) for x in ("q", "k", "v"))
    scale = 1 / math.sqrt(D)
    worst = worst_lse = 0.0
    for b in range(B):
        for h in range(Hq):
            g = oracle.kv_head(h, Hq, Hkv)
            m = lists_to_mask(res["block_idx"][b, h].numpy(), res["block_cnt"][b, h].numpy(), nB)
            o, lse = oracle.masked_attention(q[b, :, h], k[b, :, g], v[b, :, g], m, T, scale)
            err = np.abs(res["o_sp"][b, :, h].double().numpy() - o).max()
            worst = max(worst, err)
            assert err <= tol, (b, h, err)
            lerr = np.abs(res["lse_sp"][b, h].double().numpy() - lse).max()
            worst_lse = max(worst_lse, lerr)
            assert lerr <= ltol, (b, h, lerr)
    print(f"[{name}] sparse max-abs error {worst:.3e}, worst lse error {worst_lse:.3e}")


@pytest.mark.parametrize("name", list(CASES))
def test_dense_mode_matches_dense_oracle(name):
    B, S, Hq, Hkv, D, T, dt = CASES[name][:7]
    res = run(name)
    tol = TOL_F32 if dt == torch.float32 else TOL_BF16
    ltol = LSE_TOL_F32 if dt == torch.float32 else LSE_TOL_BF16
    q, k, v = (workloads.to_f64(res["inp"][x]) for x in ("q", "k", "v"))
    scale = 1 / math.sqrt(D)
    worst_lse = 0.0
    for b in range(B):
        for h in sorted({0, Hq - 1}):
            g = oracle.kv_head(h, Hq, Hkv)
            o, lse = oracle.dense_attention(q[b, :, h], k[b, :, g], v[b, :, g], scale)
            assert np.abs(res["o_dn"][b, :, h].double().numpy() - o).max() <= tol
            lerr = np.abs(res["lse_dn"][b, h].double().numpy() - lse).max()
            worst_lse = max(worst_lse, lerr)
            assert lerr <= ltol, (b, h, lerr)
    print(f"[{name}] dense worst lse error {worst_lse:.3e}")


def test_all_blocks_mask_equals_dense_kernel():
    """p_c = 1 selects every causal block; the sparse kernel then matches its
    own dense mode (same kernel, same block order) exactly."""
    import free_sparse_attention_head_amd as fsa
    inp = workloads.prefill_inputs(1, 1024, 4, 2, 128, 64, model="iid", n_spikes=0, seed=5,
                                   device="cpu")
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    c, r = fsa.block_stats(k, 64)
    sel = fsa.select_blocks(q, c, r, 64, 1.0, 0.1)
    nB = 16
    assert (sel["block_cnt"].cpu() == torch.arange(1, nB + 1, dtype=torch.int32)).all()
    o1, l1 = fsa.sparse_prefill_attn(q, k, v, 64, sel["block_idx"], sel["block_cnt"])
    o2, l2 = fsa.sparse_prefill_attn(q, k, v, 64)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_and_invalid_list_entries():
    """Rows with count 0 give O = 0 and lse = -inf; entries j > i or j < 0 are
    skipped without touching memory outside the tensors."""
    import free_sparse_attention_head_amd as fsa
    B, S, H, D, T = 1, 512, 2, 128, 64
    nB = S // T
    inp = workloads.prefill_inputs(B, S, H, H, D, T, model="iid", n_spikes=0, seed=9, device="cpu")
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    bidx = torch.zeros((B, H, nB, nB), dtype=torch.int32)
    bcnt = torch.zeros((B, H, nB), dtype=torch.int32)
    for i in range(nB):
        bidx[0, :, i, :3] = torch.tensor([-5, i, i + 3], dtype=torch.int32)
        bcnt[0, :, i] = 3
    bcnt[0, 1, 2] = 0
    o, lse = fsa.sparse_prefill_attn(q, k, v, T, bidx.cuda(), bcnt.cuda())
    o, lse = o.cpu(), lse.cpu()
    assert (o[0, 2 * T:3 * T, 1] == 0).all() and torch.isinf(lse[0, 1, 2 * T:3 * T]).all()
    qq, kk, vv = (workloads.to_f64(inp[x]) for x in ("q", "k", "v"))
    diag = np.eye(nB, dtype=bool)
    ref, _ = oracle.masked_attention(qq[0, :, 0], kk[0, :, 0], vv[0, :, 0], diag, T, 1 / math.sqrt(D))
    assert np.abs(o[0, :, 0].double().numpy() - ref).max() <= TOL_BF16


def test_anchor_selection_reused_by_a_later_layer():
    """Kascade-style prefill: the anchor layer's block lists drive a later
    layer's attention (queries and keys at cosine ~0.9 to the anchor's).  The
    result is exact masked attention of the later layer's Q, K, V under the
    anchor's mask."""
    import free_sparse_attention_head_amd as fsa
    Bb, S, Hq, Hkv, D, T = 1, 2048, 4, 2, 128, 64
    nB = S // T
    print(f"[prefill reuse case] S={S} Hq={Hq} Hkv={Hkv} D={D} T={T}", flush=True)
    base = workloads.prefill_inputs(Bb, S, Hq, Hkv, D, T, model="lowrank", n_spikes=20, seed=31,
                                    device="cpu")
    later = workloads.prefill_layer(base, 1, seed=31)
    q0, k0 = base["q"].cuda(), base["k"].cuda()
    c, r = fsa.block_stats(k0, T)
    sel = fsa.select_blocks(q0, c, r, T, 0.15, 0.06, 2, 1)
    q1, k1, v1 = (later[x].cuda() for x in ("q", "k", "v"))
    o, lse = fsa.sparse_prefill_attn(q1, k1, v1, T, sel["block_idx"], sel["block_cnt"])
    o, lse = o.cpu(), lse.cpu()
    q, k, v = (workloads.to_f64(later[x]) for x in ("q", "k", "v"))
    for h in range(Hq):
        m = lists_to_mask(sel["block_idx"][0, h].cpu().numpy(), sel["block_cnt"][0, h].cpu().numpy(), nB)
        g = oracle.kv_head(h, Hq, Hkv)
        ref, ref_lse = oracle.masked_attention(q[0, :, h], k[0, :, g], v[0, :, g], m, T,
                                               1 / math.sqrt(D))
        assert np.abs(o[0, :, h].double().numpy() - ref).max() <= TOL_BF16
        assert np.abs(lse[0, h].double().numpy() - ref_lse).max() <= LSE_TOL_BF16


def _exact_rows(res, pc, pr, band, sink, nB, rows=None):
    """Every checked mask row equals the selection rule applied exactly to the
    kernel's own fp32 scores: top k_of(p, i + 1) of each branch with ties to
    the lower block index (oracle.topk on the same values), union the forced
    blocks.  No near-threshold allowance: the same numbers, the same rule."""
    B, Hq = res["block_cnt"].shape[:2]
    rows = range(nB) if rows is None else rows
    bad = 0
    for b in range(B):
        for h in range(Hq):
            sc = res["score_c"][b, h].double().numpy()
            sr = res["score_r"][b, h].double().numpy()
            gm = lists_to_mask(res["block_idx"][b, h].numpy(), res["block_cnt"][b, h].numpy(), nB)
            bm = bits_to_mask(res["mask"][b, h].numpy(), nB)
            for i in rows:
                n = i + 1
                want = np.zeros(nB, dtype=bool)
                for p, s in ((pc, sc), (pr, sr)):
                    kk = oracle.k_of(p, n)
                    if kk > 0:
                        want[oracle.topk(s[i, :n], kk)[0]] = True
                want[:min(sink, n)] = True
                if band > 0:
                    want[max(0, i - band + 1):n] = True
                bad += int(not np.array_equal(gm[i], want)) + int(not np.array_equal(bm[i], want))
    assert bad == 0, bad


@pytest.mark.parametrize("name", list(CASES))
def test_selection_is_exact_top_k_of_kernel_scores(name):
    B, S, Hq, Hkv, D, T, dt, model, nsp, pc, pr, band, sink = CASES[name]
    _exact_rows(run(name), pc, pr, band, sink, S // T)


def _select_on(q, k, T, pc, pr, band=0, sink=0):
    import free_sparse_attention_head_amd as fsa
    c, r = fsa.block_stats(k, T)
    sel = fsa.select_blocks(q, c, r, T, pc, pr, band, sink, want_scores=True)
    torch.cuda.synchronize()
    return {x: y.cpu() for x, y in sel.items() if y is not None}


@pytest.mark.parametrize("kind", ["all_equal", "two_valued", "sparse_distinct"])
def test_selection_ties(kind):
    """Rows whose scores tie massively: every key the same (every score of a
    row equal, radius 0), keys alternating between two vectors block by block
    (two score values per row, the k-th inside a run of ties), and one
    distinct key block among equal ones.  nB = 200: several mask words, a
    ragged tail, four entries per lane."""
    S, Hq, Hkv, D, T = 12800, 2, 1, 64, 64
    nB = S // T
    print(f"[select ties {kind}] S={S} T={T} nB={nB}", flush=True)
    g = torch.Generator().manual_seed(77)
    q = torch.randn((1, S, Hq, D), generator=g)
    base = torch.randn(D, generator=g)
    other = torch.randn(D, generator=g)
    k = base.expand(1, S, Hkv, D).clone()
    if kind == "two_valued":
        blk = torch.arange(S) // T
        k[0, blk % 2 == 1, 0] = other
    elif kind == "sparse_distinct":
        k[0, 37 * T:38 * T, 0] = other
    q, k = q.to(torch.bfloat16).cuda(), k.to(torch.bfloat16).cuda()
    for pc, pr, band, sink in ((0.10, 0.04, 0, 0), (0.5, -1.0, 3, 2), (-1.0, 0.3, 0, 1)):
        _exact_rows(_select_on(q, k, T, pc, pr, band, sink), pc, pr, band, sink, nB)


@pytest.mark.parametrize("nB", [100, 300, 700, 1001, 2048, 4096])
def test_selection_long_rows(nB):
    """Row lengths for each selection instantiation not met elsewhere (2, 8,
    16, 32 and 64 entries per lane; nB = 1001 is no multiple of 4, so its rows
    are read with single-word loads): exact top-k of the kernel's own scores
    on sampled rows, the longest included."""
    T, D = 64, 64
    S = nB * T
    print(f"[select long rows] S={S} T={T} nB={nB}", flush=True)
    g = torch.Generator().manual_seed(nB)
    q = torch.randn((1, S, 1, D), generator=g).to(torch.bfloat16).cuda()
    k = torch.randn((1, S, 1, D), generator=g).to(torch.bfloat16).cuda()
    rows = sorted(set(x for x in [0, 1, 63, 64, 1000, nB // 2, nB - 2, nB - 1] if x < nB))
    _exact_rows(_select_on(q, k, T, 0.03, 0.01, 2, 1), 0.03, 0.01, 2, 1, nB, rows)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [64, 128])
def test_longest_prompt_block_lists(T, D):
    """nB = 4096 key blocks (the most a row may list), for both block sizes and
    head dims: the 4096-entry list instantiations.  Row i lists the sink block, one
    earlier block picked by a fixed hash and its own diagonal block; sampled
    rows (first and last blocks, around nB/2) against the oracle."""
    import free_sparse_attention_head_amd as fsa
    B, H = 1, 1
    nB = 4096
    S = nB * T
    print(f"[longest prompt] S={S} T={T} D={D} nB={nB}", flush=True)
    inp = workloads.prefill_inputs(B, S, H, H, D, T, model="iid", n_spikes=0, seed=31, device="cpu")
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    bidx = torch.zeros((B, H, nB, nB), dtype=torch.int32)
    bcnt = torch.zeros((B, H, nB), dtype=torch.int32)
    mask = np.zeros((nB, nB), dtype=bool)
    for i in range(nB):
        blocks = sorted({0, (i * 7919 + 13) % (i + 1), i})
        bidx[0, 0, i, :len(blocks)] = torch.tensor(blocks, dtype=torch.int32)
        bcnt[0, 0, i] = len(blocks)
        mask[i, blocks] = True
    o, lse = fsa.sparse_prefill_attn(q, k, v, T, bidx.cuda(), bcnt.cuda())
    o, lse = o.cpu(), lse.cpu()
    qq, kk, vv = (workloads.to_f64(inp[x])[0, :, 0] for x in ("q", "k", "v"))
    rows = []
    for i in (0, 1, nB // 2 - 1, nB // 2, nB - 2, nB - 1):
        rows += [i * T, i * T + T // 2, i * T + T - 1]
    ref, ref_lse = oracle.masked_attention_rows(qq, kk, vv, mask, T, 1 / math.sqrt(D), rows)
    got = o[0, rows, 0].double().numpy()
    assert np.abs(got - ref).max() <= TOL_BF16
    assert np.abs(lse[0, 0, rows].double().numpy() - ref_lse).max() <= 1e-2


@pytest.mark.parametrize("D,T", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("spike", [False, True])
def test_scores_growing_along_the_row(D, T, spike):
    """Scores that climb far above the first chunk's along each row: keys carry
    a growing component along the queries' shared direction (30-40 log2 units
    of growth over the prompt), and optionally one key with a logit about 150
    log2 units above its neighbours, past the fp32 range of exp2 against any
    earlier reference.  The attention kernel raises its reference exponent in
    both cases; the result is still the exact masked softmax (dense mode and a
    random ascending list with the diagonal block)."""
    import free_sparse_attention_head_amd as fsa
    B, S, Hq, Hkv = 1, 1024, 2, 1
    nB = S // T
    print(f"[growth case] D={D} T={T} spike={spike}", flush=True)
    rng = np.random.default_rng(77 + D + T + int(spike))
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q = 0.5 * rng.standard_normal((B, S, Hq, D)) + 4.0 * u
    ramp = 60.0 * np.arange(S) / S
    k = 0.5 * rng.standard_normal((B, S, Hkv, D)) + ramp[None, :, None, None] * u
    if spike:
        k[0, 700, 0] = 0.5 * rng.standard_normal(D) + 300.0 * u
    v = rng.standard_normal((B, S, Hkv, D))
    qt, kt, vt = (torch.tensor(x, dtype=torch.bfloat16) for x in (q, k, v))
    bidx = torch.zeros((B, Hq, nB, nB), dtype=torch.int32)
    bcnt = torch.zeros((B, Hq, nB), dtype=torch.int32)
    for h in range(Hq):
        for i in range(nB):
            keep = sorted(set(np.flatnonzero(rng.random(i) < 0.6).tolist()) | {i})
            bidx[0, h, i, :len(keep)] = torch.tensor(keep, dtype=torch.int32)
            bcnt[0, h, i] = len(keep)
    o_sp, l_sp = fsa.sparse_prefill_attn(qt.cuda(), kt.cuda(), vt.cuda(), T, bidx.cuda(), bcnt.cuda())
    o_dn, l_dn = fsa.sparse_prefill_attn(qt.cuda(), kt.cuda(), vt.cuda(), T)
    o_sp, l_sp, o_dn, l_dn = (x.cpu() for x in (o_sp, l_sp, o_dn, l_dn))
    qq, kk, vv = (workloads.to_f64(x) for x in (qt, kt, vt))
    scale = 1 / math.sqrt(D)
    worst = worst_lse = 0.0
    for h in range(Hq):
        m = lists_to_mask(bidx[0, h].numpy(), bcnt[0, h].numpy(), nB)
        for got_o, got_l, ref in (
                (o_sp, l_sp, oracle.masked_attention(qq[0, :, h], kk[0, :, 0], vv[0, :, 0], m, T, scale)),
                (o_dn, l_dn, oracle.dense_attention(qq[0, :, h], kk[0, :, 0], vv[0, :, 0], scale))):
            err = np.abs(got_o[0, :, h].double().numpy() - ref[0]).max()
            lerr = np.abs(got_l[0, h].double().numpy() - ref[1]).max()
            worst, worst_lse = max(worst, err), max(worst_lse, lerr)
            assert err <= TOL_BF16, (h, err)
            assert lerr <= LSE_TOL_BF16, (h, lerr)
    # the growth is real: the last row's LSE sits far above the first block's
    assert float(l_dn[0, 0, -1]) - float(l_dn[0, 0, T - 1]) > (60.0 if spike else 10.0)
    print(f"[growth D={D} T={T} spike={spike}] max-abs error {worst:.3e}, worst lse error {worst_lse:.3e}")

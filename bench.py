"""Benchmark of the head-aware sparse attention hot path on one MI355X.

One step runs every row of the hot path once over resident synthetic inputs:
  prefill, 128K prompt (B=1, S=131072, 32 query / 4 KV heads, D=128, bf16,
    key/query block 128, low-rank keys with 1% planted spikes, a kept
    1024-token diagonal band and the sink block): block_stats ->
    select_blocks (two-branch selector tuned to the target density) ->
    sparse_prefill_attn;
  Kascade decode group, 128K context (B=32, 32 query / 8 KV heads, D=128,
    bf16 KV in shuffled 16-token pages, 4 layers): topk_indices_scored
    (k=2048) at the anchor layer, the anchor's own attention at those indices
    from the kept keys' scores (V read only), then sparse_decode_attn at the
    same indices for the three reuse layers;
  segment decode, 1M context (B=4, same heads, shuffled pages): global, focus
    (2048-token chunk + 1024 local tail), local (1024) and streaming
    (4 sinks + 1024 window) masks, and one mixed batch whose sequences draw
    their modes by seed; caches flushed before each of the last four.
Outside the timed steps: own dense baselines, and the attention kernel at 3%
and 12% density and with the band + sink blocks only on the 128K prompt, and on
the 32K prompt with 64-token blocks at 10%, the Kascade group with one
pooled index set per KV head shared by its query heads, the anchor layer's
block lists reused by three later prefill layers, and the selectors (and the
ideal block top-k) compared at matched density on the 32K prompt for 64- and
128-token blocks at 5, 10 and 20% (skip all with --no-sweep).
Kernel times (medians, 50 timed steps after 5 warm-up steps by default) come
from HIP events on the launch stream.  The headline value
is the sparse prefill attention kernel's effective TFLOP/s on executed
blocks (4*T*T*D FLOP per executed query-block/key-block pair) over its mean
launch time in the timed steps, and so is each roofline's `achieved`; decode
is reported as admitted KV bytes per second.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--density 0.06]
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

PREFILL = dict(B=1, S=131072, Hq=32, Hkv=4, D=128, T=128, band=8, sink=1)
PREFILL_32K = dict(B=1, S=32768, Hq=32, Hkv=8, D=128, T=64, band=0, sink=0)
DECODE = dict(B=32, N=131072, Hq=32, Hkv=8, D=128, k=2048, layers=4)
SEGMENT = dict(B=4, N=1 << 20, Hq=32, Hkv=8, D=128)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """Per-kernel HIP-event timing on the current stream."""

    def __init__(self):
        self.ev = {}

    def run(self, name, fn):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        r = fn()
        e.record()
        self.ev.setdefault(name, []).append((s, e))
        return r

    def ms(self, name, skip=0):
        """(median, min) in ms of the recorded launches after the first `skip`."""
        xs = [s.elapsed_time(e) for s, e in self.ev[name][skip:]]
        return float(np.median(xs)), float(np.min(xs))

    def mean(self, name, skip=0):
        """Mean in ms of the recorded launches after the first `skip`."""
        return float(np.mean([s.elapsed_time(e) for s, e in self.ev[name][skip:]]))

    def clear(self):
        self.ev = {}


def tune_selector(fsa, q, c, r, P, density, out=None, branches="both"):
    """Bisect p_c (p_r = 0.4 p_c) until the selector's density is within
    0.25 points of the target; returns (p_c, density, selector outputs).
    branches "centroid" / "rescue" switch the other branch off and bisect the
    one left (its p is returned)."""
    nB = P["S"] // P["T"]
    visible = P["Hq"] * nB * (nB + 1) // 2
    lo, hi = 0.0, 1.0
    pc = dens = None
    for _ in range(30):
        pc = 0.5 * (lo + hi)
        p_c, p_r = {"both": (pc, 0.4 * pc), "centroid": (pc, -1.0), "rescue": (-1.0, pc)}[branches]
        out = fsa.select_blocks(q, c, r, P["T"], p_c, p_r, P["band"], P["sink"], out=out)
        dens = out["block_cnt"].sum().item() / visible
        if abs(dens - density) <= 0.0025:
            break
        if dens < density:
            lo = pc
        else:
            hi = pc
    log(f"[bench] S={P['S']} T={P['T']} selector ({branches}) p={pc:.5f} density={dens:.4f}")
    return pc, dens, out


def make_prefill(fsa, workloads, density, seed=1002, P=None):
    P = P or PREFILL
    log(f"[bench] generating prefill inputs S={P['S']} Hq={P['Hq']} Hkv={P['Hkv']} T={P['T']}")
    inp = workloads.prefill_inputs(1, P["S"], P["Hq"], P["Hkv"], P["D"], P["T"], model="lowrank",
                                   seed=seed, device="cuda")
    q, k, v = inp["q"], inp["k"], inp["v"]
    c, r = fsa.block_stats(k, P["T"])
    pc, dens, out = tune_selector(fsa, q, c, r, P, density)
    return dict(q=q, k=k, v=v, p_c=pc, p_r=0.4 * pc, density=dens, sel=out, c=c, r=r,
                spikes=inp["spikes"],
                o=torch.empty_like(q), lse=torch.empty((1, P["Hq"], P["S"]), dtype=torch.float32,
                                                      device="cuda"))


def time_attention(fsa, pf, P, reps=20):
    """Median / min of `reps` attention launches (after 2 warm-ups) on pf's selection."""
    tm = Timer()
    for _ in range(2 + reps):
        tm.run("a", lambda: fsa.sparse_prefill_attn(pf["q"], pf["k"], pf["v"], P["T"],
                                                    pf["sel"]["block_idx"], pf["sel"]["block_cnt"],
                                                    out=pf["o"], lse=pf["lse"]))
    torch.cuda.synchronize()
    xs = sorted(s.elapsed_time(e) for s, e in tm.ev["a"][2:])
    executed = int(pf["sel"]["block_cnt"].sum().item())
    flops = 4.0 * P["T"] * P["T"] * P["D"] * executed
    med = xs[len(xs) // 2]
    return {"density": round(pf["density"], 4), "attn_median_ms": round(med, 4),
            "attn_min_ms": round(xs[0], 4), "TFLOPs": round(flops / med / 1e9, 1),
            "frac_peak": round(flops / med / 1e9 / PEAK_BF16_TFLOPS, 4)}


def shared_set_recall(own, shared, G):
    """Per query head, the share of its own index set (own [B,Hq,k], -1 =
    empty) found in its KV head's shared set (shared [B,Hkv,m], ascending
    valid entries, then -1).  Returns [B,Hq] float."""
    big = torch.iinfo(torch.int32).max
    sh = torch.where(shared < 0, torch.full_like(shared, big), shared)
    sh = sh.repeat_interleave(G, dim=1).contiguous()          # [B, Hq, m]
    pos = torch.searchsorted(sh, own.contiguous()).clamp(max=sh.shape[2] - 1)
    hit = (torch.gather(sh, 2, pos) == own) & (own >= 0)
    return hit.sum(-1).float() / (own >= 0).sum(-1).clamp(min=1).float()


def decode_kv_shared(fsa, dc, reps=20):
    """GQA-shared index sets on the decode group's inputs, outside the timed
    steps (Kascade post, "Head-aware is the key to accuracy").  Two shared
    forms against the per-query-head sets of the timed steps:
      pooled: one top-k per KV head of the max over its query heads' scores
              (k entries, G times fewer K/V reads);
      union:  the union of the G per-head sets (every head keeps its own
              top-k; each chosen key is read once per KV head).
    Timings, and the accuracy of each on the anchor layer and the reuse
    layers: recall of each head's own top-k inside the shared set, the
    softmax mass kept (exp(lse_set - lse_dense), mean over heads and
    sequences), and the output's largest difference from the per-head
    result."""
    Dd = DECODE
    L = dc["layers"]
    G = Dd["Hq"] // Dd["Hkv"]
    idx = torch.empty((Dd["B"], Dd["Hkv"], Dd["k"]), dtype=torch.int32, device="cuda")
    kth = torch.empty((Dd["B"], Dd["Hkv"]), dtype=torch.float32, device="cuda")
    uni = torch.empty((Dd["B"], Dd["Hkv"], G * Dd["k"]), dtype=torch.int32, device="cuda")
    ucnt = torch.empty((Dd["B"], Dd["Hkv"]), dtype=torch.int32, device="cuda")
    own = dc["idx"]
    tm = Timer()
    for _ in range(2 + reps):
        tm.run("topk", lambda: fsa.topk_indices_kv(L[0]["q"], L[0]["k"], dc["page_table"],
                                                   dc["seq_lens"], Dd["k"], idx=idx, kth=kth,
                                                   ws=dc.get("topk_ws")))
        for li in range(Dd["layers"]):
            tm.run("dec", lambda li=li: fsa.sparse_decode_attn(
                L[li]["q"], L[li]["k"], L[li]["v"], dc["page_table"], dc["seq_lens"],
                mode=fsa.SEL_INDEX_KV, idx=idx, out=dc["out"][li], want_lse=False))
        tm.run("union", lambda: fsa.topk_union_kv(own, Dd["Hkv"], out=uni, cnt=ucnt))
        tm.run("dec_union", lambda: fsa.sparse_decode_attn(
            L[1]["q"], L[1]["k"], L[1]["v"], dc["page_table"], dc["seq_lens"],
            mode=fsa.SEL_INDEX_KV, idx=uni, out=dc["out"][1], want_lse=False))
    torch.cuda.synchronize()
    topk_ms = tm.ms("topk", skip=2)[0]
    dec_ms = tm.ms("dec", skip=2 * Dd["layers"])[0]
    union_ms = tm.ms("union", skip=2)[0]
    dec_union_ms = tm.ms("dec_union", skip=2)[0]
    layer_bytes = Dd["B"] * Dd["Hkv"] * Dd["k"] * kv_row_bytes(Dd["D"])
    union_bytes = int(ucnt.sum().item()) * kv_row_bytes(Dd["D"])
    own_bytes = Dd["B"] * Dd["Hq"] * Dd["k"] * kv_row_bytes(Dd["D"])
    # accuracy: the anchor layer itself (its per-head sets are its exact
    # top-k), the reuse layers 1-3 of the workload (fresh queries), and the
    # same reuse layers with queries correlated to the anchor's (0.9 q_0 +
    # sqrt(0.19) z, the correlation the workload gives the keys)
    recall = shared_set_recall(own, idx, G)

    def accuracy(q, layer):
        args = (q, L[layer]["k"], L[layer]["v"], dc["page_table"], dc["seq_lens"])
        _, lse_d = fsa.sparse_decode_attn(*args, mode=fsa.SEL_ALL)
        o_h, lse_h = fsa.sparse_decode_attn(*args, mode=fsa.SEL_INDEX, idx=own)
        o_p, lse_p = fsa.sparse_decode_attn(*args, mode=fsa.SEL_INDEX_KV, idx=idx)
        o_u, lse_u = fsa.sparse_decode_attn(*args, mode=fsa.SEL_INDEX_KV, idx=uni)
        r = {"mass_kept_" + key: round(torch.exp(lse - lse_d).mean().item(), 4)
             for key, lse in (("per_head", lse_h), ("pooled", lse_p), ("union", lse_u))}
        r["out_maxdiff_pooled"] = round((o_p.float() - o_h.float()).abs().max().item(), 4)
        r["out_maxdiff_union"] = round((o_u.float() - o_h.float()).abs().max().item(), 4)
        return r

    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    acc = {"anchor_layer": accuracy(L[0]["q"], 0)}
    for li in range(1, Dd["layers"]):
        acc[f"layer{li}"] = accuracy(L[li]["q"], li)
        z = torch.randn(L[0]["q"].shape, generator=gen, device="cuda")
        qc = (0.9 * L[0]["q"].float() + math.sqrt(0.19) * z).to(torch.bfloat16)
        acc[f"layer{li}_correlated_queries"] = accuracy(qc, li)
    return {"topk_kv_ms": round(topk_ms, 4), "decode_kv_ms": round(dec_ms, 4),
            "decode_kv_GBps": round(layer_bytes / (dec_ms * 1e-3) / 1e9, 1),
            "group_ms": round(topk_ms + Dd["layers"] * dec_ms, 4),
            "bytes_per_layer": layer_bytes,
            "pooled_recall_of_own_topk": {"mean": round(recall.mean().item(), 4),
                                          "min": round(recall.min().item(), 4)},
            "union_ms": round(union_ms, 4), "union_decode_ms": round(dec_union_ms, 4),
            "union_bytes_per_layer": union_bytes,
            "union_decode_GBps": round(union_bytes / (dec_union_ms * 1e-3) / 1e9, 1),
            "union_size_over_Gk": round(ucnt.float().mean().item() / (G * Dd["k"]), 4),
            "per_head_bytes_per_layer": own_bytes,
            "accuracy": acc}


def prefill_sweep(fsa, workloads, pf):
    """Attention timings outside the timed steps: the 128K prompt at 3% and 12%
    density (the steps run 6%), and the 32K prompt with 64-token blocks at 10%."""
    res = {}
    for dens in (0.03, 0.12):
        pc, d, sel = tune_selector(fsa, pf["q"], pf["c"], pf["r"], PREFILL, dens)
        res[f"128k_{int(round(dens * 100))}pct"] = time_attention(fsa, dict(pf, sel=sel, density=d), PREFILL)
        del sel
    # both selector branches off: the 1024-token band + sink block only, a
    # fixed-window mask whose cost grows linearly with the prompt
    nB = PREFILL["S"] // PREFILL["T"]
    sel = fsa.select_blocks(pf["q"], pf["c"], pf["r"], PREFILL["T"], -1.0, -1.0, PREFILL["band"],
                            PREFILL["sink"])
    d = sel["block_cnt"].sum().item() / (PREFILL["Hq"] * nB * (nB + 1) // 2)
    res["128k_band_sink_only"] = time_attention(fsa, dict(pf, sel=sel, density=d), PREFILL)
    del sel
    p32 = make_prefill(fsa, workloads, 0.10, seed=1001, P=PREFILL_32K)
    res["32k_block64_10pct"] = time_attention(fsa, p32, PREFILL_32K)
    return res, p32


def spike_recall(sel, spikes, device="cuda"):
    """Share of planted spikes whose key block is in the mask row of the query
    block and head the spike was aimed at."""
    if not spikes:
        return None
    b, g, tok, h, i = (torch.tensor(x, device=device) for x in zip(*spikes))
    T = sel["T"]
    j = tok // T
    words = sel["mask"][b, h, i, j // 32].to(torch.int64) & 0xffffffff
    return round(((words >> (j % 32)) & 1).float().mean().item(), 4)


def block_mass(fsa, q, k, v, T, lse_d):
    """Mean causal softmax mass of each query block i on each key block j, per
    query head: mass[h, i, j] = mean over the T queries t of block i of
    exp(lse_j(t) - lse_dense(t)), where lse_j comes from a sparse_prefill_attn
    launch whose every row i >= j lists block j alone (rows i < j list
    nothing and get mass 0).  One launch per key block; B = 1."""
    _, S, Hq, _ = q.shape
    nB = S // T
    dev = q.device
    mass = torch.zeros((Hq, nB, nB), dtype=torch.float32, device=dev)
    idx = torch.zeros((1, Hq, nB, nB), dtype=torch.int32, device=dev)
    cnt = torch.empty((1, Hq, nB), dtype=torch.int32, device=dev)
    ar = torch.arange(nB, device=dev)
    lse = torch.empty((1, Hq, S), dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    for j in range(nB):
        idx[..., 0] = j
        cnt.copy_((ar >= j).to(torch.int32).view(1, 1, nB).expand(1, Hq, nB))
        fsa.sparse_prefill_attn(q, k, v, T, idx, cnt, out=o, lse=lse)
        mass[:, :, j] = torch.exp(lse[0] - lse_d[0]).view(Hq, nB, T).mean(-1)
    return mass


def ideal_selection(mass, cnt):
    """Per row, the cnt[h, i] key blocks of largest mass (ties to the lower
    block index), as ascending block lists: the mask that keeps the most mass
    at those counts (no block selector can keep more)."""
    Hq, nB, _ = mass.shape
    order = torch.sort(-mass, dim=-1, stable=True).indices          # best block first
    rank_ok = torch.arange(nB, device=mass.device).view(1, 1, nB) < cnt[0].unsqueeze(-1)
    keep = torch.zeros_like(mass, dtype=torch.bool).scatter_(-1, order, rank_ok)
    ar = torch.arange(nB, device=mass.device).view(1, 1, nB)
    lists = torch.sort(torch.where(keep, ar, nB), dim=-1).values.clamp_(max=nB - 1)
    return lists.to(torch.int32).unsqueeze(0).contiguous(), cnt


def selector_quality(fsa, workloads, p32, densities=(0.05, 0.10, 0.20), blocks=(64, 128)):
    """Selectors compared at matched density on the 32K prompt (RBS-Attention
    post, "Experimental data": actual retention, matched density), for each
    key/query block size and target density: the merged two-branch selector,
    each branch alone, and the ideal block top-k at the merged selector's
    per-row counts.  Retention of token t = the share of its causal softmax
    mass on admitted keys = exp(lse_mask(t) - lse_dense(t)), both from the
    attention kernel.  Spike recall (64-token blocks, 10%): planted spikes
    whose block the selector keeps, on this prompt (spikes of norm 6) and on
    one with spikes of norm 2 sqrt(D), which then dominate the block radius."""
    names = {"both": "merged", "centroid": "centroid_only", "rescue": "rescue_only"}
    q, k, v = p32["q"], p32["k"], p32["v"]
    res = {"retention_mean": {}, "retention_p10": {}, "density": {},
           "spike_recall_norm6": {}, "spike_recall_norm2sqrtD": {}}
    for T in blocks:
        P = dict(PREFILL_32K, T=T)
        c, r = (p32["c"], p32["r"]) if T == PREFILL_32K["T"] else fsa.block_stats(k, T)
        _, lse_d = fsa.sparse_prefill_attn(q, k, v, T)
        mass = block_mass(fsa, q, k, v, T, lse_d)
        for density in densities:
            key = f"T{T}_d{int(round(density * 100)):02d}"
            rm, rp, dn = {}, {}, {}
            for br in ("both", "centroid", "rescue"):
                _, dens, sel = tune_selector(fsa, q, c, r, P, density, branches=br)
                lists = {names[br]: (sel["block_idx"], sel["block_cnt"])}
                if br == "both":
                    lists["ideal"] = ideal_selection(mass, sel["block_cnt"])
                for name, (bi, bc) in lists.items():
                    _, lse_m = fsa.sparse_prefill_attn(q, k, v, T, bi, bc)
                    ret = torch.exp(lse_m - lse_d).flatten()
                    rm[name] = round(ret.mean().item(), 4)
                    rp[name] = round(torch.quantile(ret, 0.10).item(), 4)
                    dn[name] = round(dens, 4)
                    del lse_m, ret
                if T == PREFILL_32K["T"] and abs(density - 0.10) < 1e-9:
                    res["spike_recall_norm6"][names[br]] = spike_recall(dict(sel, T=T), p32["spikes"])
                del sel, lists
            res["retention_mean"][key], res["retention_p10"][key], res["density"][key] = rm, rp, dn
        del mass, lse_d
        torch.cuda.empty_cache()
    P = PREFILL_32K
    alt = workloads.prefill_inputs(1, P["S"], P["Hq"], P["Hkv"], P["D"], P["T"], model="lowrank",
                                   spike_scale=2 * math.sqrt(P["D"]), seed=1011, device="cuda")
    c2, r2 = fsa.block_stats(alt["k"], P["T"])
    for br in ("both", "centroid", "rescue"):
        _, _, sel2 = tune_selector(fsa, alt["q"], c2, r2, P, 0.10, branches=br)
        res["spike_recall_norm2sqrtD"][names[br]] = spike_recall(dict(sel2, T=P["T"]), alt["spikes"])
        del sel2
    del alt, c2, r2
    torch.cuda.empty_cache()
    return res


def prefill_reuse(fsa, workloads, pf, anchor_path_ms, layers=4, reps=3):
    """Kascade-style prefill on the 128K prompt (outside the timed steps): the
    anchor layer's block lists (the steps' selection) drive the attention of
    three later layers whose queries and keys sit at cosine ~0.9 to the
    anchor's, against each layer running its own block_stats + select_blocks
    at the anchor's thresholds.  Also reported per later layer: the share of
    its own selection that the anchor's mask contains, and the retention
    (causal softmax mass kept) of both masks, from the kernel's LSE."""
    P = PREFILL
    T = P["T"]
    anchor = pf["sel"]
    base = {"q": pf["q"], "k": pf["k"], "v": pf["v"]}
    nwords = anchor["mask"].shape[-1]
    shifts = torch.arange(32, device="cuda", dtype=torch.int64)

    def nbits(m):
        w = m.to(torch.int64) & 0xffffffff
        return ((w.unsqueeze(-1) >> shifts) & 1).sum().item()

    tm = Timer()
    out = {"overlap_own_in_anchor": [], "retention_reused": [], "retention_own": []}
    lse_r = torch.empty_like(pf["lse"])
    lse_o = torch.empty_like(pf["lse"])
    for li in range(1, layers):
        L = workloads.prefill_layer(base, li, seed=1002)
        own = None
        for _ in range(2 + reps):
            tm.run(f"reuse_attn{li}", lambda: fsa.sparse_prefill_attn(
                L["q"], L["k"], L["v"], T, anchor["block_idx"], anchor["block_cnt"], out=pf["o"],
                lse=lse_r))
            cr = tm.run(f"own_stats{li}", lambda: fsa.block_stats(L["k"], T))
            own = tm.run(f"own_select{li}", lambda: fsa.select_blocks(
                L["q"], cr[0], cr[1], T, pf["p_c"], pf["p_r"], P["band"], P["sink"], out=own))
            tm.run(f"own_attn{li}", lambda: fsa.sparse_prefill_attn(
                L["q"], L["k"], L["v"], T, own["block_idx"], own["block_cnt"], out=pf["o"],
                lse=lse_o))
        _, lse_d = fsa.sparse_prefill_attn(L["q"], L["k"], L["v"], T)
        assert own["mask"].shape[-1] == nwords
        out["overlap_own_in_anchor"].append(round(nbits(own["mask"] & anchor["mask"]) / nbits(own["mask"]), 4))
        out["retention_reused"].append(round(torch.exp(lse_r - lse_d).mean().item(), 4))
        out["retention_own"].append(round(torch.exp(lse_o - lse_d).mean().item(), 4))
        del L, own, lse_d
        torch.cuda.empty_cache()
    later = range(1, layers)
    reuse = [tm.ms(f"reuse_attn{li}", skip=2)[0] for li in later]
    own = [sum(tm.ms(f"{x}{li}", skip=2)[0] for x in ("own_stats", "own_select", "own_attn"))
           for li in later]
    return dict(out, layers=layers, anchor_path_ms=round(anchor_path_ms, 4),
                reuse_attn_ms=[round(x, 4) for x in reuse], own_path_ms=[round(x, 4) for x in own],
                group_reused_ms=round(anchor_path_ms + sum(reuse), 4),
                group_own_ms=round(anchor_path_ms + sum(own), 4))


def make_decode(fsa, workloads, seed=1003):
    D = DECODE
    log(f"[bench] generating Kascade decode group B={D['B']} N={D['N']} layers={D['layers']}")
    d = workloads.decode_inputs(D["B"], D["N"], D["Hq"], D["Hkv"], D["D"], layers=D["layers"],
                                seed=seed, device="cuda")
    d["idx"] = torch.empty((D["B"], D["Hq"], D["k"]), dtype=torch.int32, device="cuda")
    d["scores"] = torch.empty((D["B"], D["Hq"], D["k"]), dtype=torch.float32, device="cuda")
    d["kth"] = torch.empty((D["B"], D["Hq"]), dtype=torch.float32, device="cuda")
    d["out"] = [torch.empty((D["B"], D["Hq"], D["D"]), dtype=torch.bfloat16, device="cuda")
                for _ in range(D["layers"])]
    return d


def make_segment(fsa, workloads, seed=1004):
    Sg = SEGMENT
    log(f"[bench] generating segment decode B={Sg['B']} N={Sg['N']}")
    d = workloads.decode_inputs(Sg["B"], Sg["N"], Sg["Hq"], Sg["Hkv"], Sg["D"], layers=1, seed=seed,
                                device="cuda")
    rng = np.random.default_rng(seed)
    n = Sg["N"]
    modes = {}
    for name, code in (("focus", fsa.SEG_FOCUS), ("local", fsa.SEG_LOCAL),
                       ("streaming", fsa.SEG_STREAMING)):
        segs = torch.zeros((Sg["B"], 2, 2), dtype=torch.int32)
        nseg = torch.zeros(Sg["B"], dtype=torch.int32)
        admitted = 0
        for b in range(Sg["B"]):
            st = int(rng.integers(0, n - 2048))
            rs = fsa.build_segments(code, n, chunk_start=st, chunk_len=2048, local_len=1024,
                                    n_sink=4, page=16)
            nseg[b] = len(rs)
            for x, (a, e) in enumerate(rs):
                segs[b, x, 0], segs[b, x, 1] = a, e
                admitted += e - a
        modes[name] = dict(segs=segs.cuda(), nseg=nseg.cuda(), admitted=admitted)
    # one mixed batch: each sequence's mode drawn by seed
    codes = {"global": fsa.SEG_GLOBAL, "focus": fsa.SEG_FOCUS, "local": fsa.SEG_LOCAL,
             "streaming": fsa.SEG_STREAMING}
    draw = [list(codes)[int(x)] for x in np.random.default_rng(seed + 1).integers(0, 4, Sg["B"])]
    segs = torch.zeros((Sg["B"], 2, 2), dtype=torch.int32)
    nseg = torch.zeros(Sg["B"], dtype=torch.int32)
    admitted = 0
    for b, name in enumerate(draw):
        st = int(rng.integers(0, n - 2048))
        rs = fsa.build_segments(codes[name], n, chunk_start=st, chunk_len=2048, local_len=1024,
                                n_sink=4, page=16)
        nseg[b] = len(rs)
        for x, (a, e) in enumerate(rs):
            segs[b, x, 0], segs[b, x, 1] = a, e
            admitted += e - a
    modes["mixed"] = dict(segs=segs.cuda(), nseg=nseg.cuda(), admitted=admitted, draw=draw)
    d["modes"] = modes
    d["out"] = torch.empty((Sg["B"], Sg["Hq"], Sg["D"]), dtype=torch.bfloat16, device="cuda")
    d["flush"] = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    return d


def kv_row_bytes(D):
    return 2 * D * 2  # one K row + one V row, bf16


def step(fsa, pf, dc, sg, tm, parts=("prefill", "decode", "segment")):
    P, Dd, Sg = PREFILL, DECODE, SEGMENT
    if "prefill" in parts:
        step_prefill(fsa, pf, tm)
    if "decode" in parts:
        step_decode(fsa, dc, tm)
    if "segment" in parts:
        step_segment(fsa, sg, tm)


def step_prefill(fsa, pf, tm):
    P = PREFILL
    tm.run("block_stats", lambda: fsa.block_stats(pf["k"], P["T"], pf["c"], pf["r"]))
    tm.run("select_blocks", lambda: fsa.select_blocks(pf["q"], pf["c"], pf["r"], P["T"], pf["p_c"],
                                                      pf["p_r"], P["band"], P["sink"],
                                                      out=pf["sel"], ws=pf.get("sel_ws")))
    tm.run("sparse_prefill_attn", lambda: fsa.sparse_prefill_attn(
        pf["q"], pf["k"], pf["v"], P["T"], pf["sel"]["block_idx"], pf["sel"]["block_cnt"],
        out=pf["o"], lse=pf["lse"]))


def step_decode(fsa, dc, tm):
    """Kascade group: anchor top-k (with the kept keys' scores), the anchor's
    attention at its top-k from those scores (V read only), then index decode
    for the reuse layers."""
    Dd = DECODE
    L = dc["layers"]
    tm.run("topk_indices", lambda: fsa.topk_indices_scored(
        L[0]["q"], L[0]["k"], dc["page_table"], dc["seq_lens"], Dd["k"], idx=dc["idx"],
        scores=dc["scores"], kth=dc["kth"], ws=dc.get("topk_ws")))
    tm.run("decode_index_anchor", lambda: fsa.sparse_decode_attn(
        L[0]["q"], L[0]["k"], L[0]["v"], dc["page_table"], dc["seq_lens"],
        mode=fsa.SEL_INDEX_SCORED, idx=dc["idx"], scores=dc["scores"], out=dc["out"][0],
        want_lse=False, ws=dc.get("dec_ws")))
    for li in range(1, Dd["layers"]):
        tm.run("decode_index", lambda li=li: fsa.sparse_decode_attn(
            L[li]["q"], L[li]["k"], L[li]["v"], dc["page_table"], dc["seq_lens"],
            mode=fsa.SEL_INDEX, idx=dc["idx"], out=dc["out"][li], want_lse=False,
            ws=dc.get("dec_ws")))


def step_segment(fsa, sg, tm):
    """1M-context segment decode: global, then the small modes after a cache flush."""
    G = sg["layers"][0]
    tm.run("decode_global", lambda: fsa.sparse_decode_attn(
        G["q"], G["k"], G["v"], sg["page_table"], sg["seq_lens"], mode=fsa.SEL_ALL,
        out=sg["out"], want_lse=False, ws=sg.get("ws")))
    for name, m in sg["modes"].items():
        sg["flush"].view(torch.int64).sum()  # read-evict L2 / MALL so the small modes read HBM
        tm.run("decode_" + name, lambda m=m: fsa.sparse_decode_attn(
            G["q"], G["k"], G["v"], sg["page_table"], sg["seq_lens"], mode=fsa.SEL_SEGMENT,
            segments=m["segs"], n_seg=m["nseg"], n_split=m.get("n_split", 0), out=sg["out"],
            want_lse=False, ws=sg.get("ws")))


def prefill_flops(pf):
    P = PREFILL
    executed = int(pf["sel"]["block_cnt"].sum().item())
    return 4.0 * P["T"] * P["T"] * P["D"] * executed, executed


def _threads():
    """(BLAS threads numpy's matmuls use, cores this process may run on)."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([x.get("num_threads", 1) for x in threadpool_info()
                    if x.get("user_api") == "blas"] + [1])
    except Exception:
        blas = 1
    return blas, len(os.sched_getaffinity(0))


def _host_seq(pool, page_table_row, n, g):
    """One sequence's pages of KV head g, copied to the host whole and widened
    to float64 (untimed), with its page-table entries remapped to that copy."""
    import workloads
    ids = page_table_row[: (n + 15) // 16].long()
    uniq, inv = torch.unique(ids, sorted=True, return_inverse=True)
    return workloads.to_f64(pool[uniq, g:g + 1]), inv.cpu().numpy()


def cpu_baseline(pf, dc, sg, budget_s=12.0):
    """The fp64 oracle timed on bounded samples of the same workloads, on the
    host's cores (compute only: device-to-host copies and fp64 widening are
    outside the timed regions).
      prefill: whole query blocks of head 0 at the benchmark's mask, from the
               last block backwards, for about budget_s seconds (TFLOP/s on
               executed blocks);
      top-k:   anchor scores and exact top-k of a few query heads over the
               128K decode context (GB/s of keys scanned, bf16 size);
      index decode: attention of a few query heads at their 2048 indices,
               through the paged gather (GB/s of admitted K+V, bf16 size);
      global segment decode: a few query heads over a 1M-token sequence
               (GB/s of admitted K+V, bf16 size).
    numpy matmuls use the BLAS threads; sorts and top-k run on one thread."""
    import oracle
    import workloads
    P = PREFILL
    T = P["T"]
    nB = P["S"] // T
    h, g = 0, 0
    q = workloads.to_f64(pf["q"][0, :, h])
    k = workloads.to_f64(pf["k"][0, :, g])
    v = workloads.to_f64(pf["v"][0, :, g])
    cnt = pf["sel"]["block_cnt"][0, h].cpu().numpy()
    lst = pf["sel"]["block_idx"][0, h].cpu().numpy()
    scale = 1 / math.sqrt(P["D"])
    done_blocks = 0
    t_cpu = 0.0
    rows = 0
    for i in range(nB - 1, -1, -1):
        m = np.zeros((nB, nB), dtype=bool)
        m[i, lst[i, :cnt[i]]] = True
        t0 = time.perf_counter()
        oracle.masked_attention_rows(q, k, v, m, T, scale, np.arange(i * T, (i + 1) * T))
        t_cpu += time.perf_counter() - t0
        done_blocks += int(cnt[i])
        rows += 1
        if t_cpu >= budget_s:
            break
    flops = 4.0 * T * T * P["D"] * done_blocks
    blas, affinity = _threads()
    legs = {}
    # decode legs (128K Kascade group, 1M global segment)
    Dd, Sg = DECODE, SEGMENT
    row = 2 * Dd["D"] * 2                       # one K + one V row, bf16 bytes
    L = dc["layers"]
    sc = 1 / math.sqrt(Dd["D"])
    t_topk = t_idx = 0.0
    heads = [(0, 0), (5, 17), (31, 31)]
    idx = dc["idx"].cpu().numpy()
    for b, hh in heads:
        gg = oracle.kv_head(hh, Dd["Hq"], Dd["Hkv"])
        qh = workloads.to_f64(L[0]["q"][b, hh])
        subk, pt = _host_seq(L[0]["k"], dc["page_table"][b], Dd["N"], gg)
        subv, _ = _host_seq(L[0]["v"], dc["page_table"][b], Dd["N"], gg)
        t0 = time.perf_counter()
        K = oracle.gather_pages(subk, pt, Dd["N"], 0)
        oracle.anchor_topk(qh, K, Dd["k"])
        t_topk += time.perf_counter() - t0
        t0 = time.perf_counter()
        V = oracle.gather_pages(subv, pt, Dd["N"], 0)
        oracle.index_attention(qh, K, V, idx[b, hh], sc)
        t_idx += time.perf_counter() - t0
        del K, V, subk, subv
    n_h = len(heads)
    legs["topk"] = {"value": round(n_h * Dd["N"] * Dd["D"] * 2 / t_topk / 1e9, 3), "unit": "GB/s",
                    "sample": f"{n_h} query heads x {Dd['N']} keys, k={Dd['k']} ({t_topk:.1f} s)"}
    legs["index_decode"] = {"value": round(n_h * Dd["k"] * row / t_idx / 1e9, 4), "unit": "GB/s",
                            "sample": f"{n_h} query heads x {Dd['k']} indices with their sequence's "
                                      f"paged gather ({t_idx:.1f} s)"}
    G = sg["layers"][0]
    t_seg = 0.0
    seg_heads = [(0, 0), (3, 29)]
    for b, hh in seg_heads:
        gg = oracle.kv_head(hh, Sg["Hq"], Sg["Hkv"])
        qh = workloads.to_f64(G["q"][b, hh])
        subk, pt = _host_seq(G["k"], sg["page_table"][b], Sg["N"], gg)
        subv, _ = _host_seq(G["v"], sg["page_table"][b], Sg["N"], gg)
        t0 = time.perf_counter()
        K = oracle.gather_pages(subk, pt, Sg["N"], 0)
        V = oracle.gather_pages(subv, pt, Sg["N"], 0)
        oracle.segment_attention(qh, K, V, [(0, Sg["N"])], sc)
        t_seg += time.perf_counter() - t0
        del K, V, subk, subv
    legs["global_segment_decode"] = {
        "value": round(len(seg_heads) * Sg["N"] * row / t_seg / 1e9, 4), "unit": "GB/s",
        "sample": f"{len(seg_heads)} query heads over {Sg['N']} tokens ({t_seg:.1f} s)"}
    return {"value": flops / t_cpu / 1e12, "unit": "TFLOP/s", "cores": min(blas, affinity),
            "blas_threads": blas, "affinity_cores": affinity, "kind": "oracle",
            "sample": f"fp64 masked attention, head 0, last {rows} of {nB} query blocks "
                      f"({done_blocks} executed blocks, {t_cpu:.1f} s); numpy matmuls on the "
                      f"BLAS threads, sorts and top-k on one thread",
            "legs": legs}


def profiled_traffic(key, source):
    """HBM bytes per launch recorded by the committed rocprofv3 PMC summary
    (FETCH_SIZE/WRITE_SIZE, copy-calibrated), or None when the kernel source
    has changed since the counters were taken."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", "hbm_traffic_128k_1m.md")
    src = os.path.join(ROOT, "free_sparse_attention_head_amd", "csrc", source)
    try:
        text = open(prof).read()
        cur = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    tag = source + " sha256 prefix: "
    at = text.find(tag)
    if at < 0 or text[at + len(tag):at + len(tag) + 16] != cur:
        return None
    for line in text.splitlines():
        if line.startswith(key + ":"):
            return int(line.split(":")[1])
    return None


def attach_workspaces(fsa, pf, dc, sg):
    """Pre-allocate every workspace so the timed region allocates nothing."""
    P, Dd, Sg = PREFILL, DECODE, SEGMENT
    if pf is not None:
        pshape = fsa._lib.PrefillShape(1, P["S"], P["Hq"], P["Hkv"], P["D"], P["T"])
        pf["sel_ws"] = torch.empty(fsa.workspace_size("select", pshape), dtype=torch.uint8,
                                   device="cuda")
    if dc is not None:
        dshape = fsa._lib.DecodeShape(Dd["B"], Dd["Hq"], Dd["Hkv"], Dd["D"], 16,
                                      dc["num_pages"], dc["max_pages"], Dd["N"])
        dc["topk_ws"] = torch.empty(fsa.workspace_size("topk", dshape, Dd["k"]), dtype=torch.uint8,
                                    device="cuda")
        sel = fsa._lib.KvSelect(fsa.SEL_INDEX, None, Dd["k"], None, None, 0, 0)
        dc["dec_ws"] = torch.empty(fsa.workspace_size("decode", dshape, sel), dtype=torch.uint8,
                                   device="cuda")
    if sg is not None:
        sshape = fsa._lib.DecodeShape(Sg["B"], Sg["Hq"], Sg["Hkv"], Sg["D"], 16, sg["num_pages"],
                                      sg["max_pages"], Sg["N"])
        ssel = fsa._lib.KvSelect(fsa.SEL_ALL, None, 0, None, None, 0, 0)
        wsb = fsa.workspace_size("decode", sshape, ssel)
        sg["ws"] = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        # small modes: one split per 256 admitted tokens of a sequence, at least 8
        # (measured best for focus / local / streaming), within the workspace
        for name, m in sg["modes"].items():
            per_seq = m["admitted"] // Sg["B"]
            m["n_split"] = max(1, min(wsb // (Sg["B"] * Sg["Hq"] * (Sg["D"] + 2) * 4),
                                      max(8, per_seq // 256)))


def profile_only(fsa, workloads, args):
    """Run one part of the step (for profilers); prints per-kernel times."""
    pf = make_prefill(fsa, workloads, args.density) if args.only == "prefill" else None
    dc = make_decode(fsa, workloads) if args.only == "decode" else None
    sg = make_segment(fsa, workloads) if args.only == "segment" else None
    attach_workspaces(fsa, pf, dc, sg)
    tm = Timer()
    for _ in range(args.warmup):
        step(fsa, pf, dc, sg, tm, parts=(args.only,))
    torch.cuda.synchronize()
    tm.clear()
    for _ in range(args.steps):
        step(fsa, pf, dc, sg, tm, parts=(args.only,))
    torch.cuda.synchronize()
    if args.copy_probe:
        copy_probe()
    print(json.dumps({"only": args.only, "kernel_ms": {n: round(tm.ms(n)[0], 4) for n in tm.ev}}))


def copy_probe():
    """A plain 1 GiB device-to-device copy, run 3 times: its FETCH_SIZE /
    WRITE_SIZE counters calibrate the counter units (known 1 GiB each way)."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--density", type=float, default=0.06)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the prefill density sweep")
    ap.add_argument("--no-quality", action="store_true",
                    help="skip the selector comparison at matched density")
    ap.add_argument("--only", choices=["prefill", "decode", "segment"], default=None,
                    help="profile one part of the step only (not a benchmark result)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run a 1 GiB device copy at the end (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the hot path here is a single-GPU kernel library; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import workloads
    from free_sparse_attention_head_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from free_sparse_attention_head_amd import build
        build.build()
    import free_sparse_attention_head_amd as fsa
    torch.cuda.set_device(0)

    if args.only:
        return profile_only(fsa, workloads, args)
    pf = make_prefill(fsa, workloads, args.density)
    dc = make_decode(fsa, workloads)
    sg = make_segment(fsa, workloads)
    attach_workspaces(fsa, pf, dc, sg)
    P, Dd, Sg = PREFILL, DECODE, SEGMENT
    tm = Timer()
    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(fsa, pf, dc, sg, tm)
    torch.cuda.synchronize()
    tm.clear()
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(fsa, pf, dc, sg, tm)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    log("[bench] timed region done")

    k_ms = {n: tm.ms(n) for n in tm.ev}
    flops, executed = prefill_flops(pf)
    attn_ms = tm.mean("sparse_prefill_attn")  # the rooflines take mean launch times
    tflops = flops / (attn_ms * 1e-3) / 1e12
    path_ms = sum(k_ms[n][0] for n in ("block_stats", "select_blocks", "sparse_prefill_attn"))
    idx_bytes = Dd["B"] * Dd["Hq"] * Dd["k"] * kv_row_bytes(Dd["D"])
    reuse_ms = tm.mean("decode_index")
    reuse_gbps = idx_bytes / (reuse_ms * 1e-3) / 1e9
    scan_bytes = Dd["B"] * Dd["N"] * Dd["Hkv"] * Dd["D"] * 2
    topk_ms = k_ms["topk_indices"][0]
    group_ms = topk_ms + k_ms["decode_index_anchor"][0] + 3 * k_ms["decode_index"][0]  # medians
    group_bytes = scan_bytes + 4 * idx_bytes - Dd["B"] * Dd["Hq"] * Dd["k"] * Dd["D"] * 2
    seg = {}
    for name in ("global", "focus", "local", "streaming", "mixed"):
        if name == "global":
            admitted = Sg["B"] * Sg["N"]
        else:
            admitted = sg["modes"][name]["admitted"]
        byts = admitted * Sg["Hkv"] * kv_row_bytes(Sg["D"])
        ms = k_ms["decode_" + name][0]
        seg[name] = {"ms": round(ms, 4), "GB": round(byts / 1e9, 4),
                     "GBps": round(byts / (ms * 1e-3) / 1e9, 1),
                     "frac_hbm": round(byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    seg["mixed"]["modes"] = sg["modes"]["mixed"]["draw"]

    dense = {}
    if not args.no_dense:
        log("[bench] own dense baselines")
        tmd = Timer()
        for _ in range(2):
            tmd.run("dense_prefill", lambda: fsa.sparse_prefill_attn(pf["q"], pf["k"], pf["v"], P["T"],
                                                                      out=pf["o"], lse=pf["lse"]))
            for li in range(Dd["layers"]):
                tmd.run("dense_decode", lambda li=li: fsa.sparse_decode_attn(
                    dc["layers"][li]["q"], dc["layers"][li]["k"], dc["layers"][li]["v"],
                    dc["page_table"], dc["seq_lens"], mode=fsa.SEL_ALL, out=dc["out"][li],
                    want_lse=False, ws=dc.get("dense_ws")))
        torch.cuda.synchronize()
        nB = P["S"] // P["T"]
        dflops = 4.0 * P["T"] ** 2 * P["D"] * P["Hq"] * nB * (nB + 1) // 2
        dms = tmd.ms("dense_prefill", skip=1)[0]
        ddec = tmd.ms("dense_decode", skip=4)[0] * 4
        dense = {"prefill_ms": round(dms, 3), "prefill_TFLOPs": round(dflops / dms / 1e9, 1),
                 "prefill_speedup": round(dms / attn_ms, 2),
                 "decode_4layers_ms": round(ddec, 3),
                 "decode_4layers_GBps": round(4 * Dd["B"] * Dd["N"] * Dd["Hkv"] * kv_row_bytes(Dd["D"]) /
                                              (ddec * 1e-3) / 1e9, 1),
                 "decode_group_speedup": round(ddec / group_ms, 2)}

    sweep, kv_shared, quality, reuse = {}, {}, {}, {}
    if not args.no_sweep:
        log("[bench] anchor selection reused by three later prefill layers")
        reuse = prefill_reuse(fsa, workloads, pf, path_ms)
        log("[bench] prefill density sweep and 32K prompt")
        sweep, p32 = prefill_sweep(fsa, workloads, pf)
        if not args.no_quality:
            log("[bench] selectors at matched density (32K prompt)")
            quality = selector_quality(fsa, workloads, p32)
        del p32
        torch.cuda.empty_cache()
        log("[bench] per-KV-head Kascade variant")
        kv_shared = decode_kv_shared(fsa, dc)

    if args.copy_probe:
        copy_probe()

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu oracle baseline")
        cpu = cpu_baseline(pf, dc, sg)

    res = {
        "metric": "sparse prefill TFLOP/s & decode KV GB/s at 128K ctx, % roofline, 1 MI355X",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "sparse prefill 128K (B=1, 32q/4kv heads, D=128, block 128, "
                               f"density {pf['density']:.4f}) + Kascade decode 128K (B=32, 32q/8kv, "
                               "k=2048, 4 layers) + segment decode 1M (B=4)",
                   "global_batch": 1, "seq_len": P["S"], "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiled_traffic("prefill_attn_traffic_bytes_per_launch",
                                                 "prefill_attn_bf16.hip"),
                     "kernel": "prefill_attn_bf16_kernel<128,128>",
                     "flop_per_launch": flops, "executed_blocks": executed,
                     "avg_launch_ms": round(attn_ms, 4)},
        "roofline_decode": {"bound": "hbm", "achieved": round(reuse_gbps, 1), "peak": PEAK_HBM_GBPS,
                            "unit": "GB/s", "frac": round(reuse_gbps / PEAK_HBM_GBPS, 4),
                            "traffic": profiled_traffic("decode_index_traffic_bytes_per_launch",
                                                        "decode_attn.hip"),
                            "kernel": "decode_split_kernel<128,1,INDEX> + combine",
                            "bytes_per_launch": idx_bytes, "avg_launch_ms": round(reuse_ms, 4)},
        "prefill": {"density": round(pf["density"], 4), "p_c": pf["p_c"], "p_r": pf["p_r"],
                    "attn_ms": round(attn_ms, 4),
                    "attn_median_ms": round(k_ms["sparse_prefill_attn"][0], 4),
                    "attn_min_ms": round(k_ms["sparse_prefill_attn"][1], 4),
                    "block_stats_ms": round(k_ms["block_stats"][0], 4),
                    "select_ms": round(k_ms["select_blocks"][0], 4),
                    "path_ms": round(path_ms, 4), "path_TFLOPs": round(flops / path_ms / 1e9, 2)},
        "decode": {"topk_ms": round(topk_ms, 4),
                   "topk_scan_GBps": round(scan_bytes / (topk_ms * 1e-3) / 1e9, 1),
                   "anchor_decode_ms": round(k_ms["decode_index_anchor"][0], 4),
                   "anchor_decode_GBps": round(idx_bytes / 2 / (k_ms["decode_index_anchor"][0] * 1e-3)
                                               / 1e9, 1),
                   "anchor_ms": round(topk_ms + k_ms["decode_index_anchor"][0], 4),
                   "reuse_decode_ms": round(reuse_ms, 4), "reuse_GBps": round(reuse_gbps, 1),
                   "group_ms": round(group_ms, 4),
                   "group_GBps": round(group_bytes / (group_ms * 1e-3) / 1e9, 1)},
        "segment_1M": seg,
        "dense": dense,
        "prefill_sweep": sweep,
        "decode_kv_shared": kv_shared,
        "selector_quality": quality,
        "prefill_reuse": reuse,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()

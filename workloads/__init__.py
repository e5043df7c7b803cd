"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random tensors and lays them out; it holds none of the
attention method's arithmetic, and neither the HIP library nor the oracle
imports it.  Callers hand the same tensors to both sides (the oracle receives
the exact bf16/fp32 values the GPU received, widened to float64).

Recipes (the shapes, sizes and structure of the source pages' workloads; the
public benchmarks the pages measure on are not available, so these stand in
for them):
  * prefill "iid": Q, K, V i.i.d. N(0,1).
  * prefill "lowrank": per KV head g, K = z A_g^T and V = y B_g^T with A_g, B_g
    in R^{D x 16} drawn N(0, 1/16) and z, y ~ N(0, I_16) per token (unit
    variance entries, rank 16); Q i.i.d. N(0,1).
  * planted spikes (both models): a key row replaced by 6 * u / ||u||, where u
    is the mean query of a randomly chosen query block i >= the key's block,
    of a randomly chosen query head of the key's GQA group -- a single highly
    relevant token hidden in a block ("mean dilution").
  * decode: KV cache in 16-token pages [num_pages, Hkv, 16, D] bf16, pages of
    all sequences scattered by a seeded random permutation of the pool;
    layer 0 keys/values/queries i.i.d. N(0,1); later layers of a Kascade group
    use fresh queries and values and keys 0.9 * K_0 + sqrt(0.19) * Z (cosine
    ~0.9 to the anchor layer's keys).
  * prefill layer group (anchor selection reused by later layers): layer l > 0
    has Q_l = 0.9 * Q_0 + sqrt(0.19) * Z_q and K_l = 0.9 * K_0 + sqrt(0.19) * Z_k
    (the anchor layer's planted spikes carry over, scaled) and fresh V_l.
Every tensor comes from its own generator stream seeded seed * 100 + id.
"""

import math

import numpy as np
import torch

PAGE = 16


def _gen(device, seed, sid):
    g = torch.Generator(device=device)
    g.manual_seed(seed * 100 + sid)
    return g


def _randn(shape, device, seed, sid, dtype=torch.float32):
    return torch.randn(shape, generator=_gen(device, seed, sid), device=device, dtype=dtype)


def _randint(high, shape, device, seed, sid):
    return torch.randint(0, high, shape, generator=_gen(device, seed, sid), device=device)


def _randperm(n, device, seed, sid):
    return torch.randperm(n, generator=_gen(device, seed, sid), device=device)


def prefill_inputs(B, S, Hq, Hkv, D, T, dtype=torch.bfloat16, model="lowrank",
                   n_spikes=None, spike_frac=0.01, spike_scale=6.0, seed=0, device="cpu"):
    """Q [B,S,Hq,D], K, V [B,S,Hkv,D] in `dtype`, plus the planted spike list.

    n_spikes: spikes per (batch, KV head); default round(spike_frac * S).
    Returns dict(q, k, v, spikes) where spikes is a list of
    (b, g, token, query_head, query_block).
    """
    assert S % T == 0 and Hq % Hkv == 0
    G = Hq // Hkv
    nB = S // T
    q = _randn((B, S, Hq, D), device, seed, 1)
    if model == "iid":
        k = _randn((B, S, Hkv, D), device, seed, 2)
        v = _randn((B, S, Hkv, D), device, seed, 3)
    elif model == "lowrank":
        r = 16
        A = _randn((B, Hkv, D, r), device, seed, 4) / math.sqrt(r)
        Bm = _randn((B, Hkv, D, r), device, seed, 5) / math.sqrt(r)
        k = torch.empty((B, S, Hkv, D), device=device, dtype=torch.float32)
        v = torch.empty((B, S, Hkv, D), device=device, dtype=torch.float32)
        for b in range(B):
            for g in range(Hkv):
                z = _randn((S, r), device, seed, 10 + 2 * (b * Hkv + g))
                y = _randn((S, r), device, seed, 11 + 2 * (b * Hkv + g))
                k[b, :, g] = z @ A[b, g].T
                v[b, :, g] = y @ Bm[b, g].T
                del z, y
    else:
        raise ValueError(model)

    if n_spikes is None:
        n_spikes = int(round(spike_frac * S))
    spikes = []
    rng = np.random.default_rng(seed * 100 + 7)
    for b in range(B):
        for g in range(Hkv):
            if model == "iid":
                blocks = rng.choice(nB, size=min(n_spikes, nB), replace=False)
                toks = blocks * T + rng.integers(0, T, size=blocks.size)
            else:
                toks = rng.choice(S, size=n_spikes, replace=False)
            for tok in np.sort(toks):
                jb = int(tok) // T
                i = int(rng.integers(jb, nB))
                h = g * G + int(rng.integers(0, G))
                u = q[b, i * T:(i + 1) * T, h].double().mean(0)
                k[b, int(tok), g] = (spike_scale * u / u.norm()).float()
                spikes.append((b, g, int(tok), h, i))
    return {"q": q.to(dtype), "k": k.to(dtype), "v": v.to(dtype), "spikes": spikes}


def prefill_layer(base, layer, corr=0.9, seed=0):
    """Layer `layer` >= 1 of a prefill group whose anchor layer is `base` (a
    prefill_inputs dict): queries and keys corr * anchor + sqrt(1-corr^2) * Z,
    values fresh N(0,1).  Returns dict(q, k, v) with the anchor's dtypes."""
    assert layer >= 1
    s = math.sqrt(1.0 - corr * corr)
    out = {}
    for name, sid in (("q", 40), ("k", 41)):
        t = base[name]
        z = _randn(t.shape, t.device, seed, sid + 3 * layer)
        out[name] = (corr * t.float() + s * z).to(t.dtype)
        del z
    v = base["v"]
    out["v"] = _randn(v.shape, v.device, seed, 42 + 3 * layer).to(v.dtype)
    return out


def page_table_for(B, max_pages, device, seed, sid=20):
    """[B, max_pages] int32: a seeded permutation of B * max_pages pool pages."""
    return _randperm(B * max_pages, device, seed, sid).to(torch.int32).reshape(B, max_pages)


def decode_pool(num_pages, Hkv, D, device, seed, sid, dtype=torch.bfloat16, base=None, corr=0.9,
                chunk_pages=16384):
    """[num_pages, Hkv, 16, D] pool; if base is given, corr * base + sqrt(1-corr^2) * Z."""
    out = torch.empty((num_pages, Hkv, PAGE, D), device=device, dtype=dtype)
    g = _gen(device, seed, sid)
    s = math.sqrt(1.0 - corr * corr)
    for p0 in range(0, num_pages, chunk_pages):
        p1 = min(num_pages, p0 + chunk_pages)
        z = torch.randn((p1 - p0, Hkv, PAGE, D), generator=g, device=device, dtype=torch.float32)
        if base is not None:
            z = corr * base[p0:p1].float() + s * z
        out[p0:p1] = z.to(dtype)
        del z
    return out


def decode_inputs(B, N, Hq, Hkv, D, layers=1, seq_lens=None, corr=0.9, seed=0, device="cpu",
                  dtype=torch.bfloat16):
    """Kascade-style decode group: per layer q [B,Hq,D], k_pool, v_pool.

    seq_lens: optional per-sequence lengths (<= N); default all N.
    Layer 0 keys are i.i.d.; layer l > 0 keys are corr * K_0 + sqrt(1-corr^2) Z.
    Returns dict(page_table, seq_lens, layers=[dict(q, k, v)], max_pages).
    """
    max_pages = -(-N // PAGE)
    pt = page_table_for(B, max_pages, device, seed)
    if seq_lens is None:
        seq_lens = [N] * B
    sl = torch.tensor(seq_lens, dtype=torch.int32, device=device)
    num_pages = B * max_pages
    out = []
    k0 = None
    for l in range(layers):
        q = _randn((B, Hq, D), device, seed, 30 + 3 * l).to(dtype)
        k = decode_pool(num_pages, Hkv, D, device, seed, 31 + 3 * l, dtype,
                        base=k0 if l > 0 else None, corr=corr)
        v = decode_pool(num_pages, Hkv, D, device, seed, 32 + 3 * l, dtype)
        if l == 0:
            k0 = k
        out.append({"q": q, "k": k, "v": v})
    return {"page_table": pt, "seq_lens": sl, "layers": out, "max_pages": max_pages,
            "num_pages": num_pages}


def to_f64(t):
    """Exact widening of a bf16/fp32 tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()

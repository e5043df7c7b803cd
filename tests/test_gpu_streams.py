"""Calls on two streams at once (the ABI is stream-ordered and re-entrant: a
call enqueues on the caller's stream and keeps no global state).  Prefill
attention and index decode run concurrently on two default-priority streams,
each with its own inputs, outputs and workspaces; every result must equal the
same call run alone on the default stream, bit for bit."""

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def test_prefill_and_decode_on_two_streams_match_serial():
    import free_sparse_attention_head_amd as fsa
    print("[streams] prefill S=4096 T=128 + index decode B=4 N=8192, two streams", flush=True)
    pf = [workloads.prefill_inputs(1, 4096, 8, 2, 128, 128, model="lowrank", n_spikes=8, seed=s,
                                   device="cuda") for s in (3, 4)]
    sel = []
    for p in pf:
        c, r = fsa.block_stats(p["k"], 128)
        sel.append(fsa.select_blocks(p["q"], c, r, 128, 0.2, 0.08, 2, 1))
    dc = workloads.decode_inputs(4, 8192, 8, 2, 128, layers=2, seq_lens=[8192, 5000, 3000, 777],
                                 seed=5, device="cuda")
    idx, _ = fsa.topk_indices(dc["layers"][0]["q"], dc["layers"][0]["k"], dc["page_table"],
                              dc["seq_lens"], 256)
    L1 = dc["layers"][1]

    def prefill(x):
        p, s = pf[x], sel[x]
        return fsa.sparse_prefill_attn(p["q"], p["k"], p["v"], 128, s["block_idx"], s["block_cnt"])

    def decode(n_split):
        return fsa.sparse_decode_attn(L1["q"], L1["k"], L1["v"], dc["page_table"], dc["seq_lens"],
                                      mode=fsa.SEL_INDEX, idx=idx, n_split=n_split)

    ref = [prefill(0), prefill(1), decode(3)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(s1):
            a = prefill(0)
            c = decode(3)
        with torch.cuda.stream(s2):
            b = prefill(1)
            d = decode(3)
        torch.cuda.synchronize()
        for got, want in ((a, ref[0]), (b, ref[1]), (c, ref[2]), (d, ref[2])):
            for g_, w_ in zip(got, want):
                assert torch.equal(g_, w_)

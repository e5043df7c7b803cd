"""The decode group under HIP graph capture: top-k at the anchor layer, index
decode at its indices, and a segment decode with several splits (so the
combine kernel runs), all into preallocated outputs and workspaces.  The
library enqueues kernels only (its top-k histograms are cleared by a fill
kernel, not a memset), so the captured graph must replay to the eager
results, bit for bit, on every replay, with the program's own eager library
calls and synchronisations between replays and the outputs scribbled over
before each replay."""

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def test_decode_group_graph_replays_match_eager():
    import free_sparse_attention_head_amd as fsa
    print("[graphs] decode group B=4 N=8192 Hq=8 Hkv=2 D=128 k=256, captured", flush=True)
    B, N, Hq, Hkv, D, k = 4, 8192, 8, 2, 128, 256
    dc = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=2, seq_lens=[8192, 5000, 3000, 777],
                                 seed=11, device="cuda")
    L0, L1 = dc["layers"]
    pt, sl = dc["page_table"], dc["seq_lens"]
    segs = torch.tensor([[[0, 64], [4096, 6144], [8000, 8192]], [[0, 16], [1000, 3000], [0, 0]],
                         [[2000, 3000], [0, 0], [0, 0]], [[0, 777], [0, 0], [0, 0]]],
                        dtype=torch.int32, device="cuda")
    nseg = torch.tensor([3, 2, 1, 1], dtype=torch.int32, device="cuda")
    dev = "cuda"
    idx = torch.empty((B, Hq, k), dtype=torch.int32, device=dev)
    kth = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    o_idx = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    l_idx = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    o_seg = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    l_seg = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws_topk = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    ws_dec = torch.empty(4 << 20, dtype=torch.uint8, device=dev)

    def group():
        fsa.topk_indices(L0["q"], L0["k"], pt, sl, k, idx=idx, kth=kth, ws=ws_topk)
        fsa.sparse_decode_attn(L1["q"], L1["k"], L1["v"], pt, sl, mode=fsa.SEL_INDEX, idx=idx,
                               out=o_idx, lse=l_idx, ws=ws_dec)
        fsa.sparse_decode_attn(L1["q"], L1["k"], L1["v"], pt, sl, mode=fsa.SEL_SEGMENT,
                               segments=segs, n_seg=nseg, n_split=16, out=o_seg, lse=l_seg,
                               ws=ws_dec)

    outs = (idx, kth, o_idx, l_idx, o_seg, l_seg)
    group()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        group()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        group()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got, want), rep
        # the program's own eager work between replays (other buffers)
        fsa.sparse_decode_attn(L0["q"], L0["k"], L0["v"], pt, sl, mode=fsa.SEL_ALL)
        fsa.topk_indices(L1["q"], L1["k"], pt, sl, k)
        torch.cuda.synchronize()

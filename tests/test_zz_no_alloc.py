"""The allocation-free decode entry point (sparse_decode_attn_noalloc) against
sparse_decode_attn, through the C ABI.

Both run the same kernels with the same split count, so the results must be
bit-identical; the allocation-free call keeps its split partials in the
library's own per-GPU array.  Two calls in a row, the second on a smaller
input, check that nothing left in the shared array leaks into a later call.
Sizes beyond the array are rejected before any launch.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _segments(fsa, B, N, seed):
    rng = np.random.default_rng(seed)
    segs = torch.zeros((B, 2, 2), dtype=torch.int32)
    nseg = torch.zeros(B, dtype=torch.int32)
    for b in range(B):
        mode = (fsa.SEG_GLOBAL, fsa.SEG_FOCUS, fsa.SEG_LOCAL, fsa.SEG_STREAMING)[b % 4]
        rs = fsa.build_segments(mode, N, chunk_start=int(rng.integers(0, N - 2048)))
        nseg[b] = len(rs)
        for x, (a, e) in enumerate(rs):
            segs[b, x, 0], segs[b, x, 1] = a, e
    return segs.cuda(), nseg.cuda()


@pytest.mark.parametrize("mode", ["segment", "index", "all"])
def test_noalloc_matches_workspace_entry_point(mode):
    import free_sparse_attention_head_amd as fsa
    print(f"[no-alloc {mode}] two calls, the second smaller", flush=True)
    for call, (B, N, Hq, Hkv, D, k, n_split) in enumerate([(4, 16384, 16, 4, 128, 512, 0),
                                                          (2, 6000, 8, 2, 64, 300, 3)]):
        d = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=1, seed=60 + call, device="cuda")
        L = d["layers"][0]
        pt, sl = d["page_table"], d["seq_lens"]
        kw = dict(n_split=n_split, max_seq_len=N)
        if mode == "segment":
            segs, nseg = _segments(fsa, B, N, 60 + call)
            kw.update(mode=fsa.SEL_SEGMENT, segments=segs, n_seg=nseg)
        elif mode == "index":
            idx, _ = fsa.topk_indices(L["q"], L["k"], pt, sl, k, max_seq_len=N)
            kw.update(mode=fsa.SEL_INDEX, idx=idx)
        else:
            kw.update(mode=fsa.SEL_ALL)
        o_ref, l_ref = fsa.sparse_decode_attn(L["q"], L["k"], L["v"], pt, sl, **kw)
        out = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(l_ref, float("nan"))
        o, l = fsa.sparse_decode_attn_noalloc(L["q"], L["k"], L["v"], pt, sl, out=out, lse=lse, **kw)
        torch.cuda.synchronize()
        assert o.data_ptr() == out.data_ptr() and l.data_ptr() == lse.data_ptr()
        assert torch.equal(o, o_ref), (mode, call)
        assert torch.equal(l, l_ref), (mode, call)
        # and against the oracle on one head, so that a shared wrong result fails too
        if mode == "all":
            h = Hq - 1
            g = oracle.kv_head(h, Hq, Hkv)
            n = int(sl[0])
            K = oracle.gather_pages(workloads.to_f64(L["k"].cpu()), pt[0].cpu().numpy(), n, g)
            V = oracle.gather_pages(workloads.to_f64(L["v"].cpu()), pt[0].cpu().numpy(), n, g)
            ref, ref_l = oracle.index_attention(workloads.to_f64(L["q"][0, h]), K, V, np.arange(n),
                                                1 / np.sqrt(D))
            assert np.abs(o[0, h].double().cpu().numpy() - ref).max() <= 2e-2
            assert abs(l[0, h].item() - ref_l) <= 1e-2


def test_noalloc_rejects_partials_beyond_its_array():
    """B * Hq * n_split * (D + 2) * 4 bytes of partials above 16 MiB: rejected
    with FSA_ERR_WORKSPACE before any launch; the outputs stay untouched."""
    import free_sparse_attention_head_amd as fsa
    B, N, Hq, Hkv, D = 2, 4096, 32, 8, 128
    d = workloads.decode_inputs(B, N, Hq, Hkv, D, layers=1, seed=65, device="cuda")
    L = d["layers"][0]
    n_split = 1024   # 2 * 32 * 1024 * 130 * 4 bytes = 34 MB
    out = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fsa.FsaError) as e:
        fsa.sparse_decode_attn_noalloc(L["q"], L["k"], L["v"], d["page_table"], d["seq_lens"],
                                       mode=fsa.SEL_ALL, n_split=n_split, out=out)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert (out == 0).all()

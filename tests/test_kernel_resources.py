"""Register budgets that kernels' occupancy depends on (CPU only: compiles
the device code to assembly and reads the kernel descriptors).

The top-k select kernel runs one 1024-thread workgroup per score row, and its
time is set by how many rows run per CU: two workgroups share a CU only while
a wave holds at most 64 VGPRs and about 72 SGPRs (an occupancy probe placed
one per CU at 78 SGPRs or 71 VGPRs).  The compiler does not enforce the VGPR
cap the kernel asks for, so this test does."""
import os
import re
import shutil
import subprocess

import pytest

from free_sparse_attention_head_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def _assembly(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [B._hipcc()] + [x for x in B.COMMON if x != "-fPIC"] + ["--cuda-device-only", "-S", "-o", str(out), src]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _descriptors(src, tmp_path, text=None):
    text = text if text is not None else _assembly(src, tmp_path)
    kd = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S):
        body = m.group(2)
        get = lambda key: int(re.search(r"\.amdhsa_" + key + r" (\d+)", body).group(1))
        kd[m.group(1)] = {"vgpr": get("next_free_vgpr"), "sgpr": get("next_free_sgpr"),
                          "lds": get("group_segment_fixed_size"),
                          "scratch": get("private_segment_fixed_size")}
    return kd


def _scratch_in_loops(text, kernel):
    """Scratch instructions of `kernel` that sit in a basic block the compiler
    annotates as part of a loop (its label line says "Loop")."""
    body = text[re.search(r"^" + re.escape(kernel) + r":", text, re.M).start():]
    body = body[:body.index("s_endpgm")]
    label, bad = "", []
    for line in body.splitlines():
        if re.match(r"^\.LBB\d+_\d+:", line) or line.startswith("; %bb."):
            label = line
        elif "scratch_" in line and "Loop" in label:
            bad.append((label.split()[0], line.strip()))
    return bad


def test_topk_select_kernel_fits_two_workgroups_per_cu(tmp_path):
    kd = _descriptors(os.path.join(B.CSRC, "topk.hip"), tmp_path)
    sel = [v for k, v in kd.items() if "topk_select_kernel" in k]
    assert len(sel) == 1, list(kd)
    d = sel[0]
    assert d["vgpr"] <= 64, d
    assert d["sgpr"] <= 72, d
    assert d["scratch"] == 0, d
    assert 2 * d["lds"] <= 160 * 1024, d


def test_prefill_attention_kernels_do_not_spill(tmp_path):
    """The bf16 attention kernel runs two waves per SIMD at up to 256 VGPRs a
    lane; its allocation is tight enough that unrelated code shapes have
    pushed a value to scratch.  Every instantiation stays within 256 VGPRs
    and no scratch access sits inside a loop.  The 128-row, D = 128
    instantiation keeps one value (4 bytes) in scratch across its chunk loop:
    stored once before the loop, read back after it; every other
    instantiation is spill-free."""
    src = os.path.join(B.CSRC, "prefill_attn_bf16.hip")
    text = _assembly(src, tmp_path)
    kd = _descriptors(src, tmp_path, text)
    pf = {k: v for k, v in kd.items() if "prefill_attn_bf16_kernel" in k}
    assert len(pf) >= 6, list(kd)
    for name, d in pf.items():
        assert d["scratch"] <= (8 if "ILi128ELi128E" in name else 0), (name, d)
        assert d["vgpr"] <= 256, (name, d)
        assert _scratch_in_loops(text, name) == [], name


@pytest.mark.parametrize("src", ["topk.hip", "decode_attn.hip", "select_blocks.hip",
                                 "block_stats.hip", "prefill_attn.hip"])
def test_no_kernel_spills_to_scratch(src, tmp_path):
    """Every kernel of the library keeps its registers out of scratch memory."""
    kd = _descriptors(os.path.join(B.CSRC, src), tmp_path)
    assert kd, src
    spills = {k: v["scratch"] for k, v in kd.items() if v["scratch"]}
    assert not spills, spills


def test_loop_scratch_check_sees_loop_blocks():
    """The loop check flags a scratch access in a block the compiler marks as
    part of a loop, and ignores one before the loop."""
    text = ("k:                                      ; @k\n"
            "\tscratch_store_dword off, v1, off\n"
            ".LBB0_2:                                ; =>This Inner Loop Header: Depth=1\n"
            "\tv_add_u32_e32 v2, v2, v3\n"
            ".LBB0_3:                                ;   in Loop: Header=BB0_2 Depth=1\n"
            "\tscratch_load_dword v4, off, off\n"
            ".LBB0_4:\n"
            "\tscratch_load_dword v1, off, off\n"
            "\ts_endpgm\n")
    assert _scratch_in_loops(text, "k") == [(".LBB0_3:", "scratch_load_dword v4, off, off")]

"""The host side of the C ABI under AddressSanitizer and UndefinedBehavior-
Sanitizer (CPU only; no kernel is launched).

Every source of the library is compiled with the sanitizers on its host code
alone (each -fsanitize is passed through -Xarch_host; device code is built as
usual), linked with tests/asan/abi_driver.cpp, and run: validation of every
entry point, workspace sizing over a sweep of shapes and the segment builders
over random and extreme arguments must hold their documented results with no
sanitizer report.  Skipped when hipcc is not installed.
"""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "free_sparse_attention_head_amd", "csrc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _hipcc():
    return shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc")
                                     else None)


@pytest.mark.timeout(600)
def test_c_abi_host_code_under_sanitizers():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not installed")
    from free_sparse_attention_head_amd import build as B
    tmp = tempfile.mkdtemp(prefix="fsa_asan_")
    try:
        srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "fsa_api.cpp"),
                                                                  os.path.join(ROOT, "tests", "asan",
                                                                               "abi_driver.cpp")]

        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            r = subprocess.run([hipcc] + lang + B.COMMON + ["-O1"] + SAN + ["-c", src, "-o", obj],
                               capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-3000:]
            return obj

        with cf.ThreadPoolExecutor(max_workers=8) as ex:
            objs = list(ex.map(compile_one, srcs))
        exe = os.path.join(tmp, "abi_driver")
        r = subprocess.run([hipcc, f"--offload-arch={B.ARCH}"] + SAN + objs + ["-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        report = run.stdout[-2000:] + run.stderr[-4000:]
        assert "AddressSanitizer" not in run.stderr, report
        assert "runtime error" not in run.stderr, report
        assert run.returncode == 0, report
        assert "0 failed checks" in run.stdout, report
    finally:
        shutil.rmtree(tmp, ignore_errors=True)

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C-ABI layer (argument checks, host-side rotary frequencies) is rebuilt with both sanitizers
on its host code (gqa_scaled_rope_amd/build.py: build_sanitized) and tests/test_abi_cpu.py runs
against that library in a child process with the sanitizer runtime preloaded.  A memory error or
undefined behaviour in the host code aborts the child, which fails this test.  No kernel is
launched."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
build = pytest.importorskip("gqa_scaled_rope_amd.build")

RUNNER = """
import sys, pytest
sys.path.insert(0, {root!r})
import gqa_scaled_rope_amd as g
g.LIB_PATH = {lib!r}
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {tests!r}]))
"""


def test_abi_checks_clean_under_host_sanitizers(tmp_path):
    if not os.path.exists(build.HIPCC) or shutil.which("nm") is None:
        pytest.skip("hipcc or nm not available")
    if not os.path.exists(os.path.join(build.OBJ, "attn_decode_mfma.o")):
        pytest.skip("normal build objects missing (run __graft_entry__.build())")
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("AddressSanitizer runtime not found")
    lib = build.build_sanitized(str(tmp_path / "san"))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms, "host code not instrumented"
    runner = tmp_path / "run_abi.py"
    runner.write_text(RUNNER.format(root=ROOT, lib=lib,
                                    tests=os.path.join(ROOT, "tests", "test_abi_cpu.py")))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, str(runner)], capture_output=True, text=True, env=env,
                       cwd=str(tmp_path), timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in out and "AddressSanitizer" not in out and "runtime error" not in out

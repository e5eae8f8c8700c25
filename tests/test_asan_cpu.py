"""The host code of the library (argument checks, planner, window schedule,
launch set-up) under AddressSanitizer: the library is rebuilt with the
sanitizer on its host code only and the CPU ABI and window tests run against
it in a child process that preloads the sanitizer runtime."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_code_under_asan():
    sys.path.insert(0, ROOT)
    from block_causal_attention_d2f_amd import build as B
    lib = B.build(asan=True)
    rt = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        stdout=subprocess.PIPE, text=True).stdout.strip()
    if not os.path.isfile(rt):
        pytest.skip("sanitizer runtime not found")
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               D2F_LIB=lib)
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        os.path.join(ROOT, "tests", "test_window_cpu.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    assert p.returncode == 0, p.stdout[-4000:]
    assert "AddressSanitizer" not in p.stdout, p.stdout[-4000:]
    assert " passed" in p.stdout

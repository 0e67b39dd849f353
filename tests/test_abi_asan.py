"""The ABI tests again, against the library built with AddressSanitizer on
its host code (argument validation, size helpers, error strings): any
out-of-bounds access or use-after-free in the host-side checks aborts the
run with an ASan report.  CPU only; no call reaches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_host_asan():
    from trainable_block_sparse_amd.build import asan_runtime, build_asan
    lib = build_asan()
    rt = asan_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ, INFV2_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]

"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
library's argument validation, planners and host launch code, and the input
generator, built with both sanitizers (device code unchanged) and exercised
by the C-ABI and generator tests in a child process that preloads the
sanitizer runtime.  Any report fails the child (UBSan does not recover)."""
import os
import subprocess
import sys

import sa_synth as S
from top_sparse_decode_sa_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_is_clean_under_asan_and_ubsan():
    lib = B.build_sanitized()
    synth = S.build_lib_sanitized(B.clang())
    env = dict(os.environ, LD_PRELOAD=B.sanitizer_runtime(), SA_LIBRARY=lib,
               SA_SYNTH_LIBRARY=synth, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = ("import ctypes, sa_synth as S, top_sparse_decode_sa_amd as T\n"
             "assert hasattr(ctypes.CDLL(None), '__asan_report_load4')\n"
             "print(T.lib()._name); print(S.lib()._name)\n")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.split() == [lib, synth]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-m", "not gpu",
                        "-p", "no:cacheprovider", "tests/test_boundary.py", "tests/test_synth.py",
                        "-k", "not oracle_baseline"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]

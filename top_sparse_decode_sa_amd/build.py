"""Build ``libsa.so`` (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: ``python -m top_sparse_decode_sa_amd.build`` (or call ``build()``).
Objects go to ``top_sparse_decode_sa_amd/_build/``; the shared library is
written next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsa.so")
SOURCES = ["api.hip", "attend.hip", "check.hip", "offload.hip", "score.hip", "select.hip",
           "stream.hip", "topk.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def common_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            # only the C ABI of include/sa.h is exported
            "-fvisibility=hidden",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
            # no packed fp32 instructions in any kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer variant (argument
# validation, planners, host launch code); the device code is built as usual.
SAN_DIR = os.path.join(OBJ_DIR, "sanitized")
SAN_LIB = os.path.join(SAN_DIR, "libsa.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def _compile(src: str, out_dir: str = OBJ_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, res.stderr[-4000:]))
    return obj


def _build_into(lib_path: str, out_dir: str, extra=(), link_extra=()) -> str:
    os.makedirs(out_dir, exist_ok=True)
    jobs = min(len(SOURCES), max(1, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir, extra), SOURCES))
    tmp = lib_path + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + list(link_extra) + \
        ["-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s" % res.stderr[-4000:])
    os.replace(tmp, lib_path)
    return lib_path


def build(verbose: bool = False) -> str:
    """Compile every source and link libsa.so.  Always rebuilds."""
    _build_into(LIB, OBJ_DIR)
    if verbose:
        print("built", LIB)
    return LIB


def clang() -> str:
    """The clang that hipcc drives."""
    path = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(path):
        raise RuntimeError("clang not found beside hipcc")
    return os.path.realpath(path)


def sanitizer_runtime() -> str:
    """The compiler's shared ASan (+UBSan) runtime, which a host process must
    preload to load the sanitized library."""
    res = subprocess.run([clang(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the compiler's ASan runtime was not found")
    return path


def build_sanitized(verbose: bool = False) -> str:
    """libsa.so with the host code under ASan + UBSan, in _build/sanitized/
    (load it with the runtime of sanitizer_runtime() preloaded)."""
    _build_into(SAN_LIB, SAN_DIR, SAN_FLAGS, SAN_FLAGS[:4] + ["-shared-libsan"])
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitized" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)

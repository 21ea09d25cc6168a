"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

moe_api.cpp and noalloc.hip hold all the host code of libmoe.so: argument
validation, the workspace layout and carving, the plan sizing, the error
texts.  They are rebuilt with the sanitizers on their host pass only (the
GPU code is built as usual and never runs here), linked with the kernels'
objects into a separate library, and the host ABI tests run against it in a
child process with the sanitizer runtime preloaded; any report fails them.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

from expert_ffn_layer_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJDIR = os.path.join(build.OBJDIR, "sanitized")
LIB = os.path.join(OBJDIR, "libmoe_sanitized.so")
HOST_SOURCES = ("moe_api.cpp", "noalloc.hip")
# sanitizers on the host compilation only (-Xarch_host before each)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _build_sanitized():
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [build._compile(src, OBJDIR, extra=("-g", *SAN)) for src in HOST_SOURCES]
    objs += [build._compile(src, OBJDIR) for src in build.SOURCES if src not in HOST_SOURCES]
    cmd = [build.HIPCC, f"--offload-arch={build.ARCH}", "-shared", "-fPIC",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-shared-libsan", *objs, "-o", LIB]
    subprocess.run(cmd, check=True, capture_output=True, text=True)


@pytest.mark.timeout(900)
def test_abi_host_under_sanitizers():
    rt = _runtime()
    if rt is None or not os.path.exists(build.HIPCC):
        pytest.skip("no hipcc / clang sanitizer runtime in this image")
    _build_sanitized()
    syms = subprocess.run(["nm", "-D", "--undefined-only", LIB], capture_output=True,
                          text=True).stdout
    assert "__asan_init" in syms and "__ubsan_handle" in syms, "sanitizers not compiled in"
    env = dict(os.environ, LD_PRELOAD=rt, MOE_LIB_PATH=LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cp = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                         os.path.join(ROOT, "tests", "test_abi_host.py")],
                        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = cp.stdout + cp.stderr
    assert cp.returncode == 0, out[-3000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-3000:]
    assert " passed" in out

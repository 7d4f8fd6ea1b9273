"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

abi.cpp (argument validation, workspace layouts, dispatch) is rebuilt as plain host C++ with
-fsanitize=address,undefined and linked with the library's kernel objects, which are unchanged; then
tests/test_abi.py runs against that library in a fresh interpreter with the sanitizer runtime
preloaded.  Every call in test_abi.py is rejected on the host before any HIP call, so no GPU is
involved.  Any sanitizer report aborts the run and fails this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
OUT = os.path.join(ROOT, "_build", "host_sanitized")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def _sanitized_library() -> str:
    from sparse_moe_expert_sigmoid_amd import build as B
    objs = [os.path.join(B.BUILD_DIR, os.path.splitext(src)[0] + ".o") for src in B.SOURCES if src != "abi.cpp"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    os.makedirs(OUT, exist_ok=True)
    abi_o = os.path.join(OUT, "abi.o")
    lib = os.path.join(OUT, "libmoe_q4_host_sanitized.so")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    _run([CLANG, "-x", "c++", "-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
          "-I/opt/rocm/include", "-I", B.INCLUDE, *san, "-c", os.path.join(B.CSRC, "abi.cpp"), "-o", abi_o])
    _run([CLANG, "-shared", "-fPIC", "-shared-libasan", *san, *objs, abi_o, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", lib])
    return lib


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not present")
def test_abi_validation_under_address_and_undefined_behaviour_sanitizers():
    lib = _sanitized_library()
    rt = _run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    assert os.path.exists(rt), rt
    env = dict(os.environ, MOE_Q4_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the child checks it really loaded the sanitized build, then runs the ABI tests
    probe = ("import sys; sys.path.insert(0, %r); from sparse_moe_expert_sigmoid_amd import abi; abi.lib(); "
             "maps = open('/proc/self/maps').read(); "
             "assert %r in maps and 'libclang_rt.asan' in maps, 'sanitized library not loaded'" % (ROOT, lib))
    _run([sys.executable, "-c", probe], env=env, cwd=ROOT)
    r = _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"], env=env, cwd=ROOT)
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]

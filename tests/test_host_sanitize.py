"""libkvz's host code (argument validation, workspace sizing, keep count,
status strings, the timer's host paths) under AddressSanitizer and
UndefinedBehaviorSanitizer.  The library's sources are compiled with both
sanitizers on their host side (device code as usual), linked to
tests/abi_sanitize.cpp, and run; no GPU is needed because no call in that
test program gets past validation."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_score_reduction_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="ROCm compilers not installed")
def test_abi_host_paths_under_asan_and_ubsan(tmp_path):
    from attention_score_reduction_amd import build
    objs = []
    procs = []
    for src in build.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        objs.append(obj)
        # device code as in the release build, host code instrumented: each
        # sanitizer flag applies to the host side only
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
               "-fsanitize=undefined", "-fvisibility=hidden", "-I", os.path.join(ROOT, "include"),
               "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                      text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out
    lib = str(tmp_path / "libkvz_san.so")
    hip_lib = "/opt/rocm/lib"
    r = subprocess.run([CLANG, "-shared", "-fsanitize=address,undefined", *objs, "-L" + hip_lib,
                        "-lamdhip64", "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    exe = str(tmp_path / "abi_sanitize")
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "abi_sanitize.cpp"), lib,
                        "-Wl,-rpath," + str(tmp_path) + ":" + hip_lib, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0 and "ok: 0 failure(s)" in r.stdout, r.stdout + r.stderr

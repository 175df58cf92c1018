"""Build libkvz.so for gfx950 with hipcc, in-tree (next to this file).

The library carries a build id: the sha256 of its sources, the public header
and the compiler flags (source_digest()).  The Python binding refuses to load
a libkvz.so whose id differs from the digest of the files next to it, so a
stale binary can never stand in for the checked-out source.

build(debug=True) makes libkvz_debug.so from the same sources with
-DKVZ_DEBUG: its kernels check their inputs' conditions and their own
invariants and the calls report a failed check as KVZ_ERR_INVALID_ARG (the
release library compiles those checks away).
"""
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "score.hip", "attn.hip", "select.hip", "compact.hip", "heads.hip",
           "decode.hip", "noalloc.hip"]
LIB = os.path.join(HERE, "libkvz.so")
DEBUG_LIB = os.path.join(HERE, "libkvz_debug.so")
DEBUG_FLAGS = ["-DKVZ_DEBUG"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 instructions in any device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    # MFMA accumulators in VGPRs (no AGPR copies before the softmax VALU work)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


INCLUDE = os.path.normpath(os.path.join(HERE, "..", "include"))


def source_digest(debug: bool = False) -> str:
    """sha256 over every source file of the library (csrc/*.hip, csrc/*.h,
    include/*.h, by relative path and content) and the compiler flags (those
    of the debug build when debug is set)."""
    h = hashlib.sha256()
    files = []
    for d, rel in ((CSRC, "csrc"), (INCLUDE, "include")):
        for f in sorted(os.listdir(d)):
            if f.endswith((".hip", ".h")):
                files.append((f"{rel}/{f}", os.path.join(d, f)))
    for rel, path in files:
        h.update(rel.encode() + b"\0")
        with open(path, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    h.update(" ".join(FLAGS + (DEBUG_FLAGS if debug else []) + SOURCES).encode())
    return h.hexdigest()


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libkvz.so
    (libkvz_debug.so with debug set)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "..", "_build", "debug" if debug else "release")
    os.makedirs(objdir, exist_ok=True)
    bid = source_digest(debug)
    compile_flags = [f for f in FLAGS if f != "-shared"] + (DEBUG_FLAGS if debug else [])
    lib_path = DEBUG_LIB if debug else LIB
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = ([hipcc] + compile_flags + [f'-DKVZ_BUILD_ID="{bid}"', "-I", INCLUDE, "-c",
                                          os.path.join(CSRC, src), "-o", obj])
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out)
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed compiling {failed}")
    tmp = lib_path + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed linking {os.path.basename(lib_path)}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
    print(build(verbose=True, debug=True))

"""Build libpkv.so (the gfx950 HIP library behind include/pkv.h) in place.

One hipcc invocation compiles every source under csrc/ for gfx950 and links
the shared library next to this file, where the Python binding loads it.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed FP32 instructions stay off (hand-written or compiler-made)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


# A host-sanitized build (python build.py --sanitize -> libpkv_san.so):
# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
# (argument validation, workspace carving, launch planning); the gfx950 code
# is built as usual.  Load it with PKV_LIBRARY=<path to libpkv_san.so> and
# clang's ASan runtime preloaded (libclang_rt.asan-x86_64.so of the ROCm
# LLVM, ASAN_OPTIONS=detect_leaks=0).
SAN_LIB = os.path.join(HERE, "libpkv_san.so")
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *(SANITIZE if sanitize else []), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msgs)
    if msgs.strip() and verbose:
        print(msgs, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import sys as _sys
    print(build(verbose=True, sanitize="--sanitize" in _sys.argv))

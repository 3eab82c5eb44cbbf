"""Build the CPU oracle library (test infrastructure; see oracle/oracle.c).

Plain gcc, -O2, no FMA contraction, no OpenMP, no vector intrinsics: the
oracle is meant to be slow, single-threaded and obviously correct.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(HERE, "liboracle_san.so")


# With PKV_ORACLE_SANITIZE=1 the oracle is built (liboracle_san.so) and
# loaded with AddressSanitizer and UndefinedBehaviorSanitizer (gcc's
# runtimes; python then needs them preloaded: LD_PRELOAD="$(gcc
# -print-file-name=libasan.so) $(gcc -print-file-name=libubsan.so)"
# ASAN_OPTIONS=detect_leaks=0).  Any report aborts the process.
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def sanitized() -> bool:
    return os.environ.get("PKV_ORACLE_SANITIZE", "") == "1"


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (liboracle_san.so when sanitized)
    next to it and return its path."""
    san = sanitized()
    lib = SAN_LIB if san else LIB
    if not force and os.path.exists(lib) and os.path.getmtime(lib) >= os.path.getmtime(SRC):
        return lib
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", *(SANITIZE if san else []), "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build())

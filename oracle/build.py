"""Build the CPU oracle (test infrastructure) as oracle/liboracle.so.

The oracle is plain C built with gcc at -O2 with no fast-math and no FMA
contraction, so that every binary32 operation in it rounds exactly once.

build(sanitize=True, out=path) makes a second copy instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only, every finding
fatal), which tests/test_oracle_sanitized.py loads in a child process with the
ASan runtime preloaded.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qcp_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
          "-Wall", "-Wextra", "-shared", "-fPIC"]
SANITIZE = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=all"]


def build(verbose: bool = False, sanitize: bool = False, out: str = None, src: str = SRC) -> str:
    out = out or LIB
    cmd = ["gcc", *CFLAGS, *(SANITIZE if sanitize else []), "-o", out, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


def asan_runtime() -> str:
    """Path of gcc's ASan runtime, to preload into a process that loads a
    sanitized build."""
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                          capture_output=True, text=True).stdout.strip()


if __name__ == "__main__":
    build(verbose=True)

"""Build the hardware self-test library (test infrastructure) in-tree:

    python -m tests.hw.build

Compiles qcp_hw_selftest.hip with exactly the library's compiler flags, so the
device helpers it checks are compiled as the library compiles them, into
tests/hw/libqcp_hwtest.so.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from quantized_collective_payloads_amd import build as lib_build  # noqa: E402

LIB = os.path.join(HERE, "libqcp_hwtest.so")
SRC = os.path.join(HERE, "qcp_hw_selftest.hip")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [lib_build.HIPCC, *lib_build.CXXFLAGS, "-shared", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on qcp_hw_selftest.hip")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)

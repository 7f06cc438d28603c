"""Compile tests/c_abi/decode_from_c: a host program that drives the decode
through the C ABI alone (include/pda.h, libpda.so) and checks it against the
CPU oracle (oracle/liboracle.so).  Test infrastructure: it is built with the
library (by __graft_entry__.build(), which builds the oracle first) and run by
tests/test_c_abi_driver.py.  The program finds both libraries relative to its
own location, so the tree can move.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "decode_from_c.cpp")
EXE = os.path.join(HERE, "decode_from_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_abi_driver(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "paged_kv_cache_decode_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = ["g++", "-std=c++17", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-o", EXE + ".tmp",
           "-L", pkg, "-lpda", "-L", orc, "-loracle", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../paged_kv_cache_decode_amd:$ORIGIN/../../oracle:"
           + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build_c_abi_driver(verbose=True))

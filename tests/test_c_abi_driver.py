"""The decode driven from C through include/pda.h alone (tests/c_abi/
decode_from_c.cpp): no Python binding and no torch between the caller and
the library.  On the CPU, the program's host-side validation run; on the GPU,
three shapes (block sizes 16, 784 and 5; head sizes 128, 256 and 64) under the
device plan and three forced plans, each checked against the fp32 oracle with
NaN in every unwritten tail slot."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "decode_from_c")


def test_c_driver_host_side_validation():
    if not os.path.exists(EXE):  # built with the library; a CPU-only checkout builds it here
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "c_abi_build", os.path.join(ROOT, "tests", "c_abi", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build_c_abi_driver()
    r = subprocess.run([EXE, "--host-only"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host-only validation: ok" in r.stdout


@pytest.mark.gpu
def test_decode_through_the_c_abi_alone():
    assert os.path.exists(EXE), "tests/c_abi/decode_from_c is built by __graft_entry__.build()"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]
    passed = [ln for ln in r.stdout.splitlines() if " plan " in ln and ln.endswith(" ok")]
    assert len(passed) == 12 and r.stdout.rstrip().endswith("all ok")

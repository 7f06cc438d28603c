"""The host runtime and the oracle's C code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

* tests/sanitize/host_harness.cpp links the library's host runtime
  (pda_host.cpp: validation, the plan, the workspace layout, the launch
  sequence) with stub launchers that replay every workspace, output, query
  and table index the kernels address, against buffers of exactly the sizes
  the header tells a caller to provide; then it fuzzes every pure entry
  point with arbitrary shapes and plans.
* tests/sanitize/oracle_harness.c drives oracle/oracle.c over random small
  shapes (empty contexts, single tokens, empty and clipped partial ranges)
  with exact-size buffers, and checks the properties the definition fixes.

Each harness also builds with a planted mistake (a buffer a few bytes short),
and the sanitizer must report it: a clean run is worth nothing if the
instrument cannot see a fault (page "vLLM's custom ROCm paged-attention
kernel wins all sixty cells", section 3).  Built with g++/gcc for the host
only; nothing here touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "paged_kv_cache_decode_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs the host compilers")


def _build_host(out, plant=False):
    cmd = (["g++", "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                                          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
           + (["-DPDA_HARNESS_PLANT_SHORT_WORKSPACE"] if plant else [])
           + [os.path.join(CSRC, "pda_host.cpp"), os.path.join(HERE, "host_harness.cpp"),
              "-o", out])
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def _build_oracle(out, plant=False):
    cmd = (["gcc", "-std=c99"] + SAN + ["-ffp-contract=off", "-fopenmp"]
           + (["-DORACLE_HARNESS_PLANT_SHORT_OUT"] if plant else [])
           + [os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_harness.c"),
              "-o", out, "-lm"])
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


@pytest.fixture(scope="module")
def bins(tmp_path_factory):
    d = tmp_path_factory.mktemp("sanitize")
    from concurrent.futures import ThreadPoolExecutor
    jobs = {"host": (_build_host, False), "host_plant": (_build_host, True),
            "oracle": (_build_oracle, False), "oracle_plant": (_build_oracle, True)}
    with ThreadPoolExecutor(4) as ex:
        futs = {k: ex.submit(f, str(d / k), plant) for k, (f, plant) in jobs.items()}
        return {k: f.result() for k, f in futs.items()}


def _run(exe, *args):
    return subprocess.run([exe, *map(str, args)], capture_output=True, text=True, env=ENV,
                          timeout=300)


def test_host_runtime_clean_under_asan_ubsan(bins):
    r = _run(bins["host"], 1500)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
    assert "failures 0" in r.stdout
    launches = int(r.stdout.split("launches ")[1].split()[0])
    assert launches > 1000  # the replay ran


def test_host_harness_sees_a_short_workspace(bins):
    r = _run(bins["host_plant"], 50)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr


def test_oracle_clean_under_asan_ubsan(bins):
    r = _run(bins["oracle"], 400)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
    assert "failures 0" in r.stdout


def test_oracle_harness_sees_a_short_output(bins):
    r = _run(bins["oracle_plant"], 50)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr

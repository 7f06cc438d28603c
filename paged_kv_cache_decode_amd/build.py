"""Build libpda.so in-tree with hipcc for gfx950 only.

Every translation unit is compiled in parallel into _build/, then linked into
paged_kv_cache_decode_amd/libpda.so.  The decode kernels' sources are compiled
once per (element type, head size), the matrix-core one also per KV type
(16-bit or fp8).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpda.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
# -packed-fp32-ops: never emit packed fp32 VALU ops (v_pk_fma_f32 and kin).
# -amdgpu-mfma-vgpr-form: matrix-core accumulators in VGPRs.  With them in
# AGPRs the compiler copied every accumulator out and back on each tile around
# the softmax rescale (v_accvgpr_read/write, 64-128 VALU moves per tile); the
# VGPR form has none and measured faster on every matrix-core shape.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _units(csrc=CSRC):
    units = []
    for dt in (0, 1):
        for hd in (64, 128, 256):
            units.append((os.path.join(csrc, "pda_decode_valu.hip"),
                          f"valu_{dt}_{hd}.o", [f"-DPDA_DTYPE={dt}", f"-DPDA_HEAD={hd}"]))
            units.append((os.path.join(csrc, "pda_decode_mfma.hip"),
                          f"mfma_{dt}_{hd}.o", [f"-DPDA_DTYPE={dt}", f"-DPDA_HEAD={hd}"]))
            units.append((os.path.join(csrc, "pda_decode_mfma.hip"), f"mfma8_{dt}_{hd}.o",
                          [f"-DPDA_DTYPE={dt}", f"-DPDA_HEAD={hd}", "-DPDA_KV_FP8=1"]))
    units.append((os.path.join(csrc, "pda_merge.hip"), "merge.o", []))
    units.append((os.path.join(csrc, "pda_trace.hip"), "trace.o", []))
    units.append((os.path.join(csrc, "pda_probe.hip"), "probe.o", []))
    units.append((os.path.join(csrc, "pda_fill.hip"), "fill.o", []))
    units.append((os.path.join(csrc, "pda_noalloc.hip"), "noalloc.o", []))
    flags = " ".join(CFLAGS[:1] + [f"--offload-arch={ARCH}", "-packed-fp32-ops",
                                   "-amdgpu-mfma-vgpr-form"])
    units.append((os.path.join(csrc, "pda_host.cpp"), "host.o",
                   ["-x", "hip", f'-DPDA_BUILD_FLAGS="{flags}"']))
    return units


def _compile(unit, verbose, build_dir):
    src, obj, extra = unit
    out = os.path.join(build_dir, obj)
    cmd = [HIPCC] + CFLAGS + extra + ["-c", src, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src} {extra}:\n{r.stderr}")
    # the host pass does not know the device-only feature: harmless, filter it
    warn = "\n".join(x for x in r.stderr.splitlines() if "packed-fp32-ops" not in x)
    if warn.strip() and verbose:
        print(warn, file=sys.stderr)
    return out


def build_library(verbose: bool = False, jobs: int = 8, out: str = LIB,
                  defines=(), build_dir: str = BUILD, csrc: str = CSRC) -> str:
    """Compile and link; `defines` are extra -D flags (tuning variants),
    `csrc` another copy of the sources."""
    os.makedirs(build_dir, exist_ok=True)
    units = [(src, obj, extra + [f"-D{d}" for d in defines])
             for src, obj, extra in _units(csrc)]
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, 16))) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose, build_dir), units))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))

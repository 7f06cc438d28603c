"""The benchmark's command-line contract, checked without a GPU: it measures
one GPU only and refuses any other count before touching a device, and its
HBM-traffic figure comes only from a counter summary taken from the current
sources of the kernel it describes."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_a_multi_rank_launch_is_refused():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_traffic_summary_is_keyed_to_kernel_and_sources():
    sys.path.insert(0, ROOT)
    import bench
    with open(os.path.join(ROOT, "profiles", "traffic_headline.json")) as f:
        t = json.load(f)
    # another variant's kernel never borrows the figure
    other = "valu" if t["variant"] == "mfma" else "mfma"
    assert bench.measured_traffic(other) is None
    # the figure is used exactly when the recorded hash is that of the sources
    same = t["kernel_source_sha256"] == bench.kernel_source_hash(t["variant"])
    got = bench.measured_traffic(t["variant"])
    assert (got == t["hbm_bytes_per_launch"]) if same else (got is None)

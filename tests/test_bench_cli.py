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


def test_design_table_is_the_stored_bench_line():
    """The results table of the design document is printed from the stored
    bench line (profiles/bench_full.json) by `bench.py --table`, not typed by
    hand: the rendered table appears in the document verbatim."""
    r = _run(["--table", os.path.join(ROOT, "profiles", "bench_full.json")])
    assert r.returncode == 0, r.stderr
    table = r.stdout.strip()
    assert table.startswith("| workload |")
    with open(os.path.join(ROOT, "DESIGN.md")) as f:
        design = f.read()
    assert table in design


def test_table_renders_rows_without_newer_keys():
    """A stored line from before a column existed still renders ('-')."""
    sys.path.insert(0, ROOT)
    import bench
    row = {"workload": "w", "variant": "mfma", "merge": "kernel", "P": 2, "T_p": 16,
           "us_per_call": 1.0, "pct_of_peak": 1.0, "splitkv_kernel_us": 1.0,
           "kernel_pct_of_peak": 1.0}
    out = bench.render_table({"headline": row, "parity": None, "extra": {}})
    assert out.splitlines()[2] == "| w | mfma | kernel | 2 x 16 | 1.00 | 1.0 % | 1.00 (1.0 %) | - | - | - |"

#!/usr/bin/env python3
"""Paged-attention decode benchmark on one MI355X.

Headline workload (one "step" = one decode call = split-KV kernel + merge
kernel): the pages' shape sweep at its longest context -- batch 1, 32 query
heads over 8 KV heads (ratio 4), head size 128, block size 16, 32768 cached
tokens, bf16 KV ~ N(0,1), zero-filled pool, randomly permuted block table.

Metric: achieved HBM bandwidth over the algorithmic KV bytes (valid tokens
only, K and V, 16-bit: L * Hkv * D * 2 * 2 bytes per call) as GB/s and as a
fraction of the 8 TB/s peak, plus microseconds per call.

Inputs are resident in HBM before timing starts.  Because one call's KV
(128 MiB) would fit in the 256 MB Infinity Cache, consecutive calls rotate
over enough replica pools (same content, same table) that no call finds its
KV in a cache.  Device time comes from HIP events on the stream the kernels
run on; the split-KV kernel's own duration from events the library attaches
to that launch (hipExtLaunchKernel).

Prints ONE JSON line.  Options: --gpus (1 only), --steps, --warmup,
--cpu-seconds (oracle baseline budget), --no-extra (skip the other shapes).
"""
import argparse
import subprocess
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0          # MI355X HBM3E, published
ROTATE_BYTES = 2 << 30     # >= 2 GiB of distinct KV between reuses of one pool


def _cfg():
    from kvgen import configs
    return configs


# The timed workload: the headline one by default; the others for profiling.
WORKLOADS = {
    "headline": dict(make=lambda: _cfg().cfg2(32, 32768, device="cuda"),
                     desc="paged GQA decode, batch 1, 32 query / 8 KV heads, head 128, "
                          "block 16, 32768-token context, bf16 KV ~N(0,1), permuted table"),
    "cfg4-32K": dict(make=lambda: _cfg().cfg4(32768, device="cuda"),
                     desc="low-parallelism decode, batch 1, 24 query / 4 KV heads, head 256, "
                          "block 784, 32768-token context, bf16 KV ~N(0,1)"),
    "cfg3-B8-32K": dict(make=lambda: _cfg().cfg3(8, 32768, device="cuda"),
                        desc="gemma-like decode, batch 8, 32 query / 16 KV heads, head 128, "
                             "block 16, 32768-token contexts, bf16 KV ~N(0,1)"),
    "cfg5": dict(make=lambda: _cfg().cfg5(device="cuda"),
                 desc="mixed-length decode, batch 64, 32 query / 8 KV heads, head 128, "
                      "block 16, contexts U[1K, 32K], bf16 KV ~N(0,1), fragmented tables"),
    "sliding-B8-32K": dict(make=lambda: _cfg().cfg3_sliding(8, 32768, device="cuda"),
                           desc="gemma-like sliding layer, batch 8, 32 query / 16 KV heads, "
                                "head 128, block 16, 32768-token contexts, 1024-token window, "
                                "bf16 KV ~N(0,1)"),
    "sliding-B1-32K": dict(make=lambda: _cfg().cfg3_sliding(1, 32768, device="cuda"),
                           desc="gemma-like sliding layer, batch 1, 32 query / 16 KV heads, "
                                "head 128, block 16, 32768-token context, 1024-token window, "
                                "bf16 KV ~N(0,1)"),
    "headline-1K": dict(make=lambda: _cfg().cfg2(32, 1024, device="cuda"),
                        desc="paged GQA decode, batch 1, 32 query / 8 KV heads, head 128, "
                             "block 16, 1024-token context, bf16 KV ~N(0,1)"),
    "fp8-headline": dict(make=lambda: _cfg().cfg2(32, 32768, device="cuda", kv_dtype="fp8"),
                         desc="paged GQA decode, batch 1, 32 query / 8 KV heads, head 128, "
                              "block 16, 32768-token context, fp8 E4M3 KV with per-tensor "
                              "scales, bf16 q"),
    "fp8-cfg4-32K": dict(make=lambda: _cfg().cfg4(32768, device="cuda", kv_dtype="fp8"),
                         desc="low-parallelism decode, batch 1, 24 query / 4 KV heads, head "
                              "256, block 784, 32768-token context, fp8 E4M3 KV, bf16 q"),
    "tp2-share-12-2-32K": dict(make=lambda: _cfg().cfg4_tp2(32768, device="cuda"),
                               desc="one GPU's share of the low-parallelism layer under two-way "
                                    "tensor parallelism: batch 1, 12 query / 2 KV heads, head "
                                    "256, block 784, 32768-token context, bf16 KV"),
    "q4-headline": dict(make=lambda: _cfg().cfg2(32, 32768, device="cuda", q_len=4),
                        desc="four-row decode, batch 1, 32 query / 8 KV heads, head 128, "
                             "block 16, 32768-token context, bf16 KV"),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def replicas_for(case):
    """KV pools the calls rotate through, so that no call finds the KV it reads
    in the MALL or the L2s: at least ROTATE_BYTES of distinct attended KV lie
    between two uses of one pool.  Returns (pools, block_table, num_blocks);
    the pools share the table.  A sliding window reads a small part of the
    case's pool, so its pools hold only the blocks the windows touch, in a
    seeded random order (the table's other entries point at one of them and
    are never read)."""
    import torch
    if case.sliding_window == 0:
        pool = case.k_cache.numel() * case.k_cache.element_size() * 2
        n = max(1, math.ceil(ROTATE_BYTES / pool))
        reps = [(case.k_cache, case.v_cache)]
        for _ in range(n - 1):
            reps.append((case.k_cache.clone(), case.v_cache.clone()))
        torch.cuda.synchronize()
        return reps, case.block_table, case.num_blocks
    table = case.block_table.cpu()
    need = []
    for b, L in enumerate(case.seq_lens):
        if L > 0:
            lo = max(0, L - case.sliding_window)
            need += [(b, lb) for lb in range(lo // case.bs, (L - 1) // case.bs + 1)]
    gen = torch.Generator()
    gen.manual_seed(20240)
    nb = len(need) + 1
    perm = torch.randperm(nb, generator=gen)
    idx = torch.zeros(nb, dtype=torch.int64)
    new_table = torch.full_like(table, int(perm[-1]))
    for i, (b, lb) in enumerate(need):
        idx[perm[i]] = int(table[b, lb])
        new_table[b, lb] = int(perm[i])
    idx[perm[-1]] = int(table[need[0][0], need[0][1]]) if need else 0
    idx = idx.to(case.k_cache.device)
    kc, vc = case.k_cache[idx].contiguous(), case.v_cache[idx].contiguous()
    pool = kc.numel() * kc.element_size() * 2
    n = max(1, math.ceil(ROTATE_BYTES / pool))
    reps = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(n - 1)]
    torch.cuda.synchronize()
    return reps, new_table.to(case.block_table.device), nb


GRAPH_CALLS = 20  # decode calls captured into the graph of the graph pass


def time_case(case, steps, warmup, passes=1):
    """Per-call device time from passes of plain back-to-back calls (two HIP
    events around the pass), and the split-KV kernel's own duration from
    passes in which the library attaches events to that launch; then the
    per-call time of GRAPH_CALLS calls captured once into a HIP graph and
    replayed (as a serving loop runs its decode step), which leaves out the
    host's per-call launch cost.  Returns a dict with these, the plan and the
    last output (that of the last replay)."""
    import torch
    import kvgen
    import paged_kv_cache_decode_amd as pda
    reps, table, num_blocks = replicas_for(case)
    R = len(reps)
    shape = pda.make_shape(**dict(kvgen.shape_dict(case), num_blocks=num_blocks))
    plan = pda.paged_decode_attn_plan(shape)
    out = torch.empty_like(case.q)
    ws = torch.empty(max(1, pda.pda_workspace_bytes(shape, plan)), dtype=torch.uint8,
                     device=case.q.device)
    pda.paged_decode_attn_workspace_init(ws)

    def call(i, e0=None, e1=None, stream=None):
        kc, vc = reps[i % R]
        pda.paged_decode_attn_timed(shape, plan, case.q, kc, vc, table,
                                    case.seq_lens_t, case.scale, out, ws, e0, e1, stream)

    # every replica pool is touched at least twice before timing (a pool's
    # first use in a process pays for page-table and TLB set-up)
    for i in range(max(warmup, 2 * R)):
        call(i)
    torch.cuda.synchronize()
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for e in ev0 + ev1:
        e.record()  # materialise the HIP event before the library uses it
    torch.cuda.synchronize()
    calls, kernels = [], []
    for _ in range(passes):
        # plain pass: the whole decode step, nothing else on the stream
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        start.record()
        for i in range(steps):
            call(i)
        stop.record()
        torch.cuda.synchronize()
        w1 = time.perf_counter()
        calls.append(dict(call_ms=start.elapsed_time(stop) / steps,
                          wall_ms=(w1 - w0) * 1e3 / steps))
        # instrumented pass: events on the split-KV kernel's own launch
        for i in range(steps):
            call(i, ev0[i], ev1[i])
        torch.cuda.synchronize()
        kernels.append(sum(a.elapsed_time(b) for a, b in zip(ev0, ev1)) / steps)
    order = sorted(range(passes), key=lambda k: calls[k]["call_ms"])
    med = order[len(order) // 2]
    kv = case.kv_bytes()
    # graph pass: capture on a side stream after a warm-up there, replay
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(GRAPH_CALLS):
            call(i, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(GRAPH_CALLS):
            call(i, stream=side)
    for _ in range(2):
        graph.replay()
    replays = max(2, steps // GRAPH_CALLS)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(replays):
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(stop) / (replays * GRAPH_CALLS)
    del graph
    return dict(out=out, plan=plan, replicas=R, passes=calls, call_ms=calls[med]["call_ms"],
                wall_ms=calls[med]["wall_ms"], best_call_ms=calls[order[0]]["call_ms"],
                kernel_ms=sorted(kernels)[len(kernels) // 2], kernel_passes=kernels,
                graph_ms=graph_ms, kv_bytes=kv)


def summary(name, case, r):
    us = r["call_ms"] * 1e3
    kus = r["kernel_ms"] * 1e3
    gbs = r["kv_bytes"] / (r["call_ms"] * 1e-3) / 1e9
    kgbs = r["kv_bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
    return {"workload": name, "B": case.B, "Hq": case.Hq, "Hkv": case.Hkv, "D": case.D,
            "block_size": case.bs, "dtype": case.dtype, "context_tokens": sum(case.seq_lens),
            "sliding_window": case.sliding_window, "q_len": case.q_len, "kv_dtype": case.kv_dtype,
            "kv_bytes": r["kv_bytes"], "P": r["plan"].num_partitions,
            "T_p": r["plan"].tokens_per_partition, "us_per_call": round(us, 3),
            "splitkv_kernel_us": round(kus, 3), "GBps": round(gbs, 1),
            "pct_of_peak": round(100 * gbs / PEAK_GBS, 2),
            "kernel_GBps": round(kgbs, 1), "kernel_pct_of_peak": round(100 * kgbs / PEAK_GBS, 2),
            "us_per_context_token": round(us / sum(case.seq_lens), 6),
            "graph_us_per_call": round(r["graph_ms"] * 1e3, 3),
            "variant": {1: "valu", 2: "mfma"}.get(r["plan"].variant, "?"),
            "merge": {0: "fused", 1: "kernel"}.get(r["plan"].merge, "?"),
            "replica_pools": r["replicas"],
            "passes_us": [round(p["call_ms"] * 1e3, 3) for p in r["passes"]]}


def score(case, out, ref=None):
    """The row's parity ledger entry: rel-L-inf of the GPU output against the
    oracle over the whole call (the pages' metric: against the oracle's own
    output scale), the worst per-sequence figure, and the count of
    non-finite output elements.  `ref` is the oracle's output if already
    computed."""
    import numpy as np
    import oracle
    import kvgen
    g = out.float().cpu().numpy()
    if ref is None:
        q, k, v, lens = kvgen.oracle_inputs(case)
        sc = (case.k_scale, case.v_scale) if case.kv_dtype == "fp8" else None
        if case.q_len > 1:
            ref = oracle.decode_multi(q, k, v, lens, case.scale, window=case.sliding_window,
                                      kv_scales=sc)
        else:
            ref = oracle.decode(q, k, v, lens, case.scale, window=case.sliding_window,
                                kv_scales=sc)
    nan = int(np.count_nonzero(~np.isfinite(g)))
    per_seq = [oracle.rel_linf(g[b], ref[b]) for b in range(case.B)]
    tol = {"bf16": 1e-2, "fp16": 2e-3}[case.dtype]
    return {"rel_linf": float(f"{oracle.rel_linf(g, ref):.4e}"),
            "rel_linf_worst_seq": float(f"{max(per_seq):.4e}"),
            "nonfinite": nan, "tol": tol,
            "pass": bool(nan == 0 and max(per_seq) <= tol and oracle.rel_linf(g, ref) <= tol)}


def kernel_source_hash(variant: str = "mfma") -> str:
    """sha256 over the sources the split-KV kernel of `variant` is compiled
    from (its translation unit, the device and common headers, the C ABI
    header): a change to any of them makes a committed counter summary of
    that kernel stale; changes to other kernels (the merge) do not."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_decode_amd", "csrc")
    files = [os.path.join(csrc, f"pda_decode_{variant}.hip"), os.path.join(csrc, "pda_device.h"),
             os.path.join(csrc, "pda_common.h"), os.path.join(ROOT, "include", "pda.h")]
    for path in files:
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(variant: str):
    """HBM bytes per launch of the headline split-KV kernel from the committed
    rocprofv3 counter summary (profiles/traffic_headline.json), or None when
    that summary was taken from other kernel sources than these."""
    path = os.path.join(ROOT, "profiles", "traffic_headline.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("variant") != variant or t.get("kernel_source_sha256") != kernel_source_hash(variant):
        return None
    return t.get("hbm_bytes_per_launch")


def read_probe(nbytes: int = 4 << 30, calls: int = 10, grids=(256, 512, 1024, 2048)):
    """Achievable HBM read bandwidth: the library's streaming-read probe over
    one buffer of `nbytes` (16x the 256 MB MALL), timed with HIP events over
    `calls` back-to-back reads after two untimed ones, for each grid size in
    `grids`; the best rate is the achievable figure."""
    import torch
    import paged_kv_cache_decode_amd as pda
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    rates = {}
    for wg in grids:
        for _ in range(2):
            pda.pda_read_probe(src, sink, wg)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(calls):
            pda.pda_read_probe(src, sink, wg)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / calls
        rates[wg] = nbytes / (ms * 1e-3) / 1e9
    # the same bytes as a decode call, on the decode's grid: reads of 128 MiB
    # (the 16-bit headline's K+V) and 64 MiB (its fp8 form) by 256 workgroups,
    # rotating over the buffer's slices so that no read finds its slice in the
    # MALL; and the launch floor (a 16-byte read by one workgroup)
    def per_launch_us(size, wgs, n=200):
        nsl = nbytes // size
        for i in range(4):
            pda.pda_read_probe(src[(i % nsl) * size:(i % nsl + 1) * size], sink, wgs)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(n):
            pda.pda_read_probe(src[(i % nsl) * size:(i % nsl + 1) * size], sink, wgs)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3
    same = {}
    for mib in (128, 64):
        us = per_launch_us(mib << 20, 256)
        same[f"{mib}MiB_256wg"] = {"us_per_launch": round(us, 3),
                                   "GBps": round((mib << 20) / (us * 1e-6) / 1e9, 1)}
    # the launch floor: 100 16-byte reads by one workgroup captured into a
    # graph and replayed, so that the host's per-launch cost (more than the
    # device's through the Python binding) is not what is timed
    tiny = src[:16]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pda.pda_read_probe(tiny, sink, 1, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _ in range(100):
            pda.pda_read_probe(tiny, sink, 1, stream=side)
    graph.replay()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(10):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    floor_us = a.elapsed_time(b) / 1000 * 1e3
    del graph
    del src
    torch.cuda.empty_cache()
    best = max(rates, key=rates.get)
    return {"GBps": round(rates[best], 1), "frac_of_peak": round(rates[best] / PEAK_GBS, 4),
            "bytes": nbytes, "workgroups": best,
            "GBps_by_workgroups": {str(k): round(v, 1) for k, v in rates.items()},
            "what": "one streaming read of a 4 GiB buffer with the decode kernels' 16-byte "
                    "non-temporal loads (pda_read_probe), best grid size",
            "same_bytes_same_grid": same,
            "launch_floor_us": round(floor_us, 3),
            "what_same_bytes": "back-to-back reads of 128 MiB and 64 MiB slices of the buffer "
                               "(rotating, so none is served by the MALL) by 256 workgroups, "
                               "per launch; launch floor: a 16-byte read by one workgroup, "
                               "per launch from a graph of 100"}


def cpu_identity() -> dict:
    """The host CPU as /proc/cpuinfo and the scheduler report it: model name,
    family / model / stepping, clock, logical CPUs visible and usable."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ":" not in ln:
                    if info:
                        break  # the first processor's block is enough
                    continue
                k, v = (x.strip() for x in ln.split(":", 1))
                if k in ("vendor_id", "model name", "cpu family", "model", "stepping",
                         "cpu MHz", "cache size") and k not in info:
                    info[k] = v
    except OSError:
        pass
    info["logical_cpus"] = os.cpu_count()
    try:
        info["usable_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    return info


def cpu_baseline(case, seconds):
    """The oracle as it stands, on the host cores, over the same workload."""
    import oracle
    import kvgen
    q, k, v, lens = kvgen.oracle_inputs(case)
    threads = oracle.num_threads()
    n, t = 0, 0.0
    ref = None
    while t < seconds or n == 0:
        t0 = time.perf_counter()
        ref = oracle.decode(q, k, v, lens, case.scale, nthreads=threads,
                            window=case.sliding_window)
        t += time.perf_counter() - t0
        n += 1
    per_call = t / n
    # the same call on one thread, over a bounded share of the budget
    n1, t1 = 0, 0.0
    while t1 < seconds / 4 or n1 == 0:
        t0 = time.perf_counter()
        oracle.decode(q, k, v, lens, case.scale, nthreads=1, window=case.sliding_window)
        t1 += time.perf_counter() - t0
        n1 += 1
    model = cpu_identity()
    return ref, {"value": round(case.kv_bytes() / per_call / 1e9, 3), "unit": "GB/s",
                 "cores": threads, "kind": "oracle",
                 "us_per_call": round(per_call * 1e6, 1),
                 "sample": f"{n} full decode call(s) of the headline workload "
                           f"({case.B}x{case.Hq} rows over {sum(case.seq_lens)} tokens), "
                           f"{t:.1f} s of wall-clock time (time.perf_counter around each "
                           f"call), OpenMP over rows on {threads} threads",
                 "timer": "wall-clock",
                 "single_thread": {"value": round(case.kv_bytes() / (t1 / n1) / 1e9, 3),
                                   "unit": "GB/s", "us_per_call": round(t1 / n1 * 1e6, 1),
                                   "sample": f"{n1} call(s), {t1:.1f} s of wall-clock time"},
                 "cpu_model": model}


def render_table(line: dict) -> str:
    """Markdown table of a bench JSON line: the headline row, then every
    extra row, each with its plan, call and kernel time and fraction of the
    8 TB/s peak, and its parity entry (rel-L-inf, worst sequence, non-finite
    count)."""
    rows = [line["headline"]] + [v for v in line.get("extra", {}).values() if isinstance(v, dict)]
    if line.get("parity") is not None:
        rows[0] = dict(rows[0], parity=line["parity"])
    out = ["| workload | variant | merge | P x T_p | us/call | % of 8 TB/s | split-KV kernel us "
           "(% peak) | graph us/call | rel-Linf (worst seq) | non-finite |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        par = r.get("parity")
        ptxt = "-" if par is None else f"{par['rel_linf']:.2e} ({par['rel_linf_worst_seq']:.2e})"
        ntxt = "-" if par is None else str(par["nonfinite"])
        gtxt = "-" if r.get("graph_us_per_call") is None else f"{r['graph_us_per_call']:.2f}"
        out.append(f"| {r['workload']} | {r['variant']} | {r['merge']} | {r['P']} x {r['T_p']} | "
                   f"{r['us_per_call']:.2f} | {r['pct_of_peak']:.1f} % | "
                   f"{r['splitkv_kernel_us']:.2f} ({r['kernel_pct_of_peak']:.1f} %) | {gtxt} | "
                   f"{ptxt} | {ntxt} |")
    slopes = {k: v for k, v in line.get("extra", {}).items() if not isinstance(v, dict)}
    for k, v in slopes.items():
        out.append(f"\n{k}: {v}")
    return "\n".join(out)


def extra_specs():
    """The extra rows: (name, maker) for every config shape, ladder point and
    next-row workload timed after the headline."""
    from kvgen import configs
    L = 32768
    specs = [(f"cfg2 Hq{hq} 32K", lambda hq=hq: configs.cfg2(hq, L, device="cuda"))
             for hq in (8, 16, 24)]
    specs += [(f"cfg2 Hq32 {n}", lambda n=n: configs.cfg2(32, n, device="cuda"))
              for n in configs.CFG2_LENS]
    specs += [("cfg3 B1 bf16 32K", lambda: configs.cfg3(1, L, device="cuda")),
              ("cfg3 B1 fp16 32K", lambda: configs.cfg3(1, L, dtype="fp16", device="cuda")),
              ("cfg3 B8 bf16 32K", lambda: configs.cfg3(8, L, device="cuda"))]
    specs += [(f"cfg4 {n}", lambda n=n: configs.cfg4(n, device="cuda"))
              for n in configs.CFG4_LENS]
    specs += [("cfg5 B64 mixed", lambda: configs.cfg5(device="cuda"))]
    specs += [(f"cfg3 sliding W1024 B{b} 32K", lambda b=b: configs.cfg3_sliding(b, L, device="cuda"))
              for b in (1, 8)]
    specs += [("cfg4 TP2 share 12/2 32K", lambda: configs.cfg4_tp2(L, device="cuda"))]
    specs += [("headline fp8 KV 32K", lambda: configs.cfg2(32, L, device="cuda", kv_dtype="fp8")),
              ("cfg3 B8 fp8 KV 32K", lambda: configs.cfg3(8, L, device="cuda", kv_dtype="fp8")),
              ("cfg4 fp8 KV 32K", lambda: configs.cfg4(L, device="cuda", kv_dtype="fp8")),
              ("cfg5 B64 mixed fp8 KV", lambda: configs.cfg5(device="cuda", kv_dtype="fp8"))]
    specs += [("headline q_len 4 32K", lambda: configs.cfg2(32, L, device="cuda", q_len=4)),
              ("cfg3 B8 q_len 4 32K", lambda: configs.cfg3(8, L, device="cuda", q_len=4)),
              ("cfg5 B64 mixed q_len 2", lambda: configs.cfg5(device="cuda", q_len=2))]
    specs += [(f"cfg3 TP2 share 16/8 B{b} 32K", lambda b=b: configs.cfg3_tp2(b, L, device="cuda"))
              for b in (1, 8)]
    return specs


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--passes", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle comparison of the extra rows")
    ap.add_argument("--table", metavar="JSON",
                    help="print the markdown table of a stored bench line and exit")
    ap.add_argument("--workload", default="headline", choices=sorted(WORKLOADS),
                    help="the timed workload (default: the headline one)")
    ap.add_argument("--row", metavar="NAME",
                    help="time one extra row in this process and print its summary line "
                         "(the full run starts one such process per row)")
    args = ap.parse_args()
    if args.table:
        with open(args.table) as f:
            print(render_table(json.loads(f.readline())))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode path has no cross-GPU step to measure here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import paged_kv_cache_decode_amd as pda
    from kvgen import configs

    torch.cuda.set_device(0)
    pda.load_library()
    if args.row:
        makers = dict(extra_specs())
        if args.row not in makers:
            print(f"no extra row named {args.row!r}", file=sys.stderr)
            sys.exit(2)
        log(f"timing {args.row}")
        c = makers[args.row]()
        rr = time_case(c, args.steps, args.warmup, passes=args.passes)
        row = summary(args.row, c, rr)
        if not args.no_parity:
            row["parity"] = score(c, rr["out"])
        print(json.dumps(row), flush=True)
        return
    log(f"library: {pda.pda_build_id()}")

    wl = WORKLOADS[args.workload]
    case = wl["make"]()
    log(f"timing workload {args.workload}: {wl['desc']}")
    r = time_case(case, args.steps, args.warmup, passes=args.passes)
    head = summary(args.workload, case, r)

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        ref, cpu = cpu_baseline(case, args.cpu_seconds)
        parity = score(case, r["out"], ref)

    kbytes = r["kv_bytes"]
    call_ms, kernel_ms = r["call_ms"], r["kernel_ms"]
    desc_case = dict(B=case.B, max_seq_len=case.max_seq_len)
    del case, r
    torch.cuda.empty_cache()

    extra = {}
    if not args.no_extra:
        small_steps = max(20, args.steps // 4)
        # each row in a process of its own: a row's pools are then its
        # process's first allocation, as a serving KV cache is, instead of
        # landing in memory that earlier rows freed (measured 4-6 % slower
        # per call on the 32K rows)
        for name, _ in extra_specs():
            cmd = [sys.executable, os.path.abspath(__file__), "--row", name,
                   "--steps", str(small_steps), "--warmup", str(max(5, args.warmup // 4)),
                   "--passes", "3"] + (["--no-parity"] if args.no_parity else [])
            res = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=600)
            if res.returncode != 0:
                log(f"row {name!r} failed (exit {res.returncode})")
                sys.exit(1)
            extra[name] = json.loads(res.stdout.strip().splitlines()[-1])
        # decode time added per token of context: the slope of us/call over each ladder
        def slope(points):
            xs = np.array([a for a, _ in points], dtype=np.float64)
            ys = np.array([b for _, b in points], dtype=np.float64)
            return round(float(np.polyfit(xs, ys, 1)[0]), 6)
        extra["cfg4 slope us per context token"] = slope(
            [(extra[f"cfg4 {n}"]["context_tokens"], extra[f"cfg4 {n}"]["us_per_call"])
             for n in configs.CFG4_LENS])
        extra["headline slope us per context token"] = slope(
            [(n, extra[f"cfg2 Hq32 {n}"]["us_per_call"]) for n in configs.CFG2_LENS])

    achieved = kbytes / (kernel_ms * 1e-3) / 1e9
    probe = None
    if not args.no_probe:
        log("timing the streaming-read probe")
        probe = read_probe()
        probe["decode_kernel_frac_of_probe"] = round(achieved / probe["GBps"], 4)
    line = {
        "metric": "achieved KV HBM GB/s (% of MI355X peak) and us/call at 32K-context decode",
        "value": head["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(call_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl["desc"], "global_batch": desc_case["B"],
                   "seq_len": desc_case["max_seq_len"],
                   "parallelism": "single GPU"},
        "us_per_call": head["us_per_call"],
        "pct_of_peak": head["pct_of_peak"],
        "us_per_context_token": head["us_per_context_token"],
        "plan": {"P": head["P"], "T_p": head["T_p"], "merge": head["merge"],
                 "replica_pools": head["replica_pools"]},
        "passes_us": head["passes_us"],
        "roofline": {"bound": "hbm",
                     "kernel": f"decode_{head['variant']}_kernel (split-KV)",
                     "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": measured_traffic(head["variant"]),
                     "kernel_us": round(kernel_ms * 1e3, 3),
                     "call_frac": round(head["GBps"] / PEAK_GBS, 4),
                     "call_us": head["us_per_call"],
                     "algorithmic_bytes_per_launch": kbytes},
        "cpu_baseline": cpu,
        "read_probe": probe,
        "parity_rel_linf_vs_oracle": None if parity is None else parity["rel_linf"],
        "parity": parity,
        "headline": head,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

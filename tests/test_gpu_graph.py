"""A decode call captured into a HIP graph (through torch.cuda.graph) and
replayed gives the eager result, bit for bit, on every replay: the library
enqueues its kernels on the caller's stream, allocates nothing when given a
plan, an output and a workspace, and never synchronises.  Replays are
interleaved with eager calls and synchronisations, and the query rows change
between replays (copied into the captured buffer), as a serving loop would."""
import numpy as np
import pytest
import torch

import kvgen
import paged_kv_cache_decode_amd as pda
from kvgen import configs

from helpers import bits, check, to_device

pytestmark = pytest.mark.gpu


def _call(case, out, ws, plan, stream):
    pda.paged_decode_attn_with_plan(case.q, case.k_cache, case.v_cache, case.block_table,
                                    case.seq_lens_t, case.scale, plan, out=out, workspace=ws,
                                    max_seq_len=case.max_seq_len, stream=stream,
                                    sliding_window=case.sliding_window, k_scale=case.k_scale,
                                    v_scale=case.v_scale)


CASES = {
    "tiny": lambda: configs.cfg1(device="cuda"),
    "cfg4-4K": lambda: configs.cfg4(4096, device="cuda"),
    "mixed-B16": lambda: configs.cfg5(device="cuda", B=16, lo=100, hi=3000),
    "fp8-window": lambda: to_device(kvgen.make_case(3, 16, 4, 128, 16, [900, 33, 2000], seed=11,
                                                    sliding_window=256, kv_dtype="fp8")),
}


@pytest.mark.parametrize("mk", sorted(CASES))
def test_graph_replays_match_eager(mk):
    case = CASES[mk]()
    shape = pda.make_shape(**kvgen.shape_dict(case))
    plan = pda.paged_decode_attn_plan(shape)
    ws = torch.zeros(max(1, pda.pda_workspace_bytes(shape, plan)), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(case.q)
    gen = torch.Generator(device="cpu").manual_seed(5)
    qs = [case.q.clone()] + [torch.randn(case.q.shape, generator=gen).to(case.q.dtype).cuda()
                             for _ in range(2)]
    eager = []
    for q in qs:
        case.q.copy_(q)
        _call(case, out, ws, plan, None)
        torch.cuda.synchronize()
        eager.append(out.clone())
    case.q.copy_(qs[0])
    check(case, eager[0])  # the eager call itself is right

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        _call(case, out, ws, plan, stream)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        _call(case, out, ws, plan, stream)
    torch.cuda.synchronize()
    scratch = torch.empty_like(out)
    for rep in range(6):
        k = rep % len(qs)
        case.q.copy_(qs[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(eager[k])), f"replay {rep}"
        _call(case, scratch, ws, plan, None)  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(bits(scratch), bits(eager[k])), f"eager after replay {rep}"


def test_graph_with_workspace_init_and_fused_merge():
    """The workspace fill is a kernel, so a graph may hold it: captured
    before a fused-merge call, it re-zeroes the arrival counters on every
    replay even after eager work left garbage in the workspace."""
    case = configs.cfg2(32, 2048, device="cuda")
    shape = pda.make_shape(**kvgen.shape_dict(case))
    plan = pda.paged_decode_attn_plan(shape)
    plan.merge = pda.PDA_MERGE_FUSED
    assert plan.num_partitions > 1
    ws = torch.empty(pda.pda_workspace_bytes(shape, plan), dtype=torch.uint8, device="cuda")
    pda.paged_decode_attn_workspace_init(ws)
    out = torch.empty_like(case.q)
    _call(case, out, ws, plan, None)
    torch.cuda.synchronize()
    eager = out.clone()
    check(case, eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        pda.paged_decode_attn_workspace_init(ws, stream=stream)
        _call(case, out, ws, plan, stream)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        pda.paged_decode_attn_workspace_init(ws, stream=stream)
        _call(case, out, ws, plan, stream)
    for rep in range(4):
        ws.fill_(0x7F)  # garbage counters and partials
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(eager)), f"replay {rep}"


def test_default_stream_follows_torch_current_stream():
    """With no stream argument the binding launches on torch's current stream
    (read as a raw handle): the default stream outside a stream context, the
    context's stream inside one; a capture then needs no stream argument."""
    assert pda._stream(None) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert pda._stream(None) == side.cuda_stream
    assert pda._stream(None) == torch.cuda.current_stream().cuda_stream
    case = configs.cfg1(device="cuda")
    shape = pda.make_shape(**kvgen.shape_dict(case))
    plan = pda.paged_decode_attn_plan(shape)
    ws = torch.zeros(max(1, pda.pda_workspace_bytes(shape, plan)), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(case.q)
    _call(case, out, ws, plan, None)
    torch.cuda.synchronize()
    eager = out.clone()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(case, out, ws, plan, None)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        _call(case, out, ws, plan, None)
    out.zero_()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(eager))

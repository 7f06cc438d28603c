"""The no-allocation entry point (paged_decode_attn_noalloc) against the
existing one (paged_decode_attn), through the C ABI.

Both run the same kernels under the same device plan, so the outputs must be
bit-identical, and each within the decode's tolerance of the oracle.  Two
calls in a row share the library's static per-GPU workspace, the second with
a smaller input; a plan whose workspace exceeds the static maximum is
refused before anything is launched.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_decode_amd as pda
from kvgen import configs

from helpers import bits, check, shape_of

pytestmark = pytest.mark.gpu


def _noalloc(case, out=None):
    if out is None:
        out = torch.empty_like(case.q)
    pda.paged_decode_attn_noalloc(case.q, case.k_cache, case.v_cache, case.block_table,
                                  case.seq_lens_t, case.scale, out,
                                  max_seq_len=case.max_seq_len,
                                  sliding_window=case.sliding_window, k_scale=case.k_scale,
                                  v_scale=case.v_scale)
    torch.cuda.synchronize()
    return out


def _existing(case):
    out = pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                case.seq_lens_t, case.scale, max_seq_len=case.max_seq_len,
                                sliding_window=case.sliding_window, k_scale=case.k_scale,
                                v_scale=case.v_scale)
    torch.cuda.synchronize()
    return out


# pairs of calls in a row, the second smaller; between them the four plans
# of the configs: merge kernel (32 and 64 partitions), fused merge (many
# units, and few), and a single partition (no workspace)
PAIRS = {
    "headline-then-1K": (lambda: configs.cfg2(32, 32768, device="cuda"),
                         lambda: configs.cfg2(32, 1024, device="cuda")),
    "cfg5-then-short": (lambda: configs.cfg5(device="cuda"),
                        lambda: configs.cfg5(device="cuda", lo=1, hi=3000, cell=1)),
    "cfg4-then-500": (lambda: configs.cfg4(32768, device="cuda"),
                      lambda: configs.cfg4(500, device="cuda")),
    "cfg3B8-then-tiny": (lambda: configs.cfg3(8, 4090, device="cuda", dtype="fp16"),
                         lambda: configs.cfg1("fp16", device="cuda")),
}


@pytest.mark.parametrize("name", sorted(PAIRS))
def test_noalloc_matches_existing_entry_point(name):
    merges = []
    for mk in PAIRS[name]:
        case = mk()
        plan = pda.paged_decode_attn_plan(shape_of(case))
        assert plan.workspace_bytes <= pda.PDA_NOALLOC_MAX_WORKSPACE
        merges.append((plan.num_partitions, plan.merge))
        got = _noalloc(case)
        ref = _existing(case)
        assert np.array_equal(bits(got), bits(ref)), f"{name}: differs from paged_decode_attn"
        check(case, got, per_seq=True)
    print(name, merges)


def test_noalloc_repeated_calls_and_fused_counters():
    """Fused-merge calls back to back on the shared array: each leaves its
    arrival counters zero for the next, so every call is identical."""
    case = configs.cfg2(32, 2048, device="cuda")
    plan = pda.paged_decode_attn_plan(shape_of(case))
    assert plan.num_partitions > 1 and plan.merge == pda.PDA_MERGE_FUSED
    first = bits(_noalloc(case))
    out = torch.empty_like(case.q)
    for _ in range(5):
        _noalloc(case, out)
        assert np.array_equal(first, bits(out))
    assert np.array_equal(first, bits(_existing(case)))


def test_noalloc_refuses_oversized_workspace():
    """A shape whose plan needs more than the static array: PDA_ERR_WORKSPACE,
    raised before any launch (the shape is validated on the host only)."""
    B, Hq, Hkv, D = 64, 32, 8, 256
    shape = pda.make_shape(B, Hq, Hkv, D, 16, 65536, 4096, 65536, q_len=4)
    plan = pda.paged_decode_attn_plan(shape)
    assert plan.workspace_bytes > pda.PDA_NOALLOC_MAX_WORKSPACE
    q = torch.zeros((B, 4, Hq, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, Hkv, 16, D), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((B, 4096), dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(pda.PdaError) as err:
        pda.paged_decode_attn_noalloc(q, kc, kc, table, lens, 1.0, torch.empty_like(q),
                                      max_seq_len=65536)
    assert err.value.status == pda.PDA_ERR_WORKSPACE

"""GPU parity of multi-row decode against the CPU oracle, through the C ABI.

Each sequence brings q_len query rows at its last q_len positions; row i
attends causally to the tokens up to its own position (optionally within a
sliding window).  The oracle computes each row as the plain decode of the
sequence's prefix (oracle.decode_multi).  Same tolerances as the one-row
decode; rows with no token (L < q_len) are zeros; one row through the 4-D
layout is bit-identical to the 3-D call.
"""
from dataclasses import replace

import numpy as np
import pytest

import kvgen
import paged_kv_cache_decode_amd as pda
from kvgen import configs
from oracle import bookkeeping
from oracle import plan as oplan

from helpers import bits, check, reference, run, shape_of, to_device

pytestmark = pytest.mark.gpu

VARIANTS = {"valu": pda.PDA_VARIANT_VALU, "mfma": pda.PDA_VARIANT_MFMA}


def plan_of(P, T, variant, merge=pda.PDA_MERGE_KERNEL):
    return pda.PdaPlan(num_partitions=P, tokens_per_partition=T, variant=variant, merge=merge,
                       cu_count=0, workspace_bytes=0)


def round64(x):
    return -(-x // 64) * 64


def plans_for(case, variant):
    """The device plan with the variant forced, one partition over the span,
    three partitions (both merges) and 64-token partitions (fused merge,
    two past the span)."""
    v = VARIANTS[variant]
    dev = pda.paged_decode_attn_plan(shape_of(case))
    dev.variant = v
    S = oplan.span(case.max_seq_len, case.sliding_window, case.q_len)
    T3 = max(64, round64(-(-S // 3)))
    return [dev, plan_of(1, round64(S), v), plan_of(3, T3, v),
            plan_of(3, T3, v, merge=pda.PDA_MERGE_FUSED),
            plan_of(-(-S // 64) + 2, 64, v, merge=pda.PDA_MERGE_FUSED)]


def multi_case(D, bs, G, lens, n, W=0, seed=0, dtype="bf16", Hkv=2):
    return to_device(kvgen.make_case(len(lens), G * Hkv, Hkv, D, bs, lens, dtype=dtype, seed=seed,
                                     extra_blocks=3, tail_k="nan", tail_v="nan",
                                     sliding_window=W, q_len=n))


MULTI_CASES = [
    # D, bs, G, lens, q_len, W
    (128, 16, 4, [1000, 3, 17, 0], 2, 0),
    (128, 16, 4, [2049, 40], 4, 0),
    (128, 16, 4, [777, 5], 8, 0),          # 32 rows: two 16-row chunks
    (64, 5, 1, [1234, 2, 99], 8, 0),
    (64, 16, 2, [500, 64], 3, 0),
    (256, 784, 6, [3000, 785], 2, 0),
    (256, 784, 6, [1600, 4], 5, 0),        # 30 rows at head 256
    (128, 1, 8, [300, 301], 2, 0),
    (128, 16, 2, [4090, 1, 333], 4, 1024),
    (256, 16, 4, [5000, 300], 3, 513),
    (64, 48, 16, [900, 47], 2, 0),
]


@pytest.mark.parametrize("variant", ["valu", "mfma"])
@pytest.mark.parametrize("D,bs,G,lens,n,W", MULTI_CASES)
def test_multi_row_parity(D, bs, G, lens, n, W, variant):
    case = multi_case(D, bs, G, lens, n, W, seed=D + bs + G + n + W)
    if variant == "valu" and n * G > 8:
        # beyond the VALU variant's 8 rows per unit: every plan for it is
        # refused on the host, before anything is launched
        for plan in plans_for(case, variant):
            with pytest.raises(pda.PdaError) as err:
                run(case, plan=plan)
            assert err.value.status == pda.PDA_ERR_UNSUPPORTED
        return
    ref = reference(case)
    for plan in plans_for(case, variant):
        print(f"plan P={plan.num_partitions} T={plan.tokens_per_partition} "
              f"merge={plan.merge}", flush=True)
        got = run(case, plan=plan)
        assert tuple(got.shape) == (case.B, n, case.Hq, D)
        check(case, got, ref, per_seq=True)
        g = got.float().cpu().numpy()
        for b, L in enumerate(lens):
            for i in range(n):
                if L - n + i + 1 <= 0:
                    assert np.all(g[b, i] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_multi_row_fp16_and_bf16(dtype):
    case = multi_case(128, 16, 4, [3000, 1500, 12], 4, seed=7, dtype=dtype)
    check(case, run(case), per_seq=True)


@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_one_row_in_the_4d_layout_is_the_3d_call(variant):
    case = multi_case(128, 16, 2, [1500, 777, 16], 1, seed=3)
    assert case.q.dim() == 3
    plan = pda.paged_decode_attn_plan(shape_of(case))
    plan.variant = VARIANTS[variant]
    a = run(case, plan=plan)
    case4 = replace(case, q=case.q.unsqueeze(1).contiguous())
    b = run(case4, plan=plan)
    assert tuple(b.shape) == (3, 1, case.Hq, 128)
    assert np.array_equal(bits(a), bits(b[:, 0]))


@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_multi_row_trace_bit_exact(variant):
    n, W = 3, 100
    case = multi_case(128, 16, 2, [1000, 40, 2], n, W, seed=11)
    shape = shape_of(case)
    for plan in plans_for(case, variant)[:3]:
        slot, part, ranges = pda.paged_decode_attn_trace(shape, plan, case.block_table,
                                                         case.seq_lens_t, rows=0)
        e_slot, e_part, e_ranges, valid = bookkeeping.expected_trace(
            case.block_table.cpu().numpy(), case.seq_lens, case.Hkv, case.bs, case.max_seq_len,
            plan.num_partitions, plan.tokens_per_partition, window=W, q_len=n)
        slot, part, ranges = slot.cpu().numpy(), part.cpu().numpy(), ranges.cpu().numpy()
        Lm = case.max_seq_len
        assert np.array_equal(slot[..., :Lm][valid], e_slot[valid])
        assert np.array_equal(part[..., :Lm][valid], e_part[valid])
        assert np.all(slot[..., :Lm][~valid] == -1)
        assert np.array_equal(ranges, e_ranges)


@pytest.mark.parametrize("n", [2, 4])
def test_multi_row_poison_before_window_bit_identical(n):
    case = multi_case(128, 16, 2, [4090, 2000], n, 1024, seed=13)
    bad = kvgen.poison_before_window(case, "nan")
    for plan in plans_for(case, "mfma")[:3]:
        assert np.array_equal(bits(run(case, plan=plan)), bits(run(bad, plan=plan)))


# ---- full size -----------------------------------------------------------
@pytest.mark.parametrize("mk", ["headline-q4", "cfg3-B8-q4", "cfg5-q2", "cfg4-q2"])
def test_multi_row_full_size(mk):
    case = {"headline-q4": lambda: configs.cfg2(32, 32768, device="cuda", q_len=4),
            "cfg3-B8-q4": lambda: configs.cfg3(8, 32768, device="cuda", q_len=4),
            "cfg5-q2": lambda: configs.cfg5(device="cuda", q_len=2),
            "cfg4-q2": lambda: configs.cfg4(32768, device="cuda", q_len=2)}[mk]()
    got = run(case)
    check(case, got, per_seq=True)

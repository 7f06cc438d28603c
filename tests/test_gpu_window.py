"""GPU parity of sliding-window decode against the CPU oracle, through the C ABI.

A sliding layer attends to the last W tokens of each sequence, [max(0, L-W), L)
(the sliding layers of page "vLLM's custom ROCm paged-attention kernel wins all
sixty cells", section 4, Figure 3: they scan 1024 tokens).  Same tolerances as
the full decode; slots before the window are never read, so poisoning them
leaves the output bit-identical; W >= L is the full decode.
"""
from dataclasses import replace

import numpy as np
import pytest

import kvgen
import oracle
import paged_kv_cache_decode_amd as pda
from kvgen import configs
from oracle import bookkeeping
from oracle import plan as oplan

from helpers import bits, check, reference, run, shape_of, to_device

pytestmark = pytest.mark.gpu

VARIANTS = {"valu": pda.PDA_VARIANT_VALU, "mfma": pda.PDA_VARIANT_MFMA}

WINDOW_CASES = [
    # D, bs, G, lens, W
    (128, 16, 2, [17, 40, 1000, 0], 16),
    (128, 16, 4, [4090, 1, 333], 1024),
    (256, 784, 6, [32768, 3000, 785], 4096),
    (64, 5, 3, [1234, 99, 5], 100),
    (128, 1, 8, [2000, 2001], 1),
    (64, 48, 1, [777, 1500], 700),
    (256, 16, 2, [300, 5000], 513),
    (128, 16, 11, [3000, 17], 1000),
    (128, 784, 4, [1600, 1569, 2353], 785),
]


def plan_of(P, T, variant, merge=pda.PDA_MERGE_KERNEL):
    return pda.PdaPlan(num_partitions=P, tokens_per_partition=T, variant=variant, merge=merge,
                       cu_count=0, workspace_bytes=0)


def round64(x):
    return -(-x // 64) * 64


def window_case(D, bs, G, lens, W, seed, tail="nan"):
    Hkv = 2
    return to_device(kvgen.make_case(len(lens), G * Hkv, Hkv, D, bs, lens, seed=seed,
                                     extra_blocks=3, tail_k=tail, tail_v=tail,
                                     sliding_window=W))


def plans_for(case, variant):
    """The device plan with the variant forced, plus forced plans: one
    partition over the span, three partitions (both merges), and 64-token
    partitions with two empty ones past the span."""
    v = VARIANTS[variant]
    dev = pda.paged_decode_attn_plan(shape_of(case))
    dev.variant = v
    S = oplan.span(case.max_seq_len, case.sliding_window)
    T3 = max(64, round64(-(-S // 3)))
    return [dev, plan_of(1, round64(S), v), plan_of(3, T3, v),
            plan_of(3, T3, v, merge=pda.PDA_MERGE_FUSED),
            plan_of(-(-S // 64) + 2, 64, v, merge=pda.PDA_MERGE_FUSED)]


@pytest.mark.parametrize("variant", ["valu", "mfma"])
@pytest.mark.parametrize("D,bs,G,lens,W", WINDOW_CASES)
def test_window_parity(D, bs, G, lens, W, variant):
    case = window_case(D, bs, G, lens, W, seed=D * 7 + bs + G + W)
    if variant == "valu" and G > 8:
        # beyond the VALU variant's groups of 8: refused on the host
        for plan in plans_for(case, variant):
            with pytest.raises(pda.PdaError) as err:
                run(case, plan=plan)
            assert err.value.status == pda.PDA_ERR_UNSUPPORTED
        return
    ref = reference(case)
    for plan in plans_for(case, variant):
        print(f"plan P={plan.num_partitions} T={plan.tokens_per_partition} "
              f"merge={plan.merge}", flush=True)
        check(case, run(case, plan=plan), ref, per_seq=True)


@pytest.mark.parametrize("variant", ["valu", "mfma"])
@pytest.mark.parametrize("fill", ["nan", "1e4"])
@pytest.mark.parametrize("D,bs,G,lens,W", [WINDOW_CASES[1], WINDOW_CASES[2], WINDOW_CASES[3],
                                           WINDOW_CASES[8]])
def test_poison_before_window_bit_identical(D, bs, G, lens, W, fill, variant):
    """Tokens before the window sit in cache slots the decode must not read:
    filling them with NaN or 1e4 changes no output bit."""
    case = window_case(D, bs, G, lens, W, seed=5 + W)
    bad = kvgen.poison_before_window(case, fill)
    for plan in plans_for(case, variant)[:4]:
        a = run(case, plan=plan)
        b = run(bad, plan=plan)
        assert np.array_equal(bits(a), bits(b))
    check(case, b, per_seq=True)


@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_window_covering_context_is_full_decode(variant):
    """With W >= every L the window starts at token 0: under one plan the
    result is bit-identical to the decode without a window."""
    lens = [1500, 777, 16]
    full = window_case(128, 16, 4, lens, 0, seed=3)
    plan = plan_of(4, 384, VARIANTS[variant])
    ref = bits(run(full, plan=plan))
    for W in (1500, 1501, 40000):
        assert np.array_equal(bits(run(replace(full, sliding_window=W), plan=plan)), ref)


@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_window_of_one_token_is_the_last_v_row(variant):
    lens = [1, 2, 17, 1000]
    case = window_case(128, 16, 4, lens, 1, seed=17)
    for plan in plans_for(case, variant):
        got = run(case, plan=plan)
        for b, L in enumerate(lens):
            for h in range(case.Hq):
                assert np.array_equal(bits(got[b, h]), bits(case.v[b][h // case.G, L - 1]))


@pytest.mark.parametrize("rows", [0, 1])
@pytest.mark.parametrize("variant", ["valu", "mfma"])
@pytest.mark.parametrize("D,bs,G,lens,W", WINDOW_CASES)
def test_window_trace_bit_exact(D, bs, G, lens, W, variant, rows):
    case = window_case(D, bs, G, lens, W, seed=101)
    shape = shape_of(case)
    if variant == "valu" and G > 8:
        # beyond the VALU variant's groups of 8: the trace refuses its plans
        for plan in plans_for(case, variant)[:3]:
            with pytest.raises(pda.PdaError) as err:
                pda.paged_decode_attn_trace(shape, plan, case.block_table, case.seq_lens_t,
                                            rows=rows)
            assert err.value.status == pda.PDA_ERR_UNSUPPORTED
        return
    for plan in plans_for(case, variant)[:3]:
        slot, part, ranges = pda.paged_decode_attn_trace(shape, plan, case.block_table,
                                                         case.seq_lens_t, rows=rows)
        e_slot, e_part, e_ranges, valid = bookkeeping.expected_trace(
            case.block_table.cpu().numpy(), case.seq_lens, case.Hkv, bs, case.max_seq_len,
            plan.num_partitions, plan.tokens_per_partition, window=W)
        slot, part, ranges = slot.cpu().numpy(), part.cpu().numpy(), ranges.cpu().numpy()
        Lm = case.max_seq_len
        assert np.array_equal(slot[..., :Lm][valid], e_slot[valid])
        assert np.array_equal(part[..., :Lm][valid], e_part[valid])
        # tokens before the window and past the end are never located
        assert np.all(slot[..., :Lm][~valid] == -1) and np.all(part[..., :Lm][~valid] == -1)
        assert np.array_equal(ranges, e_ranges)


# ---- the gemma-like model's sliding layers at full size ------------------
@pytest.mark.parametrize("variant", ["valu", "mfma"])
@pytest.mark.parametrize("B,L", [(1, 32768), (8, 32768), (8, 1024), (8, 1025), (1, 16391)])
def test_sliding_layer_full_size(B, L, variant):
    case = configs.cfg3_sliding(B, L, device="cuda")
    plan = pda.paged_decode_attn_plan(shape_of(case))
    plan.variant = VARIANTS[variant]
    got = run(case, plan=plan)
    check(case, got, per_seq=True)
    # the window makes a large difference once it cuts most of the context
    if L >= 2 * case.sliding_window:
        q, k, v, lens = kvgen.oracle_inputs(case, [0])
        full = oracle.decode(q, k, v, lens, case.scale)
        assert oracle.rel_linf(got[:1].float().cpu().numpy(), full) > 0.05

"""GPU parity of the fp8 (OCP E4M3) KV cache against the CPU oracle, through
the C ABI.

The caches hold E4M3 bytes with one scale per tensor; the oracle decodes the
bytes from the format's definition and runs the same fp32 decode.  Every E4M3
value is exactly a bf16, fp16 and fp32 value, and the kernel's arithmetic is
the 16-bit path's (fp32 accumulation), so the tolerances of the query type
carry over (bf16 1e-2, fp16 2e-3): parity is against the oracle on the same
quantised inputs.  The quantisation error itself belongs to the input, not to
the kernel (reported by test_fp8_quantisation_error_is_the_inputs).
"""
import numpy as np
import pytest
import torch

import kvgen
import oracle
import paged_kv_cache_decode_amd as pda
from kvgen import configs
from oracle import plan as oplan

from helpers import bits, check, reference, run, shape_of, to_device

pytestmark = pytest.mark.gpu


def plan_of(P, T, merge=pda.PDA_MERGE_KERNEL):
    return pda.PdaPlan(num_partitions=P, tokens_per_partition=T, variant=pda.PDA_VARIANT_MFMA,
                       merge=merge, cu_count=0, workspace_bytes=0)


def round64(x):
    return -(-x // 64) * 64


def fp8_case(D, bs, G, lens, n=1, W=0, seed=0, dtype="bf16", Hkv=2, tail="nan"):
    return to_device(kvgen.make_case(len(lens), G * Hkv, Hkv, D, bs, lens, dtype=dtype, seed=seed,
                                     extra_blocks=3, tail_k=tail, tail_v=tail,
                                     sliding_window=W, q_len=n, kv_dtype="fp8"))


def plans_for(case):
    dev = pda.paged_decode_attn_plan(shape_of(case))
    assert dev.variant == pda.PDA_VARIANT_MFMA
    S = oplan.span(case.max_seq_len, case.sliding_window, case.q_len)
    T3 = max(64, round64(-(-S // 3)))
    return [dev, plan_of(1, round64(S)), plan_of(3, T3),
            plan_of(3, T3, merge=pda.PDA_MERGE_FUSED),
            plan_of(-(-S // 64) + 2, 64, merge=pda.PDA_MERGE_FUSED)]


FP8_CASES = [
    # D, bs, G, lens, q_len, W
    (128, 16, 4, [2049, 1, 333, 0], 1, 0),
    (128, 16, 1, [1000, 17], 1, 0),
    (64, 5, 3, [1234, 99, 5], 1, 0),
    (256, 784, 6, [3000, 785], 1, 0),
    (256, 16, 2, [500, 1568], 1, 0),
    (128, 1, 8, [300, 301], 1, 0),
    (64, 48, 16, [900, 47], 1, 0),
    (128, 16, 2, [4090, 40], 4, 0),
    (128, 16, 4, [777, 5], 8, 0),
    (128, 16, 2, [4090, 2000], 1, 1024),
    (256, 784, 6, [1600, 1569], 2, 500),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D,bs,G,lens,n,W", FP8_CASES)
def test_fp8_parity(D, bs, G, lens, n, W, dtype):
    case = fp8_case(D, bs, G, lens, n, W, seed=D + bs + G + n + W, dtype=dtype)
    ref = reference(case)
    for plan in plans_for(case):
        print(f"plan P={plan.num_partitions} T={plan.tokens_per_partition} "
              f"merge={plan.merge}", flush=True)
        check(case, run(case, plan=plan), ref, per_seq=True)


@pytest.mark.parametrize("tail", ["nan", "1e4"])
def test_fp8_poisoned_tails_bit_identical(tail):
    """NaN (S.1111.111) or the largest finite byte in every unwritten slot
    and unreferenced block changes no output bit."""
    clean = fp8_case(128, 16, 4, [2049, 333, 17], seed=21, tail="zero")
    bad = to_device(kvgen.page(kvgen.make_case(3, 8, 2, 128, 16, [2049, 333, 17], seed=21,
                                               extra_blocks=3, kv_dtype="fp8"), tail, tail))
    for plan in plans_for(clean)[:4]:
        assert np.array_equal(bits(run(clean, plan=plan)), bits(run(bad, plan=plan)))


def test_fp8_block_permutation_bit_identical():
    case = fp8_case(256, 784, 6, [3000, 1, 2049], seed=91)
    a = run(case)
    b = run(kvgen.repermute(case, seed=92))
    assert np.array_equal(bits(a), bits(b))


def test_fp8_valu_plan_rejected():
    case = fp8_case(128, 16, 1, [100], seed=1)
    plan = pda.paged_decode_attn_plan(shape_of(case))
    plan.variant = pda.PDA_VARIANT_VALU
    with pytest.raises(pda.PdaError):
        run(case, plan=plan)


def test_fp8_quantisation_error_is_the_inputs():
    """The kernel matches the oracle on the quantised inputs to the bf16
    tolerance, while both differ from the decode of the unquantised 16-bit
    values by the E4M3 rounding (3 mantissa bits): a property of the data."""
    lens = [4096, 1500]
    f8 = fp8_case(128, 16, 4, lens, seed=33)
    ref8 = reference(f8)
    err_kernel = check(f8, run(f8), ref8)
    q, k, v, L = kvgen.oracle_inputs(f8)
    # the 16-bit KV the fp8 bytes quantise: redraw with the same seed
    full = kvgen.make_case(2, 8, 2, 128, 16, lens, seed=33, extra_blocks=3, tail_k="nan",
                           tail_v="nan")
    qf, kf, vf, _ = kvgen.oracle_inputs(full)
    err_quant = oracle.rel_linf(ref8, oracle.decode(q, kf, vf, L, f8.scale))
    print(f"kernel vs oracle on fp8 inputs {err_kernel:.2e}; fp8 vs bf16 KV {err_quant:.2e}")
    assert err_kernel <= 1e-2 and err_quant > err_kernel


# ---- full size -----------------------------------------------------------
@pytest.mark.parametrize("mk", ["headline", "cfg4-32K", "cfg5", "cfg3-B8"])
def test_fp8_full_size(mk):
    case = {"headline": lambda: configs.cfg2(32, 32768, device="cuda", kv_dtype="fp8"),
            "cfg4-32K": lambda: configs.cfg4(32768, device="cuda", kv_dtype="fp8"),
            "cfg5": lambda: configs.cfg5(device="cuda", kv_dtype="fp8"),
            "cfg3-B8": lambda: configs.cfg3(8, 32768, device="cuda", kv_dtype="fp8")}[mk]()
    got = run(case)
    check(case, got, per_seq=True)

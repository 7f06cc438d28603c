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


# every finite E4M3 code (the two NaN codes, 0x7F and 0xFF, read as 0)
FINITE_CODES = np.array([c if c not in (0x7F, 0xFF) else 0 for c in range(256)], dtype=np.uint8)


def _one_block_fp8(B, Hq, D, rows, dtype, q, scale):
    """B sequences of len(rows) tokens sharing one physical block of 16 slots
    whose K and V rows are the given (k_bytes, v_bytes) pairs; the tail
    slots and the second block hold NaN codes."""
    kc = torch.full((2, 1, 16, D), 0x7F, dtype=torch.uint8)
    vc = torch.full((2, 1, 16, D), 0x7F, dtype=torch.uint8)
    for t, (kb, vb) in enumerate(rows):
        kc[0, 0, t] = torch.from_numpy(kb)
        vc[0, 0, t] = torch.from_numpy(vb)
    L = len(rows)
    table = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = pda.paged_decode_attn(q.cuda(), kc.cuda().view(torch.float8_e4m3fn),
                                vc.cuda().view(torch.float8_e4m3fn), table, lens, scale,
                                max_seq_len=L, k_scale=1.0, v_scale=1.0)
    torch.cuda.synchronize()
    k = [np.stack([kb for kb, _ in rows])[None].repeat(1, 0) for _ in range(B)]
    v = [np.stack([vb for _, vb in rows])[None].repeat(1, 0) for _ in range(B)]
    ref = oracle.decode(q.float().numpy(), k, v, [L] * B, scale, kv_scales=(1.0, 1.0))
    return out, ref


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fp8_every_code_decodes_exactly(dtype):
    """The kernel's E4M3 decoding, code by code, against the oracle's decoder
    (written from the format's definition and pinned to torch on all 256
    codes).  V: a one-token context returns its V row exactly (the softmax of
    one score is 1), so with v_scale 1 each output element must be the E4M3
    value of its V byte, bit for bit -- the 16-bit output holds every E4M3
    value exactly (as values: the sum 0 + 1 x (-0) is +0 for the code of -0,
    in the oracle too).  K: two tokens, K row 0 zero and V rows 1 and 0, query
    row (b, h) one-hot at dimension d = 16 b + h, scale 64: the output is the
    weight of token 0, 1 / (1 + e^(64 K1[d])), a steep function of that one
    K code (a subnormal read as zero moves it by 3 % or more)."""
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    D = 256
    gen = torch.Generator().manual_seed(7)
    q = torch.randn((1, 2, D), generator=gen).to(tdt)
    one = np.full(D, 0x38, dtype=np.uint8)      # E4M3 1.0
    out, ref = _one_block_fp8(1, 2, D, [(one, FINITE_CODES)], dtype, q, 0.1)
    expect = torch.from_numpy(oracle.e4m3_value(FINITE_CODES).astype(np.float32)).to(tdt)
    for h in range(2):  # value equality: bit equality but for the sign of zero (0 + 1 x -0 = +0)
        assert torch.equal(out[0, h].cpu().float(), expect.float())
    assert np.array_equal(ref[0, 0], expect.float().numpy())
    # K codes through the scores
    q = torch.zeros((16, 16, D), dtype=tdt)
    for b in range(16):
        for h in range(16):
            q[b, h, 16 * b + h] = 1.0
    zero = np.zeros(D, dtype=np.uint8)
    out, ref = _one_block_fp8(16, 16, D, [(zero, one), (FINITE_CODES, zero)], dtype, q, 64.0)
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    # every row's elements are the same weight; compare the weight per (b, h)
    w_got, w_ref = got[..., 0], ref[..., 0]
    err = np.abs(w_got - w_ref)
    assert np.all(err <= 1e-2 * np.abs(w_ref) + 1e-6), float(err.max())


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

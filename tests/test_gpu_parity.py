"""GPU parity of the HIP decode path against the CPU oracle, through the C ABI.

Tolerances are the ones the decode is held to: relative L-infinity against
the oracle's own output scale <= 1e-2 for bf16 KV and <= 2e-3 for fp16 KV
(the pages observe 2.12e-3..4.72e-3 for bf16: page "vLLM's custom ROCm
paged-attention kernel wins all sixty cells", abstract).  NaN-freedom is
required everywhere, and runs whose unwritten tails hold NaN or 1e4 must be
bit-identical to the clean-tail run (same page, section 5, Figure 4).
"""
import numpy as np
import pytest
import torch

import kvgen
import paged_kv_cache_decode_amd as pda
from kvgen import configs
from oracle import bookkeeping

from helpers import bits, check, reference, run, shape_of, to_device

pytestmark = pytest.mark.gpu

POISON = {"K": ("nan", "zero"), "V": ("zero", "nan"), "KV": ("nan", "nan"),
          "KV_1e4": ("1e4", "1e4")}


def plan_of(P, T, variant=pda.PDA_VARIANT_VALU, merge=pda.PDA_MERGE_KERNEL):
    return pda.PdaPlan(num_partitions=P, tokens_per_partition=T, variant=variant, merge=merge,
                       cu_count=0, workspace_bytes=0)


VARIANTS = {"valu": pda.PDA_VARIANT_VALU, "mfma": pda.PDA_VARIANT_MFMA}


def device_plan(case, variant=None, merge=None):
    """The device's own plan, optionally with the variant / merge overridden."""
    plan = pda.paged_decode_attn_plan(shape_of(case))
    if variant is not None:
        plan.variant = VARIANTS[variant]
    if merge is not None:
        plan.merge = merge
    return plan


# ---- config 1: tiny paged GQA decode ------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_cfg1_tiny(dtype):
    case = to_device(configs.cfg1(dtype))
    got = run(case)
    check(case, got)
    clean = to_device(kvgen.page(configs.cfg1(dtype), "zero", "zero"))
    assert np.array_equal(bits(got), bits(run(clean)))


# ---- config 2: the pages' shape sweep ------------------------------------
@pytest.mark.parametrize("hq", configs.CFG2_HQ)
@pytest.mark.parametrize("L", configs.CFG2_LENS)
def test_cfg2_sweep(hq, L):
    case = configs.cfg2(hq, L, device="cuda")
    check(case, run(case))


# ---- config 3: gemma-like layer, straddling lengths, NaN tails -----------
@pytest.mark.parametrize("variant", ["valu", "mfma"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("L", configs.CFG3_LENS)
def test_cfg3_b1_fault_matrix(dtype, L, variant):
    clean = configs.cfg3(1, L, dtype=dtype, device="cuda", tail_k="zero", tail_v="zero")
    plan = device_plan(clean, variant)
    ref_out = run(clean, plan=plan)
    check(clean, ref_out)
    for mode, (tk, tv) in POISON.items():
        poisoned = kvgen.page(clean, tk, tv)
        got = run(poisoned, plan=plan)
        assert np.array_equal(bits(got), bits(ref_out)), f"{mode} tail changed the output"


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("L", [4090, 16391, 32768])
def test_cfg3_b8(dtype, L):
    case = configs.cfg3(8, L, dtype=dtype, device="cuda")
    got = run(case)
    check(case, got, per_seq=True)
    clean = kvgen.page(case, "zero", "zero")
    assert np.array_equal(bits(got), bits(run(clean)))


# ---- config 4: 4 KV heads, batch 1, D 256, block size 784 ----------------
@pytest.mark.parametrize("L", configs.CFG4_LENS)
def test_cfg4_low_parallelism(L):
    case = configs.cfg4(L, device="cuda")
    got = run(case)
    check(case, got)
    plan = pda.paged_decode_attn_plan(shape_of(case))
    if L >= 4096:
        assert plan.num_partitions > 1  # split-KV is exercised
    clean = kvgen.page(case, "zero", "zero")
    assert np.array_equal(bits(got), bits(run(clean)))


# ---- config 5: batched mixed lengths ------------------------------------
@pytest.mark.parametrize("variant", [None, "valu"])
def test_cfg5_mixed_batch_full_size(variant):
    """All 64 sequences (1.2M tokens, NaN tails) scored against the oracle,
    each at the tolerance, and the poisoned run bit-identical to the same
    content with zero tails; under the device's plan (the matrix cores) and
    with the VALU kernel on the same partitions."""
    case = configs.cfg5(device="cuda")
    plan = None if variant is None else device_plan(case, variant=variant)
    got = run(case, plan)
    check(case, got, per_seq=True)
    clean = kvgen.page(case, "zero", "zero")
    assert np.array_equal(bits(got), bits(run(clean, plan)))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_cfg5_mixed_batch_short(dtype):
    case = configs.cfg5(device="cuda", dtype=dtype, lo=1, hi=3000, cell=1)
    got = run(case)
    check(case, got, per_seq=True)
    clean = kvgen.page(case, "zero", "zero")
    assert np.array_equal(bits(got), bits(run(clean)))


# ---- the MFMA variant over the whole shape space ------------------------
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 6, 8, 11, 16])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_mfma_variant(D, G, dtype):
    rng = np.random.default_rng(D * 77 + G + (500 if dtype == "fp16" else 0))
    B = 3
    Hkv = int(rng.integers(1, 3))
    bs = int(rng.choice([1, 5, 16, 48, 784]))
    lens = [int(x) for x in rng.integers(1, 1500, size=B)]
    case = to_device(kvgen.make_case(B, G * Hkv, Hkv, D, bs, lens, dtype=dtype,
                                     seed=int(rng.integers(1 << 30)), tail_k="nan", tail_v="nan"))
    ref = reference(case)
    for plan in (device_plan(case, "mfma"),
                 plan_of(5, 320, variant=pda.PDA_VARIANT_MFMA),
                 plan_of(5, 320, variant=pda.PDA_VARIANT_MFMA, merge=pda.PDA_MERGE_FUSED),
                 plan_of(1, 1536, variant=pda.PDA_VARIANT_MFMA)):
        check(case, run(case, plan=plan), ref, per_seq=True)


@pytest.mark.parametrize("mk", ["cfg4-32K", "cfg2-32K", "cfg5"])
def test_mfma_variant_full_size(mk):
    case = {"cfg4-32K": lambda: configs.cfg4(32768, device="cuda"),
            "cfg2-32K": lambda: configs.cfg2(32, 32768, device="cuda"),
            "cfg5": lambda: configs.cfg5(device="cuda")}[mk]()
    got = run(case, plan=device_plan(case, "mfma"))
    check(case, got, per_seq=True)


def test_mfma_matches_valu_closely():
    """Two implementations of the same sums: both within tolerance of the
    oracle and close to each other (fp32 accumulation order, and the matrix
    cores' weights rounded to bf16: each weight moves by at most 2^-9 of
    itself, and the output stays a convex combination of the same rows)."""
    case = configs.cfg4(24576, device="cuda")
    a = run(case, plan=device_plan(case, "valu")).float()
    b = run(case, plan=device_plan(case, "mfma")).float()
    assert float((a - b).abs().max()) <= 2 * 2.0 ** -8 * float(a.abs().max())


# ---- the whole space of shapes at small sizes -------------------------
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_group_and_head_sizes(D, G, dtype):
    rng = np.random.default_rng(D * 31 + G + (1000 if dtype == "fp16" else 0))
    B = 3
    Hkv = int(rng.integers(1, 4))
    bs = int(rng.choice([1, 5, 16, 48, 784]))
    lens = [int(x) for x in rng.integers(1, 1500, size=B)]
    case = to_device(kvgen.make_case(B, G * Hkv, Hkv, D, bs, lens, dtype=dtype,
                                     seed=int(rng.integers(1 << 30)), tail_k="nan", tail_v="nan"))
    got = run(case)
    check(case, got, per_seq=True)
    P, T = 5, 320  # forced multi-partition plans (some partitions empty)
    for merge in (pda.PDA_MERGE_FUSED, pda.PDA_MERGE_KERNEL):
        got2 = run(case, plan=plan_of(P, T, merge=merge))
        check(case, got2, per_seq=True)


@pytest.mark.parametrize("mk", ["cfg4", "cfg5short"])
def test_fused_and_kernel_merge_reuse_workspace(mk):
    """Both merge paths agree with the oracle; the fused path's arrival
    counters return to zero after every call, so one workspace serves a
    sequence of calls (different plans included) with identical results."""
    case = (configs.cfg4(16384, device="cuda") if mk == "cfg4"
            else configs.cfg5(device="cuda", lo=1, hi=5000, cell=2))
    shape = shape_of(case)
    dplan = pda.paged_decode_attn_plan(shape)
    assert dplan.num_partitions > 1
    # the device plan's partitions and variant under each merge mode,
    # whichever mode the plan picked
    kplan = plan_of(dplan.num_partitions, dplan.tokens_per_partition, dplan.variant,
                    merge=pda.PDA_MERGE_KERNEL)
    planned = plan_of(dplan.num_partitions, dplan.tokens_per_partition, dplan.variant,
                      merge=pda.PDA_MERGE_FUSED)
    ws = torch.empty(pda.pda_workspace_bytes(shape, planned), dtype=torch.uint8, device="cuda")
    pda.paged_decode_attn_workspace_init(ws)
    ref = reference(case)
    first = None
    for it in range(4):
        plan = planned if it % 2 == 0 else kplan
        out = pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                    case.seq_lens_t, case.scale, workspace=ws,
                                    max_seq_len=case.max_seq_len, plan=plan)
        torch.cuda.synchronize()
        check(case, out, ref, per_seq=True)
        if plan is planned:
            if first is None:
                first = bits(out)
            else:
                assert np.array_equal(first, bits(out))
    # the counters (the fixed block at the start of the workspace) are back at zero
    ctr = ws[:16384 * 4].view(torch.int32)
    assert int(ctr.abs().sum().item()) == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fused_merge_across_xcds_repeated(dtype):
    """One KV head at batch 1 under a forced 16-partition fused plan: the
    dispatcher sends workgroup L of the (Hkv, B, P) grid to XCD L mod 8, so
    the 16 partitions of the unit run on all eight XCDs and the last one to
    arrive reads partials written on the seven others.  40 calls in a row on
    one workspace: every output bit-identical to the first and within
    tolerance of the oracle, the arrival counter back at zero."""
    case = to_device(kvgen.make_case(1, 8, 1, 128, 16, [16000], dtype=dtype, seed=404,
                                     tail_k="nan", tail_v="nan"))
    plan = plan_of(16, 1024, variant=pda.PDA_VARIANT_MFMA, merge=pda.PDA_MERGE_FUSED)
    shape = shape_of(case)
    ws = torch.zeros(pda.pda_workspace_bytes(shape, plan), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(40):
        outs.append(pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                          case.seq_lens_t, case.scale, workspace=ws,
                                          max_seq_len=case.max_seq_len, plan=plan))
    torch.cuda.synchronize()
    check(case, outs[0])
    first = bits(outs[0])
    for o in outs[1:]:
        assert np.array_equal(first, bits(o))
    assert int(ws[:16384 * 4].view(torch.int32).abs().sum().item()) == 0


def test_workspace_check_reports_stale_counters():
    """The arrival counters are all zero after fused calls; a counter left
    non-zero before a fused call (as in a workspace never zeroed) is reported
    by paged_decode_attn_workspace_check, and zeroing the workspace clears
    it.  (The planted value only keeps that unit's last workgroup from
    merging; every kernel still ends normally.)"""
    case = configs.cfg2(32, 2048, device="cuda")
    shape = shape_of(case)
    plan = pda.paged_decode_attn_plan(shape)
    plan.merge = pda.PDA_MERGE_FUSED
    assert plan.num_partitions > 1
    ws = torch.zeros(pda.pda_workspace_bytes(shape, plan), dtype=torch.uint8, device="cuda")

    def call():
        return pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                     case.seq_lens_t, case.scale, workspace=ws,
                                     max_seq_len=case.max_seq_len, plan=plan)
    check(case, call())
    assert pda.paged_decode_attn_workspace_check(ws) == 0
    ws[:4].view(torch.int32)[0] = plan.num_partitions + 3  # unit (0, 0)
    call()
    assert pda.paged_decode_attn_workspace_check(ws) == 1
    pda.paged_decode_attn_workspace_init(ws)
    assert pda.paged_decode_attn_workspace_check(ws) == 0
    check(case, call())
    assert pda.paged_decode_attn_workspace_check(ws) == 0


def test_one_workspace_serves_a_sequence_of_shapes():
    """Zeroed once, one workspace serves calls of different shapes under the
    device plan, fused merge and merge kernel alike: the arrival counters sit
    in a fixed block at its start, where no shape's partials land, and each
    fused call leaves them zero.  Every call matches the oracle and equals
    the same call on a fresh workspace bit for bit."""
    cases = [configs.cfg2(32, 1024, device="cuda"),         # fused, 8 partitions
             configs.cfg3(8, 1024, device="cuda"),          # fused, 128 units
             configs.cfg2(32, 4096, device="cuda"),         # merge kernel, 32 partitions
             configs.cfg3(1, 2048, device="cuda", cell=3),  # fused, 16 partitions
             configs.cfg2(32, 1024, device="cuda")]         # the first shape again
    need = max(pda.paged_decode_attn_workspace_size(shape_of(c)) for c in cases)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    pda.paged_decode_attn_workspace_init(ws)
    merges = set()
    for case in cases:
        merges.add(pda.paged_decode_attn_plan(shape_of(case)).merge)
        out = pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                    case.seq_lens_t, case.scale, workspace=ws,
                                    max_seq_len=case.max_seq_len)
        fresh = pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                      case.seq_lens_t, case.scale, max_seq_len=case.max_seq_len)
        torch.cuda.synchronize()
        check(case, out, per_seq=True)
        assert np.array_equal(bits(out), bits(fresh))
    assert merges == {pda.PDA_MERGE_FUSED, pda.PDA_MERGE_KERNEL}
    assert int(ws[:16384 * 4].view(torch.int32).abs().sum().item()) == 0


def test_edge_lengths():
    lens = [0, 1, 2, 15, 16, 17, 63, 64, 65, 1000]
    case = to_device(kvgen.make_case(len(lens), 6, 2, 64, 16, lens, seed=77, tail_k="nan",
                                     tail_v="nan", max_blocks_per_seq=70))
    for plan in (None, plan_of(1, 1024), plan_of(16, 64, merge=pda.PDA_MERGE_FUSED),
                 plan_of(16, 64, merge=pda.PDA_MERGE_KERNEL)):
        got = run(case, plan=plan)
        g = got.float().cpu().numpy()
        assert np.all(g[0] == 0.0)                                  # L == 0 -> zeros
        for h in range(6):                                          # L == 1 -> the V row
            assert np.array_equal(bits(got[1, h]), bits(case.v[1][h // 3, 0]))
        check(case, got, per_seq=False)


@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_units_at_the_counter_block_limit(variant):
    """B * Hkv = PDA_FUSED_MAX_UNITS (16384) under the fused merge: every
    arrival counter is in use, the last one included, over many rounds of
    workgroups; parity on every sequence, and (in `run`) the counters back at
    zero and the guard bytes intact."""
    rng = np.random.default_rng(16384)
    lens = [int(x) for x in rng.integers(17, 129, size=2048)]
    case = to_device(kvgen.make_case(2048, 8, 8, 64, 16, lens, seed=16384, tail_k="nan",
                                     tail_v="nan"))
    assert case.B * case.Hkv == 16384
    got = run(case, plan=plan_of(2, 64, variant=VARIANTS[variant], merge=pda.PDA_MERGE_FUSED))
    check(case, got, per_seq=True)


def test_block_larger_than_a_partition():
    """Blocks of 4096 tokens, far larger than a partition: each partition
    lies in one or two blocks.  Parity under the device plan and two forced
    plans (the bookkeeping trace of the same shape is one of TRACE_CASES)."""
    lens = [4096, 4097, 9000, 1]
    case = to_device(kvgen.make_case(4, 16, 4, 128, 4096, lens, seed=4096, tail_k="nan",
                                     tail_v="nan"))
    for plan in (None, plan_of(3, 4096, variant=pda.PDA_VARIANT_MFMA),
                 plan_of(16, 576, variant=pda.PDA_VARIANT_MFMA, merge=pda.PDA_MERGE_FUSED)):
        check(case, run(case, plan=plan), per_seq=True)


def test_binding_refuses_buffers_off_the_device():
    """A workspace or a table on the host is refused before the library is
    called: a host address handed to a kernel would be a GPU memory fault.
    The device buffers of the same call then still decode it."""
    case = to_device(configs.cfg1("bf16"))
    plan = pda.paged_decode_attn_plan(shape_of(case))
    plan.num_partitions, plan.tokens_per_partition = 2, 64  # P > 1: a workspace is used
    plan.workspace_bytes = pda.pda_workspace_bytes(shape_of(case), plan)
    args = (case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens_t, case.scale)
    with pytest.raises(ValueError, match="workspace"):
        pda.paged_decode_attn(*args, plan=plan,
                              workspace=torch.zeros(plan.workspace_bytes, dtype=torch.uint8))
    with pytest.raises(ValueError, match="device"):
        pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table.cpu(),
                              case.seq_lens_t, case.scale)
    ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=case.q.device)
    got = pda.paged_decode_attn(*args, plan=plan, workspace=ws)
    torch.cuda.synchronize()
    check(case, got)


def test_empty_batch_rows_only():
    case = to_device(kvgen.make_case(2, 8, 4, 128, 16, [0, 0], seed=5, max_blocks_per_seq=2,
                                     max_seq_len=32))
    for plan in (None, plan_of(1, 64), plan_of(3, 64),
                 plan_of(3, 64, merge=pda.PDA_MERGE_FUSED)):
        got = run(case, plan=plan)
        assert torch.all(got.float() == 0)


# ---- invariants --------------------------------------------------------
@pytest.mark.parametrize("variant", ["valu", "mfma"])
@pytest.mark.parametrize("bs", [16, 784, 5])
def test_block_permutation_bit_identical(bs, variant):
    case = to_device(kvgen.make_case(4, 24, 4, 256 if bs == 784 else 128, bs,
                                     [3000, 1, 2049, 800], seed=91, extra_blocks=7,
                                     tail_k="nan", tail_v="nan"))
    a = run(case, plan=device_plan(case, variant))
    perm = kvgen.repermute(case, seed=92)
    b = run(perm, plan=device_plan(perm, variant))
    assert np.array_equal(bits(a), bits(b))


@pytest.mark.parametrize("variant", ["valu", "mfma"])
def test_run_to_run_deterministic(variant):
    case = configs.cfg4(24576, device="cuda")
    plan = device_plan(case, variant)
    a = bits(run(case, plan=plan))
    for _ in range(3):
        assert np.array_equal(a, bits(run(case, plan=plan)))


@pytest.mark.parametrize("mk", ["cfg2", "cfg4"])
def test_forced_single_partition_vs_planned(mk):
    case = configs.cfg2(32, 8192, device="cuda") if mk == "cfg2" else configs.cfg4(8192, device="cuda")
    planned = pda.paged_decode_attn_plan(shape_of(case))
    assert planned.num_partitions > 1
    ref = reference(case)
    check(case, run(case), ref)
    T = -(-case.max_seq_len // 64) * 64
    check(case, run(case, plan=plan_of(1, T)), ref)
    fplan = plan_of(planned.num_partitions, planned.tokens_per_partition,
                    merge=pda.PDA_MERGE_FUSED)
    check(case, run(case, plan=fplan), ref)


# ---- bookkeeping: bit-exact against the oracle's recomputation ----------
TRACE_CASES = [
    # D, bs, G, lens, forced (P, T) or None for the device plan
    (128, 16, 2, [17, 40], None),
    (128, 16, 4, [4090, 1, 333], (7, 640)),
    (256, 784, 6, [32768], None),
    (256, 784, 6, [500, 784, 785, 1568], (4, 448)),
    (64, 1, 1, [300, 77], (5, 64)),
    (64, 5, 3, [1234, 0, 99], (3, 512)),
    (128, 48, 8, [5000, 4999], None),
    (256, 8, 2, [777, 8], (2, 512)),
    (128, 4096, 4, [4096, 4097, 9000, 1], (16, 576)),
]


@pytest.mark.parametrize("rows", [0, 1])
@pytest.mark.parametrize("variant", ["valu", "mfma"])
@pytest.mark.parametrize("D,bs,G,lens,forced", TRACE_CASES)
def test_bookkeeping_trace_bit_exact(D, bs, G, lens, forced, variant, rows):
    Hkv = 2
    case = to_device(kvgen.make_case(len(lens), G * Hkv, Hkv, D, bs, lens, seed=101,
                                     extra_blocks=3))
    shape = shape_of(case)
    plan = pda.paged_decode_attn_plan(shape) if forced is None else plan_of(*forced)
    plan.variant = VARIANTS[variant]
    slot, part, ranges = pda.paged_decode_attn_trace(shape, plan, case.block_table,
                                                     case.seq_lens_t, rows=rows)
    torch.cuda.synchronize()
    e_slot, e_part, e_ranges, valid = bookkeeping.expected_trace(
        case.block_table.cpu().numpy(), case.seq_lens, Hkv, bs, case.max_seq_len,
        plan.num_partitions, plan.tokens_per_partition)
    slot, part, ranges = slot.cpu().numpy(), part.cpu().numpy(), ranges.cpu().numpy()
    Lm = case.max_seq_len
    assert np.array_equal(slot[..., :Lm][valid], e_slot[valid])
    assert np.array_equal(part[..., :Lm][valid], e_part[valid])
    assert np.all(slot[..., :Lm][~valid] == -1) and np.all(part[..., :Lm][~valid] == -1)
    assert np.array_equal(ranges, e_ranges)


@pytest.mark.parametrize("rows", [0, 1])
@pytest.mark.parametrize("D,bs,G,lens,forced", TRACE_CASES)
def test_bookkeeping_trace_fp8_kv(D, bs, G, lens, forced, rows):
    """The matrix-core kernel's K and V rows for fp8 KV, whose whole-row K
    loads have their own lane map (a row is D bytes, not 2D)."""
    Hkv = 2
    case = to_device(kvgen.make_case(len(lens), G * Hkv, Hkv, D, bs, lens, seed=102,
                                     extra_blocks=3, kv_dtype="fp8"))
    shape = shape_of(case)
    plan = pda.paged_decode_attn_plan(shape) if forced is None else plan_of(*forced)
    plan.variant = pda.PDA_VARIANT_MFMA
    slot, part, ranges = pda.paged_decode_attn_trace(shape, plan, case.block_table,
                                                     case.seq_lens_t, rows=rows)
    torch.cuda.synchronize()
    e_slot, e_part, e_ranges, valid = bookkeeping.expected_trace(
        case.block_table.cpu().numpy(), case.seq_lens, Hkv, bs, case.max_seq_len,
        plan.num_partitions, plan.tokens_per_partition)
    slot, part, ranges = slot.cpu().numpy(), part.cpu().numpy(), ranges.cpu().numpy()
    Lm = case.max_seq_len
    assert np.array_equal(slot[..., :Lm][valid], e_slot[valid])
    assert np.array_equal(part[..., :Lm][valid], e_part[valid])
    assert np.all(slot[..., :Lm][~valid] == -1) and np.all(part[..., :Lm][~valid] == -1)
    assert np.array_equal(ranges, e_ranges)


@pytest.mark.parametrize("variant,rows", [("valu", 0), ("mfma", 0), ("mfma", 1)])
def test_bookkeeping_trace_cfg5_full_size(variant, rows):
    case = configs.cfg5(device="cuda")
    shape = shape_of(case)
    plan = pda.paged_decode_attn_plan(shape)
    plan.variant = VARIANTS[variant]
    slot, part, ranges = pda.paged_decode_attn_trace(shape, plan, case.block_table,
                                                     case.seq_lens_t, rows=rows)
    torch.cuda.synchronize()
    e_slot, e_part, e_ranges, valid = bookkeeping.expected_trace(
        case.block_table.cpu().numpy(), case.seq_lens, case.Hkv, case.bs, case.max_seq_len,
        plan.num_partitions, plan.tokens_per_partition)
    slot, part = slot.cpu().numpy(), part.cpu().numpy()
    assert np.array_equal(slot[valid], e_slot[valid])
    assert np.array_equal(part[valid], e_part[valid])
    assert np.all(slot[~valid] == -1)
    assert np.array_equal(ranges.cpu().numpy(), e_ranges)


# ---- one GPU's share of the heads under two-way tensor parallelism -------
@pytest.mark.parametrize("variant", ["valu", "mfma"])
@pytest.mark.parametrize("L", [500, 4096, 16391, 32768])
def test_tp_share_cfg4_12_2(L, variant):
    case = configs.cfg4_tp2(L, device="cuda")
    check(case, run(case, plan=device_plan(case, variant)), per_seq=True)


@pytest.mark.parametrize("variant", ["valu", "mfma"])
@pytest.mark.parametrize("B,L", [(1, 1024), (1, 16391), (1, 32768), (8, 4090), (8, 32768)])
def test_tp_share_cfg3_16_8(B, L, variant):
    case = configs.cfg3_tp2(B, L, device="cuda")
    got = run(case, plan=device_plan(case, variant))
    check(case, got, per_seq=True)

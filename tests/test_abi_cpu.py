"""CPU-only checks of the C-ABI library: it loads, exports every symbol the
header declares, its plan equals the independently re-derived plan bit for
bit, and invalid arguments are rejected by host validation before anything
is launched (no GPU is touched)."""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_cache_decode_amd as pda
from oracle import plan as oplan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pda.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = pda.load_library()
    names = header_functions()
    assert "paged_decode_attn" in names and "paged_decode_attn_workspace_size" in names
    for n in names:
        assert hasattr(lib, n), n
    assert "gfx950" in pda.pda_build_id()


def test_status_strings():
    for s in (pda.PDA_OK, pda.PDA_ERR_INVALID, pda.PDA_ERR_UNSUPPORTED, pda.PDA_ERR_WORKSPACE,
              pda.PDA_ERR_LAUNCH, pda.PDA_ERR_DEVICE):
        assert pda.pda_status_string(s) != "unknown status"


@pytest.mark.parametrize("D", [64, 128, 256])
def test_plan_matches_oracle_plan(D):
    rng = np.random.default_rng(1000 + D)
    for _ in range(3000):
        B = int(rng.integers(1, 200))
        Hkv = int(rng.integers(1, 17))
        G = int(rng.integers(1, 17))
        bs = int(rng.choice([1, 3, 16, 784]))
        L = int(rng.integers(0, 300000))
        mbs = max(1, -(-L // bs))
        cu = int(rng.choice([1, 7, 80, 256, 304]))
        W = int(rng.choice([0, 0, 1, 31, 1024]))
        n = int(rng.choice([1, 1, 2, 3, 8]))
        if n * G > 32:
            n = 1
        f8 = bool(rng.integers(0, 4) == 0)
        shape = pda.make_shape(B, Hkv * G, Hkv, D, bs, 10, mbs, L, "bf16", sliding_window=W,
                               q_len=n, kv_dtype="fp8" if f8 else "same", k_scale=0.5,
                               v_scale=0.25)
        got = pda.pda_plan_for_cus(shape, cu)
        P, T, var = oplan.partition(B, Hkv, G, D, L, cu, window=W, q_len=n, kv_fp8=f8)
        assert (got.num_partitions, got.tokens_per_partition, got.variant) == (P, T, var)
        assert got.workspace_bytes == oplan.workspace_bytes(B, Hkv * G, D, P, Hkv, q_len=n)
        assert got.merge == oplan.merge(P, n * G, D, B * Hkv)
        assert got.cu_count == cu


def test_plan_golden_through_library():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "plan_cu256.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        shape = pda.make_shape(c["B"], c["Hkv"] * c["G"], c["Hkv"], c["D"], 16, 1,
                               max(1, -(-c["Lmax"] // 16)), c["Lmax"],
                               sliding_window=c.get("W", 0), q_len=c.get("q_len", 1))
        got = pda.pda_plan_for_cus(shape, g["cu_count"])
        assert (got.num_partitions, got.tokens_per_partition, got.variant, got.merge) == \
            (c["P"], c["T_p"], c["variant"], c["merge"]), c["name"]


BAD_SHAPES = [
    (dict(num_seqs=0), pda.PDA_ERR_INVALID),
    (dict(num_q_heads=12, num_kv_heads=8), pda.PDA_ERR_INVALID),
    (dict(head_size=96), pda.PDA_ERR_UNSUPPORTED),
    (dict(head_size=512), pda.PDA_ERR_UNSUPPORTED),
    (dict(dtype=2), pda.PDA_ERR_UNSUPPORTED),
    (dict(num_q_heads=17 * 8), pda.PDA_ERR_UNSUPPORTED),
    (dict(block_size=0), pda.PDA_ERR_INVALID),
    (dict(max_seq_len=-1), pda.PDA_ERR_INVALID),
    (dict(max_seq_len=16 * 4 + 1), pda.PDA_ERR_INVALID),  # > MBS * bs
    (dict(num_blocks=0), pda.PDA_ERR_INVALID),
    (dict(sliding_window=-1), pda.PDA_ERR_INVALID),
    (dict(q_len=-1), pda.PDA_ERR_INVALID),
    (dict(q_len=9), pda.PDA_ERR_UNSUPPORTED),                       # 9 x 4 rows > 32
    (dict(q_len=33, num_q_heads=8), pda.PDA_ERR_UNSUPPORTED),      # 33 rows
    (dict(kv_dtype=2), pda.PDA_ERR_UNSUPPORTED),
    # block_size * head_size must fit the kernels' 32-bit head stride
    (dict(block_size=(1 << 23) + 1, head_size=256, max_blocks_per_seq=1, max_seq_len=64),
     pda.PDA_ERR_UNSUPPORTED),
    (dict(kv_dtype=1, k_scale=0.0, v_scale=1.0), pda.PDA_ERR_INVALID),
    (dict(kv_dtype=1, k_scale=1.0, v_scale=float("inf")), pda.PDA_ERR_INVALID),
    (dict(kv_dtype=1, k_scale=float("nan"), v_scale=1.0), pda.PDA_ERR_INVALID),
]


def _shape(**kw):
    base = dict(num_seqs=2, num_q_heads=32, num_kv_heads=8, head_size=128, block_size=16,
                num_blocks=16, max_blocks_per_seq=4, max_seq_len=64, dtype=0, q_len=1,
                kv_dtype=0, k_scale=1.0, v_scale=1.0)
    base.update(kw)
    return pda.PdaShape(**base)


@pytest.mark.parametrize("kw,status", BAD_SHAPES)
def test_invalid_shapes_rejected(kw, status):
    assert pda.pda_check_shape(_shape(**kw)) == status
    lib = pda.load_library()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    rc = lib.paged_decode_attn(ctypes.byref(_shape(**kw)), fake, fake, fake, fake, fake, 1.0,
                               fake, None, 0, None)
    assert rc == status


def test_null_pointers_rejected_before_launch():
    lib = pda.load_library()
    fake = ctypes.c_void_p(0x1000)
    s = _shape()
    args = [fake] * 5
    for i in range(6):
        ptrs = [fake] * 6
        ptrs[i] = None
        rc = lib.paged_decode_attn(ctypes.byref(s), ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4],
                                   1.0, ptrs[5], None, 0, None)
        assert rc == pda.PDA_ERR_INVALID
    del args


def test_small_workspace_rejected_before_launch():
    lib = pda.load_library()
    fake = ctypes.c_void_p(0x1000)
    s = _shape(max_seq_len=64, max_blocks_per_seq=4)
    plan = pda.PdaPlan(num_partitions=2, tokens_per_partition=64, variant=pda.PDA_VARIANT_VALU,
                       merge=pda.PDA_MERGE_FUSED, cu_count=1, workspace_bytes=0)
    need = pda.pda_workspace_bytes(s, plan)
    assert need > 0
    for ws, nbytes in ((None, 0), (fake, need - 1)):
        rc = lib.paged_decode_attn_with_plan(ctypes.byref(s), ctypes.byref(plan), fake, fake, fake,
                                             fake, fake, 1.0, fake, ws, nbytes, None)
        assert rc == pda.PDA_ERR_WORKSPACE


@pytest.mark.parametrize("P,T,variant,merge,status", [
    (0, 64, 1, 0, pda.PDA_ERR_INVALID),          # no partition
    (1, 32, 1, 0, pda.PDA_ERR_INVALID),          # not a multiple of 64
    (1, 64, 1, 0, pda.PDA_ERR_INVALID),          # does not cover max_seq_len = 100
    (2, 64, 7, 0, pda.PDA_ERR_INVALID),          # unknown variant
    (2, 64, 1, 5, pda.PDA_ERR_INVALID),          # unknown merge mode
])
def test_bad_plans_rejected(P, T, variant, merge, status):
    lib = pda.load_library()
    fake = ctypes.c_void_p(0x1000)
    s = _shape(max_seq_len=100, max_blocks_per_seq=7)
    plan = pda.PdaPlan(num_partitions=P, tokens_per_partition=T, variant=variant, merge=merge,
                       cu_count=1, workspace_bytes=0)
    rc = lib.paged_decode_attn_with_plan(ctypes.byref(s), ctypes.byref(plan), fake, fake, fake,
                                         fake, fake, 1.0, fake, fake, 1 << 30, None)
    assert rc == status


def test_fastdiv_method_is_exact():
    """The multiply-high division the kernels use for token -> (block, slot),
    checked as arithmetic over block sizes 1..2048 and 784 on dividends
    including the extremes below 2^31.  (The GPU trace test checks the
    compiled kernels against the oracle's plain division.)"""
    rng = np.random.default_rng(7)
    ns = np.concatenate([np.arange(0, 5000), rng.integers(0, 2 ** 31, 20000),
                         np.array([2 ** 31 - 1, 2 ** 31 - 2])]).astype(np.uint64)
    for d in list(range(1, 2049)) + [784, 65535, 1 << 20, 12345677]:
        l = 0
        while (1 << l) < d:
            l += 1
        mul = ((((1 << l) - d) << 32) // d + 1) & 0xFFFFFFFF
        hi = (ns * np.uint64(mul)) >> np.uint64(32)
        q = (hi + ns) >> np.uint64(l)
        assert np.array_equal(q, ns // np.uint64(d)), d


def test_fp8_kv_plans_matrix_core_and_rejects_valu():
    shape = pda.make_shape(64, 32, 8, 128, 16, 100, 2048, 32768, "bf16", kv_dtype="fp8",
                           k_scale=0.01, v_scale=0.02)
    plan = pda.pda_plan_for_cus(shape, 256)
    assert plan.variant == pda.PDA_VARIANT_MFMA
    # K and V bytes per token halve: the 1 MiB partitions hold 4096 tokens
    assert plan.tokens_per_partition == 4096
    plan.variant = pda.PDA_VARIANT_VALU
    lib = pda.load_library()
    rc = lib.paged_decode_attn_with_plan(ctypes.byref(shape), ctypes.byref(plan), 1, 1, 1, 1, 1,
                                         1.0, 1, 1, 1 << 30, None)
    assert rc == pda.PDA_ERR_UNSUPPORTED


def test_q_len_zero_is_one_row():
    a = pda.pda_plan_for_cus(pda.make_shape(3, 32, 8, 128, 16, 10, 64, 1000, q_len=0), 256)
    b = pda.pda_plan_for_cus(pda.make_shape(3, 32, 8, 128, 16, 10, 64, 1000, q_len=1), 256)
    assert a.as_dict() == b.as_dict()


def test_plan_caps_partitions_at_the_grid_limit():
    """The partition index is a grid dimension: at most 65535 partitions,
    the partition size raised to keep within it."""
    L = 1 << 30
    shape = pda.make_shape(1, 8, 1, 256, 16, 1 << 26, L // 16, L)
    got = pda.pda_plan_for_cus(shape, 256)
    P, T, var = oplan.partition(1, 1, 8, 256, L, 256)
    assert (got.num_partitions, got.tokens_per_partition, got.variant) == (P, T, var)
    assert P <= 65535 and P * T >= L and T % 64 == 0
    bad = pda.PdaPlan(num_partitions=65536, tokens_per_partition=16384, variant=pda.PDA_VARIANT_MFMA,
                      merge=pda.PDA_MERGE_KERNEL, cu_count=0, workspace_bytes=0)
    lib = pda.load_library()
    rc = lib.paged_decode_attn_with_plan(ctypes.byref(shape), ctypes.byref(bad), 1, 1, 1, 1, 1,
                                         1.0, 1, 1, 1 << 40, None)
    assert rc == pda.PDA_ERR_UNSUPPORTED


def test_forced_fused_merge_beyond_the_counter_block_is_refused():
    """A fused merge counts arrivals in the workspace's fixed block of 16384
    counters: a forced fused plan for more units is refused before launch."""
    lib = pda.load_library()
    shape = _shape(num_seqs=2049, num_kv_heads=8, num_q_heads=32, max_blocks_per_seq=4,
                   max_seq_len=64)  # 16392 units
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    for merge, status in ((pda.PDA_MERGE_FUSED, pda.PDA_ERR_UNSUPPORTED),):
        plan = pda.PdaPlan(num_partitions=2, tokens_per_partition=64, variant=pda.PDA_VARIANT_MFMA,
                           merge=merge, cu_count=0, workspace_bytes=0)
        rc = lib.paged_decode_attn_with_plan(ctypes.byref(shape), ctypes.byref(plan), fake, fake,
                                             fake, fake, fake, 1.0, fake, fake, 1 << 40, None)
        assert rc == status
    # the device-independent plan never picks it there
    got = pda.pda_plan_for_cus(shape, 256)
    assert got.num_partitions == 1 or got.merge == pda.PDA_MERGE_KERNEL

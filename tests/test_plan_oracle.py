"""Pins of the bookkeeping oracle: the partition plan against hand-derived
values and its invariants, and the expected trace against a brute-force loop
over tokens.  CPU only."""
import json
import os

import numpy as np
import pytest

import kvgen
from oracle import bookkeeping, plan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_cu256.json")


def test_plan_hand_derived_values():
    with open(GOLDEN) as f:
        g = json.load(f)
    for c in g["cases"]:
        P, T, var = plan.partition(c["B"], c["Hkv"], c["G"], c["D"], c["Lmax"], g["cu_count"],
                                   window=c.get("W", 0), q_len=c.get("q_len", 1))
        assert (P, T, var) == (c["P"], c["T_p"], c["variant"]), c["name"]
        R = c["G"] * c.get("q_len", 1)
        assert plan.merge(P, R, c["D"], c["B"] * c["Hkv"]) == c["merge"], c["name"]


@pytest.mark.parametrize("D", [64, 128, 256])
def test_plan_invariants(D):
    rng = np.random.default_rng(D)
    t_min, t_many, t_one = plan.token_bounds(D)
    for _ in range(2000):
        B = int(rng.integers(1, 129))
        Hkv = int(rng.integers(1, 33))
        G = int(rng.integers(1, 17))
        L = int(rng.integers(0, 200000))
        cu = int(rng.choice([1, 80, 104, 256, 304]))
        W = int(rng.choice([0, 0, 1, 17, 1024, 4096]))
        n = int(rng.choice([1, 1, 2, 4, 8]))
        P, T, var = plan.partition(B, Hkv, G, D, L, cu, window=W, q_len=n)
        S = plan.span(L, W, n)
        assert S <= L and (W == 0 or S <= W + n - 1 + 15)
        assert T % plan.TP_ALIGN == 0 and t_min <= T <= t_one
        assert P >= 1 and P * T >= S
        L = S
        if L > 0:
            assert (P - 1) * T < L          # no partition is empty at the span
            # either one round of one workgroup per CU covers the job, or the
            # partitions are T_many
            assert P * B * Hkv <= cu + B * Hkv or T == t_many
        else:
            assert P == 1
        assert var == plan.MFMA if n * G > 8 else var in (plan.VALU, plan.MFMA)
        m = plan.merge(P, n * G, D, B * Hkv)
        assert m == plan.MERGE_KERNEL if P == 1 or P > 16 else m in (plan.MERGE_FUSED,
                                                                       plan.MERGE_KERNEL)
        if m == plan.MERGE_FUSED:
            assert P * n * G * D * 4 <= 32 * 1024


def test_workspace_bytes():
    counters = 16384 * 4  # the fixed block of arrival counters, first
    assert plan.workspace_bytes(1, 32, 128, 1) == 0
    assert plan.workspace_bytes(1, 24, 256, 128, 4) == \
        counters + 24 * 128 * 256 * 4 + 24 * 128 * 2 * 4
    # q_len rows per sequence: q_len times the partial rows
    assert plan.workspace_bytes(2, 8, 64, 3, 2, q_len=4) == \
        counters + 2 * 4 * 8 * 3 * 64 * 4 + 2 * 4 * 8 * 3 * 2 * 4


def test_fused_merge_needs_the_units_to_fit_the_counter_block():
    # 16 partitions of 2 rows at D 128: 16 KiB of partials, fused up to 16384 units
    assert plan.merge(16, 2, 128, 16384) == plan.MERGE_FUSED
    assert plan.merge(16, 2, 128, 16385) == plan.MERGE_KERNEL


def test_expected_trace_matches_token_loop():
    case = kvgen.make_case(3, 8, 2, 64, 5, [0, 23, 61], seed=43, extra_blocks=2)
    P, T = 2, 64  # partitions of 64 tokens, 2 of them cover Lmax=61
    slot, part, ranges, valid = bookkeeping.expected_trace(
        case.block_table.numpy(), case.seq_lens, 2, case.bs, 64, P, T)
    table = case.block_table.numpy()
    for b in range(3):
        L = case.seq_lens[b]
        for g in range(2):
            for t in range(64):
                assert valid[b, g, t] == (t < L)
                if t < L:
                    assert slot[b, g, t] == table[b][t // 5] * 5 + t % 5
                    assert part[b, g, t] == t // T
            for p in range(P):
                t0, t1 = ranges[b, g, p]
                assert t0 == p * T and t1 == min(p * T + T, L)


def test_expected_trace_with_window_matches_token_loop():
    W = 21
    case = kvgen.make_case(3, 8, 2, 64, 5, [0, 23, 61], seed=44, extra_blocks=2, sliding_window=W)
    P, T = 1, 64   # span min(61, 36) = 36 tokens: one 64-token partition
    slot, part, ranges, valid = bookkeeping.expected_trace(
        case.block_table.numpy(), case.seq_lens, 2, case.bs, 64, P, T, window=W)
    table = case.block_table.numpy()
    for b in range(3):
        L = case.seq_lens[b]
        lo = max(0, L - W)
        base = lo - lo % 16
        for g in range(2):
            for t in range(64):
                assert valid[b, g, t] == (lo <= t < L)
                if lo <= t < L:
                    assert slot[b, g, t] == table[b][t // 5] * 5 + t % 5
                    assert part[b, g, t] == (t - base) // T
            assert tuple(ranges[b, g, 0]) == (base, min(base + T, L))


def test_expected_trace_with_window_and_rows_matches_token_loop():
    W, n = 21, 3
    case = kvgen.make_case(3, 8, 2, 64, 5, [0, 23, 61], seed=45, extra_blocks=2,
                           sliding_window=W, q_len=n)
    P, T = 1, 64
    slot, part, ranges, valid = bookkeeping.expected_trace(
        case.block_table.numpy(), case.seq_lens, 2, case.bs, 64, P, T, window=W, q_len=n)
    table = case.block_table.numpy()
    for b in range(3):
        L = case.seq_lens[b]
        lo = max(0, L - n + 1 - W)           # the earliest row's window
        base = lo - lo % 16
        for g in range(2):
            for t in range(64):
                assert valid[b, g, t] == (lo <= t < L)
                if lo <= t < L:
                    assert slot[b, g, t] == table[b][t // 5] * 5 + t % 5
                    assert part[b, g, t] == (t - base) // T
            assert tuple(ranges[b, g, 0]) == (base, min(base + T, L))

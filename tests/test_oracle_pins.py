"""Pins of the CPU oracle against things other than itself.

Each test fixes a part of the oracle that a plausible mistake would break:
  * torch's own scaled_dot_product_attention in float64 with its GQA mode, a
    library routine for exactly this operation (catches dropped terms, wrong
    signs, transposed operands, a wrong scale, a wrong head mapping);
  * closed forms: one-token context, zero query, constant V, a hand-computed
    worked example (catch normalisation and max-subtraction mistakes);
  * invariants: convex combination of V rows, GQA == MHA on repeated KV
    heads, thread-count invariance, the log-sum-exp merge of partials;
  * the size of the pages' error metric under plain output rounding.
CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import kvgen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa_f64(q, k, v, lens, scale):
    """torch SDPA in float64, per sequence (lengths differ), GQA enabled."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        if lens[b] == 0:
            continue
        qt = torch.from_numpy(np.asarray(q[b], dtype=np.float64))[None, :, None, :]
        kt = torch.from_numpy(np.asarray(k[b], dtype=np.float64))[None]
        vt = torch.from_numpy(np.asarray(v[b], dtype=np.float64))[None]
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale,
                                                              enable_gqa=True)
        out[b] = o[0, :, 0, :].numpy()
    return out


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 6, 8])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_matches_torch_sdpa_float64(D, G, dtype):
    rng = np.random.default_rng(D * 100 + G + (7 if dtype == "fp16" else 0))
    B = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 3))
    lens = [int(x) for x in rng.integers(1, 65, size=B)]
    case = kvgen.make_case(B, G * Hkv, Hkv, D, bs=int(rng.choice([1, 5, 16])), seq_lens=lens,
                           dtype=dtype, seed=int(rng.integers(1 << 30)))
    q, k, v, L = kvgen.oracle_inputs(case)
    got = oracle.decode(q, k, v, L, case.scale)
    ref = sdpa_f64(q, k, v, L, case.scale)
    assert oracle.rel_linf(got, ref) <= 1e-5


def test_long_context_accumulation_error():
    """At 32K tokens the oracle's own fp32 error stays >= 100x below the
    tightest tolerance used against it (2e-3)."""
    case = kvgen.make_case(1, 2, 1, 128, 16, [32768], seed=11)
    q, k, v, L = kvgen.oracle_inputs(case)
    got = oracle.decode(q, k, v, L, case.scale)
    ref = sdpa_f64(q, k, v, L, case.scale)
    assert oracle.rel_linf(got, ref) <= 2e-5


def test_single_token_is_exactly_the_v_row():
    case = kvgen.make_case(3, 8, 2, 128, 16, [1, 1, 1], seed=3)
    q, k, v, L = kvgen.oracle_inputs(case)
    got = oracle.decode(q, k, v, L, case.scale)
    for b in range(3):
        for h in range(8):
            np.testing.assert_array_equal(got[b, h], v[b][h // 4, 0])


@pytest.mark.parametrize("how", ["zero_q", "zero_scale"])
def test_uniform_weights_give_the_mean(how):
    case = kvgen.make_case(2, 4, 2, 64, 16, [37, 300], seed=5)
    q, k, v, L = kvgen.oracle_inputs(case)
    scale = case.scale
    if how == "zero_q":
        q = np.zeros_like(q)
    else:
        scale = 0.0
    got = oracle.decode(q, k, v, L, scale)
    for b in range(2):
        for h in range(4):
            mean = np.asarray(v[b][h // 2], dtype=np.float64).mean(axis=0)
            assert np.max(np.abs(got[b, h] - mean)) <= 1e-6 * max(1.0, np.max(np.abs(mean)))


def test_constant_v_rows():
    case = kvgen.make_case(1, 6, 3, 128, 16, [513], seed=9)
    q, k, v, L = kvgen.oracle_inputs(case)
    c = np.linspace(-3, 3, 128, dtype=np.float32)
    v = [np.broadcast_to(c, vb.shape).copy() for vb in v]
    got = oracle.decode(q, k, v, L, case.scale)
    # Both sums of the second pass are recursive fp32 sums of n positive
    # terms; each carries a relative error of at most (n-1)u (u = 2^-24), so
    # the quotient is c to within about 2nu relative (Higham, "Accuracy and
    # Stability of Numerical Algorithms", recursive summation).
    bound = 2 * L[0] * 2.0 ** -24 * np.abs(c) + np.spacing(np.abs(c))
    assert np.all(np.abs(got - c[None, None, :]) <= bound[None, None, :])


def test_convex_combination_bounds():
    case = kvgen.make_case(2, 8, 4, 128, 16, [77, 1000], seed=13)
    q, k, v, L = kvgen.oracle_inputs(case)
    got = oracle.decode(q, k, v, L, case.scale)
    for b in range(2):
        for h in range(8):
            vb = v[b][h // 2]
            lo, hi = vb.min(axis=0), vb.max(axis=0)
            eps = 1e-5 * np.maximum(1.0, np.abs(vb).max())
            assert np.all(got[b, h] >= lo - eps) and np.all(got[b, h] <= hi + eps)


@pytest.mark.parametrize("G", [2, 3, 6])
def test_gqa_equals_mha_on_repeated_kv(G):
    case = kvgen.make_case(2, 2 * G, 2, 128, 16, [50, 129], seed=17 + G)
    q, k, v, L = kvgen.oracle_inputs(case)
    got = oracle.decode(q, k, v, L, case.scale)
    k_rep = [np.repeat(kb, G, axis=0) for kb in k]
    v_rep = [np.repeat(vb, G, axis=0) for vb in v]
    mha = oracle.decode(q, k_rep, v_rep, L, case.scale)
    np.testing.assert_array_equal(got, mha)


def test_worked_example_golden():
    with open(os.path.join(GOLDEN, "worked_softmax.json")) as f:
        g = json.load(f)
    q = np.asarray(g["q"], dtype=np.float32)[None, None, :]
    K = np.asarray(g["K"], dtype=np.float32)[None]
    V = np.asarray(g["V"], dtype=np.float32)[None]
    got = oracle.decode(q, [K], [V], [K.shape[1]], g["scale"])
    np.testing.assert_allclose(got[0, 0], g["expected_out"], atol=g["tolerance_abs"], rtol=0)
    # the weights themselves: V = identity columns picks them out
    eye = np.eye(3, dtype=np.float32)[None]
    got_w = oracle.decode(np.pad(q, ((0, 0), (0, 0), (0, 1))),
                          [np.pad(K, ((0, 0), (0, 0), (0, 1)))], [eye], [3], g["scale"])
    np.testing.assert_allclose(got_w[0, 0], g["expected_weights"], atol=g["tolerance_abs"], rtol=0)


def test_empty_sequence_gives_zeros():
    case = kvgen.make_case(2, 4, 2, 64, 16, [0, 9], seed=19)
    q, k, v, L = kvgen.oracle_inputs(case)
    got = oracle.decode(q, k, v, L, case.scale)
    assert np.all(got[0] == 0.0) and np.all(np.isfinite(got))


def test_thread_count_does_not_change_results():
    case = kvgen.make_case(3, 8, 2, 128, 16, [400, 33, 1500], seed=23)
    q, k, v, L = kvgen.oracle_inputs(case)
    a = oracle.decode(q, k, v, L, case.scale, nthreads=1)
    b = oracle.decode(q, k, v, L, case.scale, nthreads=8)
    np.testing.assert_array_equal(a, b)


def test_rows_subset_matches_full():
    case = kvgen.make_case(3, 8, 2, 128, 16, [40, 33, 150], seed=29)
    q, k, v, L = kvgen.oracle_inputs(case)
    full = oracle.decode(q, k, v, L, case.scale)
    rows = [(2, 7), (0, 0), (1, 3)]
    sub = oracle.decode_rows(q, k, v, L, case.scale, rows)
    for i, (b, h) in enumerate(rows):
        np.testing.assert_array_equal(sub[i], full[b, h])


@pytest.mark.parametrize("cuts", [[0, 100, 333], [0, 1, 2, 640, 999], [0, 512]])
def test_lse_merge_of_partials_equals_direct(cuts):
    """Splitting the context, computing (o_p, m_p, l_p) per piece and merging
    with weights l_p * exp(m_p - M) reproduces the unsplit row: the algebra
    the split-KV reduction relies on (page "Hybrid-SSM decode rate on dual
    Radeon cards", split-KV passage: split the KV range, reduce afterwards)."""
    L = 1000
    case = kvgen.make_case(1, 4, 1, 128, 16, [L], seed=31)
    q, k, v, lens = kvgen.oracle_inputs(case)
    direct = oracle.decode(q, k, v, lens, case.scale)
    bounds = list(cuts) + [L]
    for h in range(4):
        parts = [oracle.partial(q, k, v, lens, case.scale, 0, h, bounds[i], bounds[i + 1])
                 for i in range(len(bounds) - 1)]
        parts = [p for p in parts if p[2] > 0]
        M = max(p[1] for p in parts)
        w = [p[2] * math.exp(p[1] - M) for p in parts]
        merged = sum(wi * p[0].astype(np.float64) for wi, p in zip(w, parts)) / sum(w)
        # both sides are fp32 recursive sums over <= 1000 terms: allow 1e-5
        # relative to the row's scale (the worst case n*u is 6e-5)
        assert np.max(np.abs(merged - direct[0, h])) <= 1e-5 * np.max(np.abs(direct[0, h]))


@pytest.mark.parametrize("dtype,bound", [("bf16", 2.0 ** -8), ("fp16", 2.0 ** -11)])
def test_metric_floor_of_output_rounding(dtype, bound):
    """Rounding the fp32 reference to the 16-bit output type alone costs at
    most one half-ulp relative to the largest output, and (for many outputs)
    more than a quarter of that: the floor under the pages' 2.12e-3..4.72e-3
    bf16 band (page "vLLM's custom ROCm paged-attention kernel wins all sixty
    cells", abstract and section 3)."""
    case = kvgen.make_case(2, 32, 8, 128, 16, [4096, 1000], seed=37)
    q, k, v, L = kvgen.oracle_inputs(case)
    ref = oracle.decode(q, k, v, L, case.scale)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    rounded = torch.from_numpy(ref).to(tdt).float().numpy()
    err = oracle.rel_linf(rounded, ref)
    assert bound / 4 < err <= bound


# ---- sliding window (the sliding layers of page "vLLM's custom ROCm
# paged-attention kernel wins all sixty cells", section 4, Figure 3) -------

def sdpa_f64_masked(q, k, v, lens, scale, window):
    """torch SDPA in float64 over each sequence's whole context with a key
    mask that keeps t >= L - W: the window fixed by masking, not by slicing
    (the oracle slices)."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = lens[b]
        if L == 0:
            continue
        qt = torch.from_numpy(np.asarray(q[b], dtype=np.float64))[None, :, None, :]
        kt = torch.from_numpy(np.asarray(k[b], dtype=np.float64))[None]
        vt = torch.from_numpy(np.asarray(v[b], dtype=np.float64))[None]
        keep = (torch.arange(L) >= L - window)[None, :]     # [1 query, L keys]
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=keep,
                                                              scale=scale, enable_gqa=True)
        out[b] = o[0, :, 0, :].numpy()
    return out


@pytest.mark.parametrize("lens,W", [([40, 33], 1), ([40, 33], 17), ([40, 33], 40),
                                    ([40, 33], 64), ([100, 57], 33), ([64, 48], 16),
                                    ([300, 1], 129)])
def test_window_matches_masked_sdpa(lens, W):
    case = kvgen.make_case(2, 8, 2, 64, 16, lens, seed=7 + W, sliding_window=W)
    q, k, v, L = kvgen.oracle_inputs(case)
    got = oracle.decode(q, k, v, L, case.scale, window=W)
    ref = sdpa_f64_masked(q, k, v, L, case.scale, W)
    assert oracle.rel_linf(got, ref) <= 1e-5
    # and a window changes the result whenever it cuts the context
    full = oracle.decode(q, k, v, L, case.scale)
    if W < max(lens):
        assert oracle.rel_linf(got, full) > 1e-3


def test_window_of_one_token_is_the_last_v_row():
    case = kvgen.make_case(2, 4, 2, 128, 16, [37, 9], seed=11, sliding_window=1)
    q, k, v, L = kvgen.oracle_inputs(case)
    got = oracle.decode(q, k, v, L, case.scale, window=1)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(got[b, h], v[b][h // 2, L[b] - 1])


def test_window_covering_the_context_is_the_full_decode():
    case = kvgen.make_case(2, 8, 4, 128, 16, [40, 17], seed=12)
    q, k, v, L = kvgen.oracle_inputs(case)
    full = oracle.decode(q, k, v, L, case.scale)
    for W in (40, 41, 1000):
        assert np.array_equal(oracle.decode(q, k, v, L, case.scale, window=W), full)


# ---- multi-row decode: q_len causal rows per sequence ----------------------

def sdpa_f64_causal(q, k, v, lens, scale, window=0):
    """torch SDPA in float64 with an explicit [n, L] key mask: row i keeps
    t <= L - n + i (and t > L - n + i - W with a window).  Rows whose mask is
    empty are defined as zero (returned as such)."""
    B, n, Hq, D = q.shape
    out = np.zeros((B, n, Hq, D), dtype=np.float64)
    for b in range(B):
        L = lens[b]
        if L == 0:
            continue
        t = torch.arange(L)[None, :]
        e = (L - n + torch.arange(n) + 1)[:, None]          # exclusive end per row
        keep = t < e
        if window > 0:
            keep &= t >= e - window
        qt = torch.from_numpy(np.asarray(q[b], dtype=np.float64)).permute(1, 0, 2)[None]  # [1,Hq,n,D]
        kt = torch.from_numpy(np.asarray(k[b], dtype=np.float64))[None]
        vt = torch.from_numpy(np.asarray(v[b], dtype=np.float64))[None]
        rows = keep.any(dim=1)
        mask = keep.clone()
        mask[~rows] = True                                   # avoid an all-masked row in SDPA
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                              scale=scale, enable_gqa=True)
        o = o[0].permute(1, 0, 2).numpy()                    # [n, Hq, D]
        o[~rows.numpy()] = 0.0
        out[b] = o
    return out


@pytest.mark.parametrize("lens,n,W", [([40, 33], 2, 0), ([40, 33], 4, 0), ([100, 7], 8, 0),
                                      ([3, 60], 5, 0), ([64, 48], 3, 17), ([200, 9], 4, 1),
                                      ([37, 2], 6, 5)])
def test_multi_row_matches_causal_sdpa(lens, n, W):
    case = kvgen.make_case(2, 8, 2, 64, 16, lens, seed=30 + n + W, q_len=n, sliding_window=W)
    q, k, v, L = kvgen.oracle_inputs(case)
    got = oracle.decode_multi(q, k, v, L, case.scale, window=W)
    ref = sdpa_f64_causal(q, k, v, L, case.scale, window=W)
    assert got.shape == (2, n, 8, 64)
    assert oracle.rel_linf(got, ref) <= 1e-5
    # rows with no token (L < n) are zeros
    for b in range(2):
        for i in range(n):
            if lens[b] - n + i + 1 <= 0:
                assert np.all(got[b, i] == 0)


def test_multi_row_last_row_is_the_plain_decode_and_one_row_is_decode():
    n = 4
    case = kvgen.make_case(3, 8, 4, 128, 16, [50, 17, 300], seed=41, q_len=n)
    q, k, v, L = kvgen.oracle_inputs(case)
    got = oracle.decode_multi(q, k, v, L, case.scale)
    last = oracle.decode(q[:, n - 1], k, v, L, case.scale)
    assert np.array_equal(got[:, n - 1], last)
    # row 0 is the decode of the sequence without its last n - 1 tokens
    k0 = [x[:, :Lb - n + 1] for x, Lb in zip(k, L)]
    v0 = [x[:, :Lb - n + 1] for x, Lb in zip(v, L)]
    first = oracle.decode(q[:, 0], k0, v0, [Lb - n + 1 for Lb in L], case.scale)
    assert np.array_equal(got[:, 0], first)
    # one row per sequence through decode_multi is decode
    q1 = q[:, :1]
    assert np.array_equal(oracle.decode_multi(q1, k, v, L, case.scale)[:, 0],
                          oracle.decode(q[:, 0], k, v, L, case.scale))


# ---- fp8 KV: the OCP E4M3 decode and dequantisation ------------------------

def test_e4m3_closed_form_values():
    v = oracle.e4m3_value
    assert v(0x00) == 0.0 and v(0x80) == 0.0 and np.signbit(v(0x80))
    assert v(0x38) == 1.0 and v(0xB8) == -1.0 and v(0xC0) == -2.0
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0          # largest finite
    assert v(0x01) == 2.0 ** -9                              # smallest subnormal
    assert v(0x07) == 7 / 8 * 2.0 ** -6                      # largest subnormal
    assert v(0x08) == 2.0 ** -6                              # smallest normal
    assert v(0x39) == 1.125 and v(0x30) == 0.5
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))           # the only NaNs
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_value(codes)
    assert np.isnan(vals).sum() == 2
    finite = vals[~np.isnan(vals)]
    assert np.all(np.isfinite(finite)) and finite.max() == 448.0


def test_e4m3_matches_torch_float8_e4m3fn_on_every_code():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = oracle.e4m3_value(codes.numpy())
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_fp8_decode_closed_form_equal_keys():
    """All K bytes equal: every score is equal, so each output row is the
    plain mean of its sequence's dequantised V rows."""
    B, Hq, Hkv, D = 2, 4, 2, 64
    lens = [37, 5]
    rng = np.random.default_rng(3)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    k = [np.full((Hkv, L, D), 0x38, dtype=np.uint8) for L in lens]      # all 1.0
    v = [rng.integers(0, 256, size=(Hkv, L, D)).astype(np.uint8) for L in lens]
    for x in v:
        x[(x & 0x7F) == 0x7F] = 0x38                                       # no NaN codes
    ks, vs = 0.25, 0.0625
    got = oracle.decode(q, k, v, lens, 0.1, kv_scales=(ks, vs))
    for b, L in enumerate(lens):
        vals = oracle.e4m3_value(v[b]) * vs                                # [Hkv, L, D]
        for h in range(Hq):
            ref = vals[h // (Hq // Hkv)].mean(axis=0)
            assert np.max(np.abs(got[b, h] - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_fp8_generator_round_trip():
    """The generator's fp8 codes decode to within one E4M3 rounding step of
    the drawn values (relative half-ULP 2^-4 for normals)."""
    case = kvgen.make_case(2, 8, 2, 64, 16, [40, 33], seed=5, kv_dtype="fp8")
    assert case.k_cache.dtype == torch.float8_e4m3fn
    q, k, v, lens = kvgen.oracle_inputs(case)
    assert k[0].dtype == np.uint8
    kk = oracle.dequantize_e4m3(k[0], case.k_scale)
    assert np.isfinite(kk).all() and np.max(np.abs(kk)) <= 448 * case.k_scale * (1 + 1e-6)

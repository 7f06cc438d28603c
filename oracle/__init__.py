"""CPU oracle for single-token paged-attention decode.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke entry
point (``__graft_entry__.smoke``) and the CPU-baseline leg of ``bench.py`` may
import it.  It shares no code with the GPU library (``paged_kv_cache_decode_amd``)
and never imports it; the GPU library never imports this package.

Contents
  decode / decode_rows / partial   fp32 two-pass softmax(q K^T * scale) V over
                                   the contiguous, pre-paging K/V tensors
                                   (optionally over each sequence's last W
                                   tokens: a sliding window)
                                   (oracle.c, via ctypes).  The pages fix the
                                   reference at fp32 computed from pre-paging
                                   KV (page "vLLM's custom ROCm paged-attention
                                   kernel wins all sixty cells", section 1).
  decode_multi                     multi-row decode: q_len query rows per
                                   sequence at its last q_len positions, row
                                   i attending causally to the prefix that
                                   ends at its own position -- each row is
                                   plain decode over that prefix (the
                                   speculative / multi-token decode the
                                   pages ask about: first page, section 6,
                                   "One machine, and the model runner
                                   question").
  plan                             the partition plan, re-derived from its
                                   documentation in include/pda.h (plan.py).
  bookkeeping                      expected per-token physical slot and
                                   partition, and per-unit token ranges
                                   (bookkeeping.py).
  e4m3_value / dequantize_e4m3     the OCP FP8 E4M3 code -> value map, from
                                   the format's definition, and per-tensor
                                   dequantisation (fp8 KV: the fp8 KV the
                                   first page lists as untested, section 6);
                                   decode* take kv_scales=(k_scale, v_scale)
                                   to read K/V given as E4M3 bytes.
  rel_linf                         the pages' score: relative L-infinity
                                   against the reference's own scale.

Inputs to decode*: ``q`` float32 [B, Hq, D]; ``k`` and ``v`` lists over b of
float32 [Hkv, L_b, D] (exact upcasts of the 16-bit data).
"""
import ctypes
import os

import numpy as np

from . import plan  # noqa: F401  (re-export)
from . import bookkeeping  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from .build import build_oracle
        build_oracle()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.oracle_decode_rows.argtypes = [i32, i32, i32, i32, P, P, P, P, P, ctypes.c_float,
                                       i32, P, P, P, i32]
    lib.oracle_decode_rows.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [i32, i32, i32, i32, P, P, P, P, P, ctypes.c_float, P, i32]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_partial.argtypes = [i32, i32, i32, i32, P, P, P, P, P, ctypes.c_float,
                                   i32, i32, i32, i32, P, P, P]
    lib.oracle_partial.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class _Packed:
    """Concatenates per-sequence [Hkv, L_b, D] tensors into one buffer."""

    def __init__(self, q, k, v, seq_lens):
        self.q = np.ascontiguousarray(q, dtype=np.float32)
        B, Hq, D = self.q.shape
        self.B, self.Hq, self.D = B, Hq, D
        self.seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        assert self.seq_lens.shape == (B,)
        assert len(k) == B and len(v) == B
        Hkv = k[0].shape[0]
        self.Hkv = Hkv
        sizes = []
        for b in range(B):
            L = int(self.seq_lens[b])
            assert k[b].shape == (Hkv, L, D), (k[b].shape, (Hkv, L, D))
            assert v[b].shape == (Hkv, L, D)
            sizes.append(Hkv * L * D)
        self.kv_off = np.zeros(B, dtype=np.int64)
        if B > 1:
            self.kv_off[1:] = np.cumsum(sizes[:-1])
        total = max(1, int(sum(sizes)))
        self.k = np.empty(total, dtype=np.float32)
        self.v = np.empty(total, dtype=np.float32)
        for b in range(B):
            o, n = int(self.kv_off[b]), sizes[b]
            self.k[o:o + n] = np.asarray(k[b], dtype=np.float32).reshape(-1)
            self.v[o:o + n] = np.asarray(v[b], dtype=np.float32).reshape(-1)


def e4m3_value(codes) -> np.ndarray:
    """Values (float64) of OCP FP8 E4M3 bytes, from the format's definition:
    bit 7 the sign, bits 6-3 the exponent e with bias 7, bits 2-0 the
    mantissa m; e == 0 is subnormal, m/8 * 2^-6; otherwise (1 + m/8) * 2^(e-7);
    e == 15 with m == 7 is NaN; there is no infinity (largest value 448)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    val = np.where(c & 0x80, -mag, mag)
    return np.where((e == 15) & (c & 0x7 == 7), np.nan, val)


def dequantize_e4m3(codes, scale: float) -> np.ndarray:
    """float32 values of E4M3 bytes under a per-tensor scale: value * scale
    (one rounding to fp32)."""
    return (e4m3_value(codes) * float(scale)).astype(np.float32)


def _kv_values(k, v, kv_scales):
    if kv_scales is None:
        return k, v
    ks, vs = kv_scales
    return ([dequantize_e4m3(x, ks) for x in k], [dequantize_e4m3(x, vs) for x in v])


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _window(k, v, seq_lens, window: int):
    """Restrict each sequence to its last `window` tokens (window > 0): the
    sliding-window layers attend to t in [max(0, L - W), L) (page "vLLM's
    custom ROCm paged-attention kernel wins all sixty cells", section 4,
    Figure 3).  window == 0 keeps the whole context."""
    if window <= 0:
        return k, v, seq_lens
    lens = [int(L) for L in seq_lens]
    lo = [max(0, L - window) for L in lens]
    k = [np.asarray(k[b])[:, lo[b]:lens[b]] for b in range(len(lens))]
    v = [np.asarray(v[b])[:, lo[b]:lens[b]] for b in range(len(lens))]
    return k, v, [lens[b] - lo[b] for b in range(len(lens))]


def decode(q, k, v, seq_lens, scale, nthreads: int = 0, window: int = 0,
           kv_scales=None) -> np.ndarray:
    """All rows: float32 [B, Hq, D].  kv_scales=(k_scale, v_scale): k and v
    are E4M3 bytes, dequantised first."""
    lib = _load()
    k, v = _kv_values(k, v, kv_scales)
    k, v, seq_lens = _window(k, v, seq_lens, window)
    pk = _Packed(q, k, v, seq_lens)
    out = np.empty((pk.B, pk.Hq, pk.D), dtype=np.float32)
    rc = lib.oracle_decode(pk.B, pk.Hq, pk.Hkv, pk.D, _ptr(pk.seq_lens), _ptr(pk.kv_off),
                           _ptr(pk.q), _ptr(pk.k), _ptr(pk.v), float(scale), _ptr(out),
                           int(nthreads))
    if rc != 0:
        raise ValueError("oracle_decode failed")
    return out


def decode_multi(q, k, v, seq_lens, scale, nthreads: int = 0, window: int = 0,
                 kv_scales=None) -> np.ndarray:
    """q float32 [B, n, Hq, D]: n query rows per sequence, row i at position
    L - n + i.  Row i attends to the tokens t <= L - n + i (causal among the
    new rows, whose K/V are the sequence's last n), and with a sliding window
    W > 0 to the last W of those.  So row i is the plain decode of the
    sequence truncated to its first L - n + i + 1 tokens (zeros when that is
    not positive).  Returns float32 [B, n, Hq, D]."""
    q = np.asarray(q, dtype=np.float32)
    B, n, Hq, D = q.shape
    k, v = _kv_values(k, v, kv_scales)
    kk, vv, ll = [], [], []
    for b in range(B):
        L = int(seq_lens[b])
        for i in range(n):
            e = max(0, L - n + i + 1)
            kk.append(np.asarray(k[b])[:, :e])
            vv.append(np.asarray(v[b])[:, :e])
            ll.append(e)
    out = decode(q.reshape(B * n, Hq, D), kk, vv, ll, scale, nthreads=nthreads, window=window)
    return out.reshape(B, n, Hq, D)


def decode_rows(q, k, v, seq_lens, scale, rows, nthreads: int = 0, window: int = 0) -> np.ndarray:
    """Selected (b, h) rows: float32 [len(rows), D]."""
    lib = _load()
    k, v, seq_lens = _window(k, v, seq_lens, window)
    pk = _Packed(q, k, v, seq_lens)
    rows = list(rows)
    rb = np.ascontiguousarray([r[0] for r in rows], dtype=np.int32)
    rh = np.ascontiguousarray([r[1] for r in rows], dtype=np.int32)
    out = np.empty((len(rows), pk.D), dtype=np.float32)
    rc = lib.oracle_decode_rows(pk.B, pk.Hq, pk.Hkv, pk.D, _ptr(pk.seq_lens), _ptr(pk.kv_off),
                                _ptr(pk.q), _ptr(pk.k), _ptr(pk.v), float(scale), len(rows),
                                _ptr(rb), _ptr(rh), _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_decode_rows failed")
    return out


def partial(q, k, v, seq_lens, scale, b, h, t0, t1):
    """Two-pass softmax over tokens [t0, t1) of row (b, h): (o[D], m, l),
    natural-exp domain, o normalised by l."""
    lib = _load()
    pk = _Packed(q, k, v, seq_lens)
    o = np.empty(pk.D, dtype=np.float32)
    m = np.zeros(1, dtype=np.float32)
    l = np.zeros(1, dtype=np.float32)
    rc = lib.oracle_partial(pk.B, pk.Hq, pk.Hkv, pk.D, _ptr(pk.seq_lens), _ptr(pk.kv_off),
                            _ptr(pk.q), _ptr(pk.k), _ptr(pk.v), float(scale), int(b), int(h),
                            int(t0), int(t1), _ptr(o), _ptr(m), _ptr(l))
    if rc != 0:
        raise ValueError("oracle_partial failed")
    return o, float(m[0]), float(l[0])


def rel_linf(got, ref) -> float:
    """max |got - ref| / max |ref| -- relative L-infinity against the
    reference's own scale (page "vLLM's custom ROCm paged-attention kernel
    wins all sixty cells", section 1).  A NaN anywhere in ``got`` gives inf;
    an all-zero reference compares absolutely."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"shape mismatch {got.shape} vs {ref.shape}")
    if got.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got - ref)))
    return err / scale if scale > 0 else err

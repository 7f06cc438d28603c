"""Partition plan, re-derived from its documentation in include/pda.h.

TEST INFRASTRUCTURE.  This is an independent re-implementation, written from
the formula stated in the header's comment, not from the library's C++; the
tests require the library's plan to equal this one bit for bit.

The pages do not print the split heuristic of the split-KV decode they
measure (page "Hybrid-SSM decode rate on dual Radeon cards", split-KV
passage: the KV range is split over more workgroups and reduced afterwards),
so the rule is this library's own; what the pages fix is the reason for it:
4 KV heads at batch 1 leave too little to spread over the compute units
(same page, the occupancy table and the paragraph under it).
"""

TP_ALIGN = 64
VALU_MAX_GROUP = 8
MFMA_MIN_GROUP = 2
WG_MIN_BYTES = 64 * 1024
WG_MANY_BYTES = 1024 * 1024
WG_ONE_BYTES = 1024 * 1024
MAX_PARTITIONS = 65535
VALU, MFMA = 1, 2
MERGE_FUSED, MERGE_KERNEL = 0, 1
FUSED_MAX_PARTS = 16
FUSED_MAX_BYTES = 32 * 1024
FUSED_MAX_UNITS = 16384


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def variant(num_seqs: int, num_kv_heads: int, group: int, q_len: int = 1,
            kv_fp8: bool = False) -> int:
    """MFMA for fp8 KV or for R = q_len * G >= 2 rows per unit; VALU for
    one row."""
    rows = max(1, q_len) * group
    if kv_fp8 or rows >= MFMA_MIN_GROUP:
        return MFMA
    return VALU


def token_bounds(head_size: int, kv_fp8: bool = False):
    """(T_min, T_many, T_one) in tokens."""
    bpt = (2 if kv_fp8 else 4) * head_size  # K and V bytes of one token and KV head
    t_min = max(TP_ALIGN, (WG_MIN_BYTES // bpt // TP_ALIGN) * TP_ALIGN)
    t_many = max(t_min, (WG_MANY_BYTES // bpt // TP_ALIGN) * TP_ALIGN)
    t_one = max(t_many, (WG_ONE_BYTES // bpt // TP_ALIGN) * TP_ALIGN)
    return t_min, t_many, t_one


def span(max_seq_len: int, window: int = 0, q_len: int = 1) -> int:
    """Tokens the partitions must cover: max_seq_len, or with a sliding
    window W > 0 at most W + q_len - 1 + 15 (the union of the q_len rows'
    windows, from its first token rounded down to a multiple of 16)."""
    n = max(1, q_len)
    return min(max_seq_len, window + n - 1 + 15) if window > 0 else max_seq_len


def partition(num_seqs: int, num_kv_heads: int, group: int, head_size: int, max_seq_len: int,
              cu_count: int, window: int = 0, q_len: int = 1, kv_fp8: bool = False):
    """(P, T_p, variant) for the documented rule."""
    var = variant(num_seqs, num_kv_heads, group, q_len, kv_fp8)
    t_min, t_many, t_one = token_bounds(head_size, kv_fp8)
    units = num_seqs * num_kv_heads
    p_fill = _cdiv(cu_count, units)
    lspan = span(max_seq_len, window, q_len)
    if lspan <= 0:
        t_p = t_min
    else:
        t_fill = max(t_min, _cdiv(_cdiv(lspan, p_fill), TP_ALIGN) * TP_ALIGN)
        t_p = t_fill if t_fill <= t_one else t_many
        t_p = max(t_p, _cdiv(_cdiv(lspan, MAX_PARTITIONS), TP_ALIGN) * TP_ALIGN)
    p = max(1, _cdiv(lspan, t_p))
    return p, t_p, var


def merge(p: int, rows: int, head_size: int, units: int = 1) -> int:
    """Merge mode: fused (the last workgroup of a unit merges) when the
    context is split (P > 1) into at most 16 partitions whose fp32 partial
    outputs, P * R * D * 4 bytes for the unit's R rows, are at most 32 KiB,
    and the B * Hkv units fit the workspace's 16384 arrival counters; the
    separate merge kernel otherwise (and when P == 1, where nothing is
    merged)."""
    if (1 < p <= FUSED_MAX_PARTS and units <= FUSED_MAX_UNITS
            and p * rows * head_size * 4 <= FUSED_MAX_BYTES):
        return MERGE_FUSED
    return MERGE_KERNEL


def workspace_bytes(num_seqs: int, num_q_heads: int, head_size: int, p: int,
                    num_kv_heads: int = 1, q_len: int = 1) -> int:
    """16384 int32 arrival counters (a fixed block, the same for every
    shape), then partial outputs [B][q_len][Hq][P][D] fp32, then (m, l)
    [B][q_len][Hq][P][2] fp32, each part rounded up to 256 bytes; none when
    P == 1.  num_kv_heads does not change the size: the counter block is
    fixed."""
    if p <= 1:
        return 0

    def r256(x):
        return _cdiv(x, 256) * 256
    rows = num_seqs * max(1, q_len) * num_q_heads
    return (FUSED_MAX_UNITS * 4
            + r256(rows * p * head_size * 4)
            + r256(rows * p * 2 * 4))

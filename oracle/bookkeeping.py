"""Expected block-table bookkeeping of the paged decode.

TEST INFRASTRUCTURE.  Written from the definition of the paged cache: token t
of sequence b lives in logical block t // bs at slot t % bs, and the logical
block maps to the physical block block_table[b][t // bs] (the paging whose
bugs the pre-paging reference must not cancel: page "vLLM's custom ROCm
paged-attention kernel wins all sixty cells", section 1).  Partition p of a
(sequence, KV head) unit covers [base + p*T_p, min(base + (p+1)*T_p, L_b))
(the split of the KV range over workgroups: page "Hybrid-SSM decode rate on
dual Radeon cards", split-KV passage; the size rule is in include/pda.h);
base is 0, or with a sliding window W (the sliding layers of the first
page's section 4) the window's first token max(0, L_b - W) rounded down to a
multiple of 16, and only tokens inside the window are attended to.

Plain integer numpy; no code shared with the GPU library.
"""
import numpy as np


def expected_trace(block_table, seq_lens, num_kv_heads: int, block_size: int,
                   max_seq_len: int, num_partitions: int, tokens_per_partition: int,
                   window: int = 0, q_len: int = 1):
    """Returns (slot, part, ranges, valid):
      slot  [B, Hkv, max_seq_len] int64  physical slot block_id*bs + t%bs
      part  [B, Hkv, max_seq_len] int64  partition that owns token t
      ranges [B, Hkv, P, 2] int64        (t0, t1) per unit
      valid [B, Hkv, max_seq_len] bool   t attended to: lo_b <= t < seq_lens[b]
    With a sliding window W > 0, lo_b = max(0, L_b - q_len + 1 - W) (the
    window of the first of the q_len query rows, the earliest one) and the
    partitions of sequence b tile [base_b, L_b), base_b = lo_b rounded down
    to a multiple of 16; without one, lo_b = base_b = 0.
    """
    bt = np.asarray(block_table, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    B = bt.shape[0]
    n = max(1, q_len)
    lo = np.maximum(lens - n + 1 - window, 0) if window > 0 else np.zeros_like(lens)
    base = (lo // 16) * 16
    t = np.arange(max_seq_len, dtype=np.int64)
    valid = (t[None, :] < lens[:, None]) & (t[None, :] >= lo[:, None])   # [B, Lmax]
    logical = t // block_size
    safe_logical = np.minimum(logical, bt.shape[1] - 1)
    phys = np.take_along_axis(bt, np.broadcast_to(safe_logical, (B, max_seq_len)), axis=1)
    slot = phys * block_size + (t % block_size)[None, :]
    part = (t[None, :] - base[:, None]) // tokens_per_partition           # [B, Lmax]
    slot = np.broadcast_to(slot[:, None, :], (B, num_kv_heads, max_seq_len))
    part = np.broadcast_to(part[:, None, :], (B, num_kv_heads, max_seq_len))
    valid3 = np.broadcast_to(valid[:, None, :], (B, num_kv_heads, max_seq_len))
    p = np.arange(num_partitions, dtype=np.int64)
    t0 = base[:, None] + p[None, :] * tokens_per_partition                # [B, P]
    t1 = np.minimum(t0 + tokens_per_partition, lens[:, None])
    ranges = np.stack([t0, t1], axis=-1)                                   # [B, P, 2]
    ranges = np.broadcast_to(ranges[:, None], (B, num_kv_heads, num_partitions, 2))
    return slot, part, ranges, valid3

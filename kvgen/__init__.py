"""Seeded synthetic inputs for paged-attention decode.

This module generates data and lays it out; it holds none of the attention
arithmetic.  Both sides use it: the CPU oracle receives the contiguous,
pre-paging K/V tensors (upcast exactly to fp32), the GPU library receives the
same values scattered into a block-paged pool through a permuted block table.
It imports neither the oracle nor the GPU library.

Recipe (the pages use no dataset: page "vLLM's custom ROCm paged-attention
kernel wins all sixty cells", sections 1 and 3):
  * q, K, V ~ N(0, 1) in fp32 from a seeded torch generator, rounded to
    bf16/fp16 with round-to-nearest-even; drawn in the order q, then K_b and
    V_b for b = 0..B-1, then the block permutation.
  * Physical pool: every block a sequence needs, plus `extra_blocks` blocks no
    sequence references.  A random permutation of all block ids is dealt out in
    sequence order, so tables are fragmented over one shared pool.
  * Unwritten tail slots (slots L_b .. ceil(L_b/bs)*bs-1 of a sequence's last
    block) and every unreferenced block hold `tail` (zero, NaN or 1e4) in K
    and/or V; block-table entries past a sequence's last block point at an
    unreferenced block.  The pages' sweep ran on a zero-filled cache; their
    fault test filled the unwritten tail with NaN, and their control used
    finite 1e4 garbage (same page, section 3 and section 5 / Figure 4).
"""
from dataclasses import dataclass, field, replace
from typing import List, Optional, Sequence

import torch

SEED_BASE = 20261202


def seed_for(cfg: int, cell: int = 0) -> int:
    """Seed of one configuration cell."""
    return SEED_BASE * 10000 + cfg * 1000 + cell


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
_TAIL = {"zero": 0.0, "nan": float("nan"), "1e4": 1.0e4}
# the same fills as OCP E4M3 bytes (fp8 KV): zero, NaN (S.1111.111), and
# the largest finite value 448 standing in for a large finite garbage value
_TAIL_FP8 = {"zero": 0x00, "nan": 0x7F, "1e4": 0x7E}
FP8_MAX = 448.0


@dataclass
class Case:
    B: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    dtype: str
    seq_lens: List[int]
    q: torch.Tensor                 # [B, Hq, D] 16-bit ([B, q_len, Hq, D] for q_len > 1)
    k: List[torch.Tensor]           # per b: [Hkv, L_b, D] 16-bit, pre-paging
    v: List[torch.Tensor]
    k_cache: torch.Tensor           # [NB, Hkv, bs, D] 16-bit
    v_cache: torch.Tensor
    block_table: torch.Tensor       # [B, MBS] int32
    seq_lens_t: torch.Tensor        # [B] int32
    scale: float
    num_blocks: int
    max_blocks_per_seq: int
    max_seq_len: int
    unref_ids: List[int] = field(default_factory=list)
    tail_k: str = "zero"
    tail_v: str = "zero"
    sliding_window: int = 0         # W > 0: decode attends to the last W tokens
    q_len: int = 1                  # query rows per sequence (causal among themselves)
    kv_dtype: str = "same"          # "fp8": k, v and the pools hold E4M3 bytes (float8_e4m3fn)
    k_scale: float = 1.0            # fp8: value = decode(byte) * scale, per tensor
    v_scale: float = 1.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def attended(self, b: int) -> int:
        """Tokens of sequence b the decode reads: the union of its rows'
        ranges (the last W + q_len - 1 tokens with a sliding window W)."""
        L = self.seq_lens[b]
        if self.sliding_window > 0:
            return min(L, self.sliding_window + self.q_len - 1)
        return L

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes: attended tokens only, K and V, 2 bytes per
        element (1 for fp8 KV)."""
        eb = 1 if self.kv_dtype == "fp8" else 2
        return sum(self.attended(b) for b in range(self.B)) * self.Hkv * self.D * 2 * eb


def make_case(B: int, Hq: int, Hkv: int, D: int, bs: int, seq_lens: Sequence[int],
              dtype: str = "bf16", seed: int = 0, device="cpu", extra_blocks: int = 1,
              max_blocks_per_seq: Optional[int] = None, tail_k: str = "zero",
              tail_v: str = "zero", scale: Optional[float] = None,
              max_seq_len: Optional[int] = None, sliding_window: int = 0,
              q_len: int = 1, kv_dtype: str = "same") -> Case:
    assert len(seq_lens) == B and Hq % Hkv == 0
    tdt = _DT[dtype]
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    lens = [int(x) for x in seq_lens]
    qshape = (B, Hq, D) if q_len == 1 else (B, q_len, Hq, D)
    q = torch.randn(qshape, generator=gen, device=device).to(tdt)
    k, v = [], []
    for b in range(B):
        k.append(torch.randn((Hkv, lens[b], D), generator=gen, device=device))
        v.append(torch.randn((Hkv, lens[b], D), generator=gen, device=device))
    k_scale = v_scale = 1.0
    if kv_dtype == "fp8":
        # per-tensor scales that map the largest |value| to the largest E4M3
        # value, then round to E4M3 (nearest even; within range by construction)
        def amax(xs):
            return max([float(x.abs().max()) for x in xs if x.numel()] + [1e-30])
        k_scale, v_scale = amax(k) / FP8_MAX, amax(v) / FP8_MAX
        k = [(x / k_scale).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn) for x in k]
        v = [(x / v_scale).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn) for x in v]
    else:
        k = [x.to(tdt) for x in k]
        v = [x.to(tdt) for x in v]
    nbs = [cdiv(L, bs) for L in lens]
    used = sum(nbs)
    NB = used + max(1, int(extra_blocks))
    perm = torch.randperm(NB, generator=gen, device=device).cpu()
    MBS = max_blocks_per_seq if max_blocks_per_seq is not None else max(1, max(nbs))
    assert MBS >= max(nbs)
    unref = perm[used:].tolist()
    table = torch.full((B, MBS), unref[0], dtype=torch.int32)
    off = 0
    for b in range(B):
        table[b, :nbs[b]] = perm[off:off + nbs[b]].to(torch.int32)
        off += nbs[b]
    case = Case(B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, dtype=dtype, seq_lens=lens, q=q, k=k, v=v,
                k_cache=None, v_cache=None, block_table=table.to(device),
                seq_lens_t=torch.tensor(lens, dtype=torch.int32, device=device),
                scale=float(scale) if scale is not None else D ** -0.5,
                num_blocks=NB, max_blocks_per_seq=MBS,
                max_seq_len=int(max_seq_len) if max_seq_len is not None else max(lens),
                unref_ids=unref, tail_k=tail_k, tail_v=tail_v,
                sliding_window=int(sliding_window), q_len=int(q_len), kv_dtype=kv_dtype,
                k_scale=float(k_scale), v_scale=float(v_scale))
    return page(case, tail_k=tail_k, tail_v=tail_v)


def page(case: Case, tail_k: str = "zero", tail_v: str = "zero",
         block_table: Optional[torch.Tensor] = None, unref_ids: Optional[List[int]] = None) -> Case:
    """Scatter the contiguous K/V of `case` into fresh paged pools through
    `block_table` (default: the case's own), filling unwritten tail slots and
    unreferenced blocks with the given fills.  Returns a new Case."""
    table = case.block_table if block_table is None else block_table
    unref = case.unref_ids if unref_ids is None else unref_ids
    dev = case.q.device
    fp8 = case.kv_dtype == "fp8"
    tdt = torch.uint8 if fp8 else case.q.dtype     # fp8 pools are built as their bytes
    fills = _TAIL_FP8 if fp8 else _TAIL
    shape = (case.num_blocks, case.Hkv, case.bs, case.D)
    kc = torch.full(shape, fills[tail_k], dtype=tdt, device=dev)
    vc = torch.full(shape, fills[tail_v], dtype=tdt, device=dev)
    tcpu = table.cpu()
    for b in range(case.B):
        L = case.seq_lens[b]
        nb = cdiv(L, case.bs)
        if nb == 0:
            continue
        ids = tcpu[b, :nb].to(torch.int64).to(dev)
        for src, dst, fill in ((case.k[b], kc, tail_k), (case.v[b], vc, tail_v)):
            padded = torch.full((case.Hkv, nb * case.bs, case.D), fills[fill], dtype=tdt, device=dev)
            padded[:, :L] = src.view(torch.uint8) if fp8 else src
            dst[ids] = padded.view(case.Hkv, nb, case.bs, case.D).permute(1, 0, 2, 3)
    if fp8:
        kc, vc = kc.view(torch.float8_e4m3fn), vc.view(torch.float8_e4m3fn)
    return replace(case, k_cache=kc, v_cache=vc, block_table=table.to(dev),
                   unref_ids=list(unref), tail_k=tail_k, tail_v=tail_v)


def repermute(case: Case, seed: int) -> Case:
    """The same logical content at a different physical placement: a fresh
    random permutation of the block ids, dealt out again."""
    gen = torch.Generator()
    gen.manual_seed(int(seed))
    NB = case.num_blocks
    perm = torch.randperm(NB, generator=gen)
    nbs = [cdiv(L, case.bs) for L in case.seq_lens]
    used = sum(nbs)
    unref = perm[used:].tolist()
    table = torch.full((case.B, case.max_blocks_per_seq), unref[0], dtype=torch.int32)
    off = 0
    for b in range(case.B):
        table[b, :nbs[b]] = perm[off:off + nbs[b]].to(torch.int32)
        off += nbs[b]
    return page(case, tail_k=case.tail_k, tail_v=case.tail_v, block_table=table, unref_ids=unref)


def poison_before_window(case: Case, fill: str = "nan") -> Case:
    """The same case with the cache slots of every token before its sequence's
    sliding window (t < L_b - q_len + 1 - W, before the window of its earliest
    query row) overwritten with `fill`: tokens the decode must not read."""
    assert case.sliding_window > 0
    fp8 = case.kv_dtype == "fp8"
    kc, vc = case.k_cache.clone(), case.v_cache.clone()
    if fp8:
        kc, vc = kc.view(torch.uint8), vc.view(torch.uint8)
    value = _TAIL_FP8[fill] if fp8 else _TAIL[fill]
    table = case.block_table.cpu().to(torch.int64)
    for b in range(case.B):
        lo = max(0, case.seq_lens[b] - case.q_len + 1 - case.sliding_window)
        if lo == 0:
            continue
        t = torch.arange(lo)
        blocks = table[b, t // case.bs].to(kc.device)
        slots = (t % case.bs).to(kc.device)
        for h in range(case.Hkv):
            kc[blocks, h, slots] = value
            vc[blocks, h, slots] = value
    if fp8:
        kc, vc = kc.view(torch.float8_e4m3fn), vc.view(torch.float8_e4m3fn)
    return replace(case, k_cache=kc, v_cache=vc)


def oracle_inputs(case: Case, seqs: Optional[Sequence[int]] = None):
    """Numpy inputs for the oracle, optionally for a subset of sequences
    (re-indexed 0..len(seqs)-1): q as fp32 (an exact upcast); K and V as fp32
    exact upcasts, or for fp8 KV as their E4M3 bytes (uint8), which the
    oracle decodes with case.k_scale / case.v_scale."""
    idx = list(range(case.B)) if seqs is None else list(seqs)
    q = case.q[idx].float().cpu().numpy()
    if case.kv_dtype == "fp8":
        k = [case.k[b].view(torch.uint8).cpu().numpy() for b in idx]
        v = [case.v[b].view(torch.uint8).cpu().numpy() for b in idx]
        lens = [case.seq_lens[b] for b in idx]
        return q, k, v, lens
    k = [case.k[b].float().cpu().numpy() for b in idx]
    v = [case.v[b].float().cpu().numpy() for b in idx]
    lens = [case.seq_lens[b] for b in idx]
    return q, k, v, lens


def shape_dict(case: Case) -> dict:
    return dict(num_seqs=case.B, num_q_heads=case.Hq, num_kv_heads=case.Hkv,
                head_size=case.D, block_size=case.bs, num_blocks=case.num_blocks,
                max_blocks_per_seq=case.max_blocks_per_seq, max_seq_len=case.max_seq_len,
                dtype=case.dtype, sliding_window=case.sliding_window, q_len=case.q_len,
                kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale)

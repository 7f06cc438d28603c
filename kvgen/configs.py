"""The five workload shapes, as seeded synthetic cases.

  cfg1  tiny paged GQA decode: B 2, Hq 8 / Hkv 4, D 128, bs 16, L {17, 40};
        an 8-block pool, permuted table, NaN in every unwritten tail slot and
        unreferenced block.
  cfg2  the pages' shape sweep: B 1, Hkv 8 with Hq 8/16/24/32 (ratios 1-4),
        D 128, bs 16, L in 1K..32K, zero-filled pool (page "vLLM's custom ROCm
        paged-attention kernel wins all sixty cells", section 1).
  cfg3  gemma-3-27B-like layer: Hq 32 / Hkv 16, D 128, bs 16, B 1 or 8,
        L in 1K..32K plus lengths that straddle the final tile; bf16 and
        fp16; NaN tails in K, V or both (same page, section 5, Figure 4).
        Its sliding layers (cfg3_sliding) attend to the last 1024 tokens only
        (same page, section 4, Figure 3).
  cfg4  low-parallelism layer: B 1, Hq 24 / Hkv 4 (ratio 6), D 256, block
        size 784 = 16 x 49 (page "Hybrid-SSM decode rate on dual Radeon
        cards", the gate passage), L {500, 1K, 4K, 8K, 16K, 24K, 32K}.
  cfg5  batched mixed-length decode: B 64, Hq 32 / Hkv 8, D 128, bs 16,
        L_b ~ U[1K, 32K] redrawn while a multiple of 16, fragmented tables over
        one shared pool, NaN tails.
  TP shares: one GPU's half of cfg4 (Hq 12 / Hkv 2) and of cfg3 (Hq 16 / Hkv 8)
        when the heads are split over two GPUs (the pages run the model at
        TP=2: page "vLLM's custom ROCm paged-attention kernel wins all sixty
        cells", section 4); same shapes otherwise.
Every shape takes q_len > 1 for multi-row decode (that many query rows at
the end of each sequence, causal among themselves) and kv_dtype="fp8" for an
OCP E4M3 KV cache (K and V drawn as above, then rounded to E4M3 under one
scale per tensor that maps the largest |value| to 448).
Lengths "1K..32K" are read as powers of two, 1024..32768; "16k+1" and "16k+7"
as 16385 and 16391.
"""
import torch

from . import Case, make_case, seed_for

CFG2_HQ = (8, 16, 24, 32)
CFG2_LENS = (1024, 2048, 4096, 8192, 16384, 32768)
CFG3_LENS = (1024, 2048, 4096, 4090, 8192, 16384, 16385, 16391, 32767, 32768)
CFG4_LENS = (500, 1024, 4096, 8192, 16384, 24576, 32768)


def cfg1(dtype: str = "bf16", device="cpu", tail: str = "nan") -> Case:
    return make_case(B=2, Hq=8, Hkv=4, D=128, bs=16, seq_lens=[17, 40], dtype=dtype,
                     seed=seed_for(1), device=device, extra_blocks=3, max_blocks_per_seq=3,
                     tail_k=tail, tail_v=tail)


def cfg2(hq: int, L: int, device="cpu", dtype: str = "bf16", cell: int = 0,
         q_len: int = 1, kv_dtype: str = "same") -> Case:
    return make_case(B=1, Hq=hq, Hkv=8, D=128, bs=16, seq_lens=[L], dtype=dtype,
                     seed=seed_for(2, cell), device=device, extra_blocks=1, q_len=q_len,
                     kv_dtype=kv_dtype)


def cfg3(B: int, L: int, dtype: str = "bf16", device="cpu", tail_k: str = "nan",
         tail_v: str = "nan", cell: int = 0, q_len: int = 1, kv_dtype: str = "same") -> Case:
    return make_case(B=B, Hq=32, Hkv=16, D=128, bs=16, seq_lens=[L] * B, dtype=dtype,
                     seed=seed_for(3, cell), device=device, extra_blocks=1,
                     tail_k=tail_k, tail_v=tail_v, q_len=q_len, kv_dtype=kv_dtype)


def cfg3_sliding(B: int, L: int, W: int = 1024, dtype: str = "bf16", device="cpu",
                 tail: str = "nan", cell: int = 0) -> Case:
    return make_case(B=B, Hq=32, Hkv=16, D=128, bs=16, seq_lens=[L] * B, dtype=dtype,
                     seed=seed_for(3, 100 + cell), device=device, extra_blocks=1,
                     tail_k=tail, tail_v=tail, sliding_window=W)


def cfg4(L: int, device="cpu", dtype: str = "bf16", tail: str = "nan", cell: int = 0,
         q_len: int = 1, kv_dtype: str = "same") -> Case:
    return make_case(B=1, Hq=24, Hkv=4, D=256, bs=784, seq_lens=[L], dtype=dtype,
                     seed=seed_for(4, cell), device=device, extra_blocks=1,
                     tail_k=tail, tail_v=tail, q_len=q_len, kv_dtype=kv_dtype)


def cfg4_tp2(L: int, device="cpu", dtype: str = "bf16", tail: str = "nan", cell: int = 0) -> Case:
    return make_case(B=1, Hq=12, Hkv=2, D=256, bs=784, seq_lens=[L], dtype=dtype,
                     seed=seed_for(4, 200 + cell), device=device, extra_blocks=1,
                     tail_k=tail, tail_v=tail)


def cfg3_tp2(B: int, L: int, dtype: str = "bf16", device="cpu", tail: str = "nan",
             cell: int = 0) -> Case:
    return make_case(B=B, Hq=16, Hkv=8, D=128, bs=16, seq_lens=[L] * B, dtype=dtype,
                     seed=seed_for(3, 200 + cell), device=device, extra_blocks=1,
                     tail_k=tail, tail_v=tail)


def cfg5_lens(seed: int, B: int = 64, lo: int = 1024, hi: int = 32768):
    gen = torch.Generator()
    gen.manual_seed(int(seed))
    lens = []
    while len(lens) < B:
        x = int(torch.randint(lo, hi + 1, (1,), generator=gen).item())
        if x % 16 != 0:
            lens.append(x)
    return lens


def cfg5(device="cpu", dtype: str = "bf16", B: int = 64, lo: int = 1024, hi: int = 32768,
         cell: int = 0, q_len: int = 1, kv_dtype: str = "same") -> Case:
    seed = seed_for(5, cell)
    lens = cfg5_lens(seed + 1, B=B, lo=lo, hi=hi)
    return make_case(B=B, Hq=32, Hkv=8, D=128, bs=16, seq_lens=lens, dtype=dtype, seed=seed,
                     device=device, extra_blocks=1, tail_k="nan", tail_v="nan", q_len=q_len,
                     kv_dtype=kv_dtype)

"""The pages' NaN-tail fault test, reproduced on the CPU so the instrument is
known to see the fault before it is pointed at the GPU kernel.

A small numpy paged reader (test-only, not the oracle and not the product)
walks the block table like a paged kernel.  With the planted prior-art
mistake -- the score mask is applied, but the V rows of the whole final block
are multiplied in -- it reproduces the pattern the pages report (golden
fault_pattern.json); reading V exactly up to the sequence end removes every
poisoned cell.  The oracle never reads the pool, so it is immune by
construction; that is why its output is the clean reference.
"""
import json
import os

import numpy as np
import pytest

import kvgen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fault_pattern.json")

MODES = {"K": ("nan", "zero"), "V": ("zero", "nan"), "KV": ("nan", "nan"), "KV_1e4": ("1e4", "1e4")}


def paged_reader(case, whole_block_v: bool):
    kc = case.k_cache.float().numpy()
    vc = case.v_cache.float().numpy()
    table = case.block_table.numpy()
    q = case.q.float().numpy()
    out = np.zeros((case.B, case.Hq, case.D), dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        for b in range(case.B):
            L = case.seq_lens[b]
            nb = kvgen.cdiv(L, case.bs)
            ids = table[b, :nb]
            for h in range(case.Hq):
                g = h // case.G
                K = kc[ids, g].reshape(nb * case.bs, case.D)   # whole blocks
                V = vc[ids, g].reshape(nb * case.bs, case.D)
                s = (K @ q[b, h]) * case.scale
                t = np.arange(nb * case.bs)
                s = np.where(t < L, s, -np.inf)                 # score mask by select
                p = np.exp(s - s[:L].max())
                p = p / p[:L].sum()
                if whole_block_v:
                    out[b, h] = p @ V                           # 0 * NaN reaches the sum
                else:
                    out[b, h] = p[:L] @ V[:L]
    return out


@pytest.mark.parametrize("whole_block_v", [True, False])
def test_fault_pattern_matches_pages(whole_block_v):
    with open(GOLDEN) as f:
        g = json.load(f)
    key = "poisoned_with_whole_block_v_read" if whole_block_v else "poisoned_with_exact_v_read"
    for mode, (tk, tv) in MODES.items():
        for L in g["lengths"]:
            case = kvgen.make_case(1, 4, 2, 64, g["block_size"], [L], seed=41, tail_k=tk, tail_v=tv)
            got = paged_reader(case, whole_block_v)
            poisoned = bool(np.isnan(got).any())
            assert poisoned == g[key][mode][str(L)], (mode, L, whole_block_v)
            if not poisoned:
                q, k, v, lens = kvgen.oracle_inputs(case)
                ref = oracle.decode(q, k, v, lens, case.scale)
                assert oracle.rel_linf(got, ref) < 1e-5

"""Shared helpers of the GPU tests: run a kvgen case through the C-ABI
library and score it against the oracle with the pages' metric."""
import numpy as np
import torch

import kvgen
import oracle
import paged_kv_cache_decode_amd as pda

TOL = {"bf16": 1e-2, "fp16": 2e-3}


def to_device(case: kvgen.Case, device="cuda") -> kvgen.Case:
    from dataclasses import replace
    return replace(case, q=case.q.to(device), k=[x.to(device) for x in case.k],
                   v=[x.to(device) for x in case.v], k_cache=case.k_cache.to(device),
                   v_cache=case.v_cache.to(device), block_table=case.block_table.to(device),
                   seq_lens_t=case.seq_lens_t.to(device))


def shape_of(case: kvgen.Case) -> pda.PdaShape:
    d = kvgen.shape_dict(case)
    return pda.make_shape(**d)


def run(case: kvgen.Case, plan=None, out=None) -> torch.Tensor:
    out = pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                case.seq_lens_t, case.scale, out=out,
                                max_seq_len=case.max_seq_len, plan=plan,
                                sliding_window=case.sliding_window, k_scale=case.k_scale,
                                v_scale=case.v_scale)
    torch.cuda.synchronize()
    return out


def reference(case: kvgen.Case, seqs=None) -> np.ndarray:
    q, k, v, lens = kvgen.oracle_inputs(case, seqs)
    sc = (case.k_scale, case.v_scale) if case.kv_dtype == "fp8" else None
    if case.q_len > 1:
        return oracle.decode_multi(q, k, v, lens, case.scale, window=case.sliding_window,
                                   kv_scales=sc)
    return oracle.decode(q, k, v, lens, case.scale, window=case.sliding_window, kv_scales=sc)


def check(case: kvgen.Case, got: torch.Tensor, ref: np.ndarray = None, seqs=None,
          per_seq: bool = False) -> float:
    """rel-L-inf of the GPU output against the oracle, NaN-freedom, and
    (optionally) the same score per sequence."""
    g = got.float().cpu().numpy()
    if seqs is not None:
        g = g[list(seqs)]
    if ref is None:
        ref = reference(case, seqs)
    assert np.all(np.isfinite(g)), "non-finite value in the GPU output"
    err = oracle.rel_linf(g, ref)
    tol = TOL[case.dtype]
    assert err <= tol, f"rel-Linf {err:.3e} > {tol:.1e}"
    if per_seq:
        for i in range(g.shape[0]):
            e = oracle.rel_linf(g[i], ref[i])
            assert e <= tol, f"sequence {i}: rel-Linf {e:.3e} > {tol:.1e}"
    return err


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy()

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


GUARD_BYTES = 4096          # canary bytes on each side of `out` and the workspace
_CANARY_SEED = 0x5EED


def _guarded(nbytes: int, device) -> tuple:
    """A device buffer of nbytes with GUARD_BYTES of seeded random canary
    bytes on each side; returns (whole buffer, inner slice, canary copy).
    The inner slice starts 4096-byte aligned, as a fresh allocation would."""
    gen = torch.Generator()
    gen.manual_seed(_CANARY_SEED + nbytes)
    whole = torch.randint(0, 256, (2 * GUARD_BYTES + max(nbytes, 0),), dtype=torch.uint8,
                          generator=gen).to(device)
    return whole, whole[GUARD_BYTES:GUARD_BYTES + nbytes], whole.clone()


def _check_guards(name: str, whole: torch.Tensor, before: torch.Tensor, nbytes: int):
    """The canary bytes on both sides of a guarded buffer are untouched."""
    for lo, hi, side in ((0, GUARD_BYTES, "before"),
                         (GUARD_BYTES + nbytes, 2 * GUARD_BYTES + nbytes, "after")):
        changed = int((whole[lo:hi] != before[lo:hi]).sum().item())
        assert changed == 0, f"{changed} canary bytes {side} `{name}` were overwritten"


def run(case: kvgen.Case, plan=None, out=None) -> torch.Tensor:
    """One decode call through the C ABI.  `out` and the workspace are carved
    out of larger buffers whose canary bytes on either side must survive the
    call (an out-of-bounds store by the decode, the fused merge or the merge
    kernel shows up here), and the fused merge's arrival counters must be
    back at zero afterwards."""
    shape = shape_of(case)
    need = (pda.paged_decode_attn_workspace_size(shape) if plan is None
            else pda.pda_workspace_bytes(shape, plan))
    dev = case.q.device
    guards = []
    if out is None:
        nb = case.q.numel() * case.q.element_size()
        whole, inner, before = _guarded(nb, dev)
        out = inner.view(case.q.dtype).view(case.q.shape)
        guards.append(("out", whole, before, nb))
    ws = None
    if need > 0:
        whole, ws, _ = _guarded(need, dev)
        ws.zero_()  # the state a workspace starts in (the counters must be zero)
        guards.append(("workspace", whole, whole.clone(), need))
    out = pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                case.seq_lens_t, case.scale, out=out, workspace=ws,
                                max_seq_len=case.max_seq_len, plan=plan,
                                sliding_window=case.sliding_window, k_scale=case.k_scale,
                                v_scale=case.v_scale)
    torch.cuda.synchronize()
    for g in guards:
        _check_guards(*g)
    if ws is not None:
        ctr = ws[:COUNTER_BYTES].view(torch.int32)
        assert int(ctr.abs().sum().item()) == 0, "arrival counters left non-zero"
    return out


COUNTER_BYTES = 16384 * 4   # the workspace's fixed block of arrival counters


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
    # NaN-freedom over the whole output, before any subset is scored
    bad = int(np.count_nonzero(~np.isfinite(g)))
    assert bad == 0, f"{bad} non-finite values in the GPU output"
    if seqs is not None:
        g = g[list(seqs)]
    if ref is None:
        ref = reference(case, seqs)
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

"""Python binding of libpda.so, the gfx950 paged-attention decode library.

Argument marshalling only: every step of the decode runs in the library's HIP
kernels.  torch supplies device memory and the current stream; nothing else
from torch touches the path.  The binding raises if libpda.so is missing --
there is no CPU fallback.

Names mirror the C ABI in include/pda.h:
  paged_decode_attn(q, k_cache, v_cache, block_table, seq_lens, scale, out, ...)
  paged_decode_attn_workspace_size(shape)
  paged_decode_attn_plan(shape) / pda_plan_for_cus(shape, cu_count)
  paged_decode_attn_with_plan(...) / paged_decode_attn_trace(...)
  pda_status_string(status) / pda_build_id()
"""
import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpda.so")

PDA_OK = 0
PDA_ERR_INVALID = -1
PDA_ERR_UNSUPPORTED = -2
PDA_ERR_WORKSPACE = -3
PDA_ERR_LAUNCH = -4
PDA_ERR_DEVICE = -5
PDA_BF16 = 0
PDA_FP16 = 1
PDA_KV_SAME = 0
PDA_KV_FP8_E4M3 = 1
PDA_VARIANT_VALU = 1
PDA_VARIANT_MFMA = 2
PDA_MERGE_FUSED = 0
PDA_MERGE_KERNEL = 1

_DTYPES = {"bf16": PDA_BF16, "fp16": PDA_FP16}
_KV_DTYPES = {"same": PDA_KV_SAME, "fp8": PDA_KV_FP8_E4M3, "fp8_e4m3": PDA_KV_FP8_E4M3}


class PdaShape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_size", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("sliding_window", ctypes.c_int32),
                ("q_len", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class PdaPlan(ctypes.Structure):
    _fields_ = [("num_partitions", ctypes.c_int32), ("tokens_per_partition", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("merge", ctypes.c_int32),
                ("cu_count", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class PdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {pda_status_string(status)} (status {status})")
        self.status = status


_lib = None


def load_library():
    """Load libpda.so (built in-tree by __graft_entry__.build()); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    sp, pp = ctypes.POINTER(PdaShape), ctypes.POINTER(PdaPlan)
    lib.pda_check_shape.argtypes = [sp]
    lib.pda_check_shape.restype = ctypes.c_int
    lib.pda_plan_for_cus.argtypes = [sp, ctypes.c_int32, pp]
    lib.pda_plan_for_cus.restype = ctypes.c_int
    lib.paged_decode_attn_plan.argtypes = [sp, pp]
    lib.paged_decode_attn_plan.restype = ctypes.c_int
    lib.paged_decode_attn_workspace_size.argtypes = [sp]
    lib.paged_decode_attn_workspace_size.restype = ctypes.c_int64
    lib.pda_workspace_bytes.argtypes = [sp, pp]
    lib.pda_workspace_bytes.restype = ctypes.c_int64
    lib.paged_decode_attn.argtypes = [sp, P, P, P, P, P, ctypes.c_float, P, P, ctypes.c_int64, P]
    lib.paged_decode_attn.restype = ctypes.c_int
    lib.paged_decode_attn_with_plan.argtypes = [sp, pp, P, P, P, P, P, ctypes.c_float, P, P,
                                                ctypes.c_int64, P]
    lib.paged_decode_attn_with_plan.restype = ctypes.c_int
    lib.paged_decode_attn_timed.argtypes = [sp, pp, P, P, P, P, P, ctypes.c_float, P, P,
                                            ctypes.c_int64, P, P, P]
    lib.paged_decode_attn_timed.restype = ctypes.c_int
    lib.paged_decode_attn_trace.argtypes = [sp, pp, ctypes.c_int32, P, P, P, P, P, P]
    lib.paged_decode_attn_trace.restype = ctypes.c_int
    lib.paged_decode_attn_workspace_init.argtypes = [P, ctypes.c_int64, P]
    lib.paged_decode_attn_workspace_init.restype = ctypes.c_int
    lib.paged_decode_attn_workspace_check.argtypes = [P, ctypes.c_int64, P,
                                                      ctypes.POINTER(ctypes.c_int32)]
    lib.paged_decode_attn_workspace_check.restype = ctypes.c_int
    lib.paged_decode_attn_noalloc.argtypes = [sp, P, P, P, P, P, ctypes.c_float, P, P]
    lib.paged_decode_attn_noalloc.restype = ctypes.c_int
    lib.pda_status_string.argtypes = [ctypes.c_int]
    lib.pda_status_string.restype = ctypes.c_char_p
    lib.pda_build_id.argtypes = []
    lib.pda_build_id.restype = ctypes.c_char_p
    lib.pda_read_probe.argtypes = [P, ctypes.c_int64, P, ctypes.c_int32, P]
    lib.pda_read_probe.restype = ctypes.c_int
    _lib = lib
    return lib


def make_shape(num_seqs, num_q_heads, num_kv_heads, head_size, block_size, num_blocks,
               max_blocks_per_seq, max_seq_len, dtype="bf16", sliding_window=0,
               q_len=1, kv_dtype="same", k_scale=1.0, v_scale=1.0) -> PdaShape:
    """sliding_window W > 0: attend to the last W tokens of each sequence.
    q_len > 1: that many query rows per sequence, causal among themselves.
    kv_dtype "fp8": the caches hold OCP E4M3 bytes, value = byte * k_scale /
    v_scale."""
    dt = _DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    kvt = _KV_DTYPES[kv_dtype] if isinstance(kv_dtype, str) else int(kv_dtype)
    return PdaShape(int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_size),
                    int(block_size), int(num_blocks), int(max_blocks_per_seq), int(max_seq_len),
                    dt, int(sliding_window), int(q_len), kvt, float(k_scale), float(v_scale))


def shape_from_tensors(q, k_cache, block_table, max_seq_len: int,
                       sliding_window: int = 0, k_scale: float = 1.0,
                       v_scale: float = 1.0) -> PdaShape:
    """q is [B, Hq, D] (one query row per sequence) or [B, q_len, Hq, D];
    k_cache of q's dtype, or float8_e4m3fn with per-tensor scales."""
    import torch
    if q.dim() == 3:
        B, Hq, D = q.shape
        q_len = 1
    elif q.dim() == 4:
        B, q_len, Hq, D = q.shape
    else:
        raise ValueError("q must be [B, Hq, D] or [B, q_len, Hq, D]")
    NB, Hkv, bs, D2 = k_cache.shape
    if D2 != D:
        raise ValueError("head size of q and k_cache differ")
    dt = {torch.bfloat16: "bf16", torch.float16: "fp16"}.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    kvt = "fp8" if k_cache.dtype == torch.float8_e4m3fn else "same"
    return make_shape(B, Hq, Hkv, D, bs, NB, block_table.shape[1], max_seq_len, dt,
                      sliding_window, q_len, kvt, k_scale, v_scale)


def pda_status_string(status: int) -> str:
    return load_library().pda_status_string(int(status)).decode()


def pda_build_id() -> str:
    return load_library().pda_build_id().decode()


def pda_check_shape(shape: PdaShape) -> int:
    return int(load_library().pda_check_shape(ctypes.byref(shape)))


def pda_plan_for_cus(shape: PdaShape, cu_count: int) -> PdaPlan:
    plan = PdaPlan()
    rc = load_library().pda_plan_for_cus(ctypes.byref(shape), int(cu_count), ctypes.byref(plan))
    if rc != PDA_OK:
        raise PdaError(rc, "pda_plan_for_cus")
    return plan


def paged_decode_attn_plan(shape: PdaShape) -> PdaPlan:
    plan = PdaPlan()
    rc = load_library().paged_decode_attn_plan(ctypes.byref(shape), ctypes.byref(plan))
    if rc != PDA_OK:
        raise PdaError(rc, "paged_decode_attn_plan")
    return plan


def paged_decode_attn_workspace_size(shape: PdaShape) -> int:
    n = int(load_library().paged_decode_attn_workspace_size(ctypes.byref(shape)))
    if n < 0:
        raise PdaError(n, "paged_decode_attn_workspace_size")
    return n


def pda_workspace_bytes(shape: PdaShape, plan: PdaPlan) -> int:
    return int(load_library().pda_workspace_bytes(ctypes.byref(shape), ctypes.byref(plan)))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        # the raw handle of torch's current stream on the current device;
        # torch.cuda.current_stream() builds a Stream object for it, which
        # took 2.7 us per call, a third of a short decode call's host time
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return raw(torch.cuda.current_device())
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


_TENSOR_NAMES = ("q", "k_cache", "v_cache", "block_table", "seq_lens", "out")


def _check_tensors(q, k_cache, v_cache, block_table, seq_lens, out):
    import torch
    ts = (q, k_cache, v_cache, block_table, seq_lens, out)
    # the library launches on the current device: every buffer must be a
    # contiguous tensor there (get_device() is -1 for a host tensor)
    dev = q.get_device()
    ok = dev >= 0
    for t in ts:
        ok = ok and t.get_device() == dev and t.is_contiguous()
    if not ok or dev != torch.cuda.current_device():
        for name, t in zip(_TENSOR_NAMES, ts):
            if not t.is_cuda:
                raise ValueError(f"{name} must be a device tensor")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        if any(t.get_device() != dev for t in ts):
            raise ValueError("q, k_cache, v_cache, block_table, seq_lens and out must share one "
                             "device")
        raise ValueError("the tensors must be on the current device")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if q.dtype != out.dtype or k_cache.dtype != v_cache.dtype:
        raise ValueError("q and out, and k_cache and v_cache, must share one dtype")
    if k_cache.dtype not in (q.dtype, torch.float8_e4m3fn):
        raise ValueError("k_cache/v_cache must have q's dtype or be float8_e4m3fn")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    if seq_lens.shape != (q.shape[0],) or block_table.shape[0] != q.shape[0]:
        raise ValueError("seq_lens / block_table do not match the batch")


# The shape descriptor and the device plan's workspace size of recent calls,
# by the tensors' geometry: a decode loop calls with the same geometry every
# step, and building the descriptor and querying the plan cost more host
# time than the rest of the binding.  The descriptors are private (passed by
# reference to the library only, never handed out).
_SHAPE_CACHE = {}
_SHAPE_CACHE_MAX = 256


def _shape_and_workspace(q, k_cache, block_table, max_seq_len, sliding_window, k_scale,
                         v_scale):
    key = (q.get_device(), q.shape, q.dtype, k_cache.shape, k_cache.dtype, block_table.shape[1],
           max_seq_len, sliding_window, k_scale, v_scale)
    hit = _SHAPE_CACHE.get(key)
    if hit is None:
        shape = shape_from_tensors(q, k_cache, block_table, max_seq_len, sliding_window, k_scale,
                                   v_scale)
        if len(_SHAPE_CACHE) >= _SHAPE_CACHE_MAX:
            _SHAPE_CACHE.clear()
        hit = _SHAPE_CACHE[key] = (shape, paged_decode_attn_workspace_size(shape))
    return hit


def paged_decode_attn(q, k_cache, v_cache, block_table, seq_lens, scale: float, out=None,
                      workspace=None, max_seq_len: Optional[int] = None, plan: Optional[PdaPlan] = None,
                      stream=None, sliding_window: int = 0, k_scale: float = 1.0,
                      v_scale: float = 1.0):
    """Decode the query rows of each sequence over the paged KV cache.

    q [B, Hq, D] (one row per sequence) or [B, q_len, Hq, D] (q_len rows at
    the sequence's last q_len positions, causal among themselves),
    k_cache/v_cache [NB, Hkv, bs, D] (q's bf16/fp16 dtype, or float8_e4m3fn
    with per-tensor scales k_scale / v_scale),
    block_table [B, MBS] int32, seq_lens [B] int32, all on the current device.
    max_seq_len must bound every seq_lens entry (default: block_table width *
    block size, which is always valid but may over-partition).
    sliding_window W > 0 attends to the last W tokens only.  Returns `out`.
    """
    import torch
    if out is None:
        out = torch.empty_like(q)
    _check_tensors(q, k_cache, v_cache, block_table, seq_lens, out)
    if max_seq_len is None:
        max_seq_len = block_table.shape[1] * k_cache.shape[2]
    shape, need = _shape_and_workspace(q, k_cache, block_table, max_seq_len, sliding_window,
                                       k_scale, v_scale)
    lib = load_library()
    if plan is not None:
        need = pda_workspace_bytes(shape, plan)
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous() or
                                  workspace.get_device() != q.get_device()):
        raise ValueError("workspace must be a contiguous tensor on q's device")
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)  # zeroed, as required
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if plan is None:
        rc = lib.paged_decode_attn(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(block_table), _ptr(seq_lens), float(scale), _ptr(out),
                                   _ptr(workspace), ws_bytes, _stream(stream))
    else:
        rc = lib.paged_decode_attn_with_plan(ctypes.byref(shape), ctypes.byref(plan), _ptr(q),
                                             _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                             _ptr(seq_lens), float(scale), _ptr(out),
                                             _ptr(workspace), ws_bytes, _stream(stream))
    if rc != PDA_OK:
        raise PdaError(rc, "paged_decode_attn")
    return out


def paged_decode_attn_with_plan(q, k_cache, v_cache, block_table, seq_lens, scale: float,
                                plan: PdaPlan, out=None, workspace=None,
                                max_seq_len: Optional[int] = None, stream=None,
                                sliding_window: int = 0, k_scale: float = 1.0,
                                v_scale: float = 1.0):
    return paged_decode_attn(q, k_cache, v_cache, block_table, seq_lens, scale, out=out,
                             workspace=workspace, max_seq_len=max_seq_len, plan=plan,
                             stream=stream, sliding_window=sliding_window, k_scale=k_scale,
                             v_scale=v_scale)


PDA_NOALLOC_MAX_WORKSPACE = 64 * 1024 * 1024


def paged_decode_attn_noalloc(q, k_cache, v_cache, block_table, seq_lens, scale: float, out,
                              max_seq_len: Optional[int] = None, stream=None,
                              sliding_window: int = 0, k_scale: float = 1.0,
                              v_scale: float = 1.0):
    """paged_decode_attn into a caller's `out` with the library's static
    per-GPU workspace: allocates nothing (no torch allocation either).
    Raises PdaError (PDA_ERR_WORKSPACE) when the device plan's workspace
    exceeds PDA_NOALLOC_MAX_WORKSPACE.  Calls overlapping on one GPU race."""
    _check_tensors(q, k_cache, v_cache, block_table, seq_lens, out)
    if max_seq_len is None:
        max_seq_len = block_table.shape[1] * k_cache.shape[2]
    shape = shape_from_tensors(q, k_cache, block_table, max_seq_len, sliding_window, k_scale,
                               v_scale)
    rc = load_library().paged_decode_attn_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(seq_lens), float(scale), _ptr(out), _stream(stream))
    if rc != PDA_OK:
        raise PdaError(rc, "paged_decode_attn_noalloc")
    return out


def paged_decode_attn_workspace_init(workspace, stream=None):
    """Zero a workspace tensor on the stream (needed once before its first use)."""
    nbytes = workspace.numel() * workspace.element_size()
    rc = load_library().paged_decode_attn_workspace_init(_ptr(workspace), nbytes, _stream(stream))
    if rc != PDA_OK:
        raise PdaError(rc, "paged_decode_attn_workspace_init")


def paged_decode_attn_workspace_check(workspace, stream=None) -> int:
    """Number of non-zero arrival counters in a workspace, after the work on
    the stream (0 unless a fused call started on counters that were not
    zero).  Synchronises the stream: a validation aid, not for the hot path."""
    nbytes = workspace.numel() * workspace.element_size()
    n = ctypes.c_int32(0)
    rc = load_library().paged_decode_attn_workspace_check(_ptr(workspace), nbytes,
                                                          _stream(stream), ctypes.byref(n))
    if rc != PDA_OK:
        raise PdaError(rc, "paged_decode_attn_workspace_check")
    return int(n.value)


def pda_read_probe(src, sink, workgroups: int = 2048, stream=None):
    """HBM streaming-read probe: read the device tensor `src` once and XOR
    its 32-bit words into the int32 device tensor `sink` (one element,
    zeroed by the caller).  Asynchronous on the stream."""
    nbytes = src.numel() * src.element_size()
    rc = load_library().pda_read_probe(_ptr(src), nbytes, _ptr(sink), int(workgroups),
                                       _stream(stream))
    if rc != PDA_OK:
        raise PdaError(rc, "pda_read_probe")


def paged_decode_attn_timed(shape: PdaShape, plan: Optional[PdaPlan], q, k_cache, v_cache,
                            block_table, seq_lens, scale: float, out, workspace,
                            start_event=None, stop_event=None, stream=None):
    """Low-level instrumented call for benchmarks: no argument conversion,
    pre-allocated `out` / `workspace`; start_event / stop_event are
    torch.cuda.Event objects (already recorded once, so they exist) that the
    library attaches to the split-KV kernel's own start and end."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ev0 = None if start_event is None else start_event.cuda_event
    ev1 = None if stop_event is None else stop_event.cuda_event
    rc = load_library().paged_decode_attn_timed(
        ctypes.byref(shape), None if plan is None else ctypes.byref(plan), _ptr(q),
        _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), float(scale),
        _ptr(out), _ptr(workspace), ws_bytes, ev0, ev1, _stream(stream))
    if rc != PDA_OK:
        raise PdaError(rc, "paged_decode_attn_timed")


def paged_decode_attn_trace(shape: PdaShape, plan: PdaPlan, block_table, seq_lens,
                            rows: int = 0, stream=None, fill: int = -1):
    """Run the bookkeeping trace of the plan's variant (rows 0: the rows its K
    loads read, 1: its V loads); returns (slot [B,Hkv,Lmax], part [B,Hkv,Lmax],
    ranges [B,Hkv,P,2]) as int32 device tensors pre-filled with `fill`."""
    import torch
    dev = block_table.device
    B, Hkv, Lmax, P = shape.num_seqs, shape.num_kv_heads, shape.max_seq_len, plan.num_partitions
    slot = torch.full((B, Hkv, max(Lmax, 1)), fill, dtype=torch.int32, device=dev)
    part = torch.full_like(slot, fill)
    ranges = torch.full((B, Hkv, P, 2), fill, dtype=torch.int32, device=dev)
    rc = load_library().paged_decode_attn_trace(ctypes.byref(shape), ctypes.byref(plan),
                                                int(rows), _ptr(block_table), _ptr(seq_lens),
                                                _ptr(slot),
                                                _ptr(part), _ptr(ranges), _stream(stream))
    if rc != PDA_OK:
        raise PdaError(rc, "paged_decode_attn_trace")
    return slot, part, ranges

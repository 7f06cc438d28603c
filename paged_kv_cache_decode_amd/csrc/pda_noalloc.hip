// The decode step for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): paged_decode_attn_noalloc runs the same kernels under the same
// device plan as paged_decode_attn, but its workspace -- the fused merge's
// arrival counters and the fp32 split-KV partials -- is `scratch`, a
// file-scope device array of PDA_NOALLOC_MAX_WORKSPACE bytes that every GPU
// the library runs on holds until the process ends.
//
// Host code never passes the array's name to a kernel: in host code that
// name is a host-side stand-in, not a device address.  The device address is
// obtained once per device with hipGetSymbolAddress, with that device
// current, and kept per device; the kernels receive that pointer as they
// receive a caller's workspace.
#include <mutex>

#include "pda_common.h"

namespace pda {

static __device__ __align__(256) char scratch[PDA_NOALLOC_MAX_WORKSPACE];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch`, per device

// The device address of this device's `scratch`.  On a device's first call:
// resolve the address, and zero the array's counter block with a fill kernel
// on `stream` (the counters must be zero when a fused call starts; every
// completed fused call leaves them zero again, so later calls find them so).
int scratch_for_device(hipStream_t stream, void** ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
        return PDA_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return PDA_ERR_DEVICE;
        if (launch_zero_fill(p, (int64_t)PDA_FUSED_MAX_UNITS * 4, stream) != hipSuccess)
            return PDA_ERR_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PDA_OK;
}

}  // namespace
}  // namespace pda

extern "C" int paged_decode_attn_noalloc(const pda_shape_t* shape, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         const int32_t* block_table, const int32_t* seq_lens,
                                         float scale, void* out, void* stream) {
    int rc = pda_check_shape(shape);
    if (rc != PDA_OK) return rc;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return PDA_ERR_INVALID;
    pda_plan_t plan;
    rc = paged_decode_attn_plan(shape, &plan);
    if (rc != PDA_OK) return rc;
    // checked before the array is touched, so an oversized call changes nothing
    if (plan.workspace_bytes > (int64_t)PDA_NOALLOC_MAX_WORKSPACE) return PDA_ERR_WORKSPACE;
    void* ws = nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (plan.workspace_bytes > 0) {
        rc = pda::scratch_for_device(st, &ws);
        if (rc != PDA_OK) return rc;
    }
    return pda::run_decode(shape, &plan, q, k_cache, v_cache, block_table, seq_lens, scale, out,
                           ws, plan.workspace_bytes, stream, nullptr, nullptr);
}

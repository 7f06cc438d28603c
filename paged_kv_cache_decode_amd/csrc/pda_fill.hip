// Zero fill of a caller's workspace, for gfx950: a plain kernel of vector
// stores (16 bytes per thread and step when the buffer allows, else single
// bytes), so that a caller may capture it into a HIP graph (a memset node is
// avoided there).
#include "pda_common.h"

namespace pda {

__global__ __launch_bounds__(256) void zero_fill16_kernel(uint4* dst, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * 256)
        dst[i] = make_uint4(0u, 0u, 0u, 0u);
}

__global__ __launch_bounds__(256) void zero_fill1_kernel(uint8_t* dst, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = 0;
}

hipError_t launch_zero_fill(void* dst, int64_t bytes, hipStream_t stream) {
    const bool wide = reinterpret_cast<uintptr_t>(dst) % 16 == 0 && bytes % 16 == 0;
    const int64_t items = wide ? bytes / 16 : bytes;
    const int64_t wgs = (items + 255) / 256;
    const dim3 grid((unsigned)(wgs < 1024 ? (wgs > 0 ? wgs : 1) : 1024));
    if (wide)
        hipLaunchKernelGGL(zero_fill16_kernel, grid, dim3(256), 0, stream,
                           static_cast<uint4*>(dst), items);
    else
        hipLaunchKernelGGL(zero_fill1_kernel, grid, dim3(256), 0, stream,
                           static_cast<uint8_t*>(dst), items);
    return hipGetLastError();
}

}  // namespace pda

// HBM streaming-read probe, for gfx950: the achievable read bandwidth that
// the decode kernels' roofline fraction is read against.  Not part of the
// decode.
//
// Every 16-byte chunk of the buffer is read exactly once, with the same
// non-temporal 16-byte loads the decode kernels use for K/V rows, in a
// grid-stride loop: workgroup w, thread t reads chunks (w * 256 + t) +
// k * (grid * 256) in batches of kUnroll independent loads.  The 32-bit words
// are folded with XOR (an order-independent checksum, so the compiler keeps
// every load and a test can check the result exactly); each workgroup adds
// its part to `sink` with one atomic XOR.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pda.h"

namespace pda {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int kUnroll>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4_t* __restrict__ src,
                                                         int64_t chunks, uint32_t* sink) {
    __shared__ uint32_t part[4];
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < chunks; i += stride * kUnroll) {
        u32x4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + u * stride;
            v[u] = j < chunks ? __builtin_nontemporal_load(src + j) : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // fold the wave, then the four waves, in registers and LDS
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) atomicXor(sink, part[0] ^ part[1] ^ part[2] ^ part[3]);
}

}  // namespace pda

extern "C" int pda_read_probe(const void* src, int64_t bytes, void* sink, int32_t workgroups,
                              void* stream) {
    if (!src || !sink || bytes < 16 || bytes % 16 != 0 || workgroups < 1 ||
        workgroups > (1 << 20))
        return PDA_ERR_INVALID;
    hipLaunchKernelGGL(pda::read_probe_kernel<8>, dim3(workgroups), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const pda::u32x4_t*>(src),
                       bytes / 16, static_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? PDA_OK : PDA_ERR_LAUNCH;
}

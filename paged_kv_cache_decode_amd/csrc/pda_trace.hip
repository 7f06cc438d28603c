// Bookkeeping trace of the paged decode, for gfx950.
//
// Same grid, partition bounds, table staging, tile walk and token location
// (ValuGeom, stage_table_slice, locate_token) as the decode kernel, but each
// lane that would load a token row records which physical slot and which
// partition it used, instead of loading it.  Tests compare the trace bit for
// bit with a recomputation from the definition of the paged cache.
#include "pda_device.h"

namespace pda {

template <int D, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void trace_kernel(DecodeParams p) {
    using Geo = ValuGeom<D>;
    constexpr int LPT = Geo::LPT, R = Geo::R, U = Geo::U, TT = Geo::TT;
    extern __shared__ int32_t tbl[];
    const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c = lane % LPT, r = lane / LPT;
    const int L = context_len(p, b);
    const int t0 = part * p.tokens_per_part;
    const int t1 = min(t0 + p.tokens_per_part, L);
    const int64_t unit = (int64_t)b * p.num_kv_heads + g;
    if (threadIdx.x == 0) {
        p.trace_range[(unit * p.num_partitions + part) * 2] = t0;
        p.trace_range[(unit * p.num_partitions + part) * 2 + 1] = t1;
    }
    if (t0 >= L) return;
    const int lb0 = (int)fastdiv((uint32_t)t0, p.bs_div);
    const int lb1 = (int)fastdiv((uint32_t)(t1 - 1), p.bs_div);
    stage_table_slice(p, b, lb0, lb1, tbl);
    __syncthreads();
    const int ntiles = (t1 - t0 + TT - 1) / TT;
    for (int j = wave; j < ntiles; j += kWaves) {
        const int tile_base = t0 + j * TT;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int phys, slot0, dt;
            locate_token<R, ALIGNED>(p, tbl, lb0, tile_base, t1, u, r, phys, slot0, dt);
            const int t = tile_base + u * R + r;
            if (c == 0 && t < t1) {
                const int64_t at = unit * p.max_seq_len + t;
                p.trace_slot[at] = phys * p.block_size + slot0 + dt;
                p.trace_part[at] = part;
            }
        }
    }
}

template <int D, bool ALIGNED>
static hipError_t launch_trace_t(const DecodeParams& p, int batch, hipStream_t stream) {
    const dim3 grid(p.num_partitions, p.num_kv_heads, batch);
    hipLaunchKernelGGL((trace_kernel<D, ALIGNED>), grid, dim3(kThreads),
                       (size_t)p.tbl_capacity * sizeof(int32_t), stream, p);
    return hipGetLastError();
}

hipError_t launch_trace(int head_size, bool aligned, const DecodeParams& p, int batch,
                        hipStream_t stream) {
    switch (head_size) {
        case 64: return aligned ? launch_trace_t<64, true>(p, batch, stream)
                                : launch_trace_t<64, false>(p, batch, stream);
        case 128: return aligned ? launch_trace_t<128, true>(p, batch, stream)
                                 : launch_trace_t<128, false>(p, batch, stream);
        case 256: return aligned ? launch_trace_t<256, true>(p, batch, stream)
                                 : launch_trace_t<256, false>(p, batch, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pda

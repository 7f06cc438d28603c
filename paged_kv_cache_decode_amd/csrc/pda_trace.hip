// Bookkeeping trace of the paged decode, for gfx950.
//
// Same grid, partition bounds, table staging, tile walk and row location
// (stage_table_slice, locate_token / locate_row and the lane-to-row maps of
// ValuGeom and MfmaGeom) as the decode kernels -- on the aligned path also
// the blocks of each wave's first two tiles from the table entries loaded
// before the context length is known (first_tile_entries /
// first_tile_blocks) -- but each lane that would load a token row records
// which physical slot and which partition it used, instead of loading it.
// ROWS selects whose rows: 0 the VALU kernel's (K and V alike), 1 the MFMA
// kernel's K rows (whole-row loads of KB-byte elements), 2 its V rows.  Tests
// compare the
// trace bit for bit with a recomputation from the definition of the paged
// cache.
#include "pda_device.h"

namespace pda {

template <int D, int KB, bool ALIGNED, int ROWS>
__global__ __launch_bounds__(kThreads) void trace_kernel(DecodeParams p) {
    using Geo = ValuGeom<D>;
    constexpr int LPT = Geo::LPT, R = Geo::R, U = Geo::U;
    constexpr int TT = ROWS == 0 ? Geo::TT : 16;
    extern __shared__ int32_t tbl[];
    // grid (Hkv, B, P): the partition index varies slowest (see the launcher)
    const int g = blockIdx.x, b = blockIdx.y, part = blockIdx.z;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c = lane % LPT, r = lane / LPT;
    const int32_t* trow = p.block_table + (int64_t)b * p.max_blocks_per_seq;
    FirstTiles ft{{0, 0}, {0, 0}};
    if constexpr (ALIGNED) ft = first_tile_entries(p, trow, part, wave, TT);
    const SeqRange rg = seq_range(p, b);
    const int L = rg.L;
    const int t0 = rg.base + part * p.tokens_per_part;
    const int t1 = min(t0 + p.tokens_per_part, L);
    const int64_t unit = (int64_t)b * p.num_kv_heads + g;
    if (threadIdx.x == 0) {
        p.trace_range[(unit * p.num_partitions + part) * 2] = t0;
        p.trace_range[(unit * p.num_partitions + part) * 2 + 1] = t1;
    }
    if (t0 >= L) return;
    const int lb0 = (int)fastdiv((uint32_t)t0, p.bs_div);
    const int lb1 = (int)fastdiv((uint32_t)(t1 - 1), p.bs_div);
    if (!ALIGNED) {
        stage_table_slice(p, b, lb0, lb1, tbl);
        __syncthreads();
    }
    const int32_t* tv = table_view<ALIGNED>(p, b, tbl);
    const int tlb0 = ALIGNED ? 0 : lb0;
    const int ntiles = (t1 - t0 + TT - 1) / TT;
    // the decode kernels' buffer-load choice on the aligned path: always for
    // the matrix-core kernel, for one packed row in the VALU kernel
    const bool buf = ALIGNED && (ROWS != 0 || p.rows == 1);
    TileBlock first[2] = {{0, 0}, {0, 0}};
    if constexpr (ALIGNED)
        first_tile_blocks(p, trow, ft, part, wave, TT, rg, t0, ntiles, buf, first);
    // the row a lane would load at in-tile offset o of tile j: the first two
    // tiles of the wave from the early entries, the rest looked up
    auto locate = [&](int j, int tile_base, int o, int& phys, int& slot0, int& dt) {
        if (ALIGNED && (j == wave || j == wave + kWaves)) {
            const TileBlock& tb = first[j == wave ? 0 : 1];
            phys = tb.phys;
            slot0 = tb.slot0;
            dt = tile_row(tile_base, rg.lo, t1, o);
        } else {
            locate_row<ALIGNED>(p, tv, tlb0, tile_base, rg.lo, t1, o, phys, slot0, dt);
        }
    };
    auto record = [&](int t, int phys, int slot) {
        const int64_t at = unit * p.max_seq_len + t;
        p.trace_slot[at] = phys * p.block_size + slot;
        p.trace_part[at] = part;
    };
    for (int j = wave; j < ntiles; j += kWaves) {
        const int tile_base = t0 + j * TT;
        int phys, slot0, dt;
        if constexpr (ROWS == 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                locate(j, tile_base, u * R + r, phys, slot0, dt);
                const int t = tile_base + u * R + r;
                if (c == 0 && t >= rg.lo && t < t1) record(t, phys, slot0 + dt);
            }
        } else if constexpr (ROWS == 1) {
            if (mfma_k_whole_rows(D, KB, p.tokens_per_part, (int64_t)p.num_kv_heads * gridDim.y)) {
                constexpr int LPT = KB * D / 16, KL = 16 / (64 / LPT);
#pragma unroll
                for (int s = 0; s < KL; ++s) {
                    const int o = mfma_k_token(lane, s, LPT);
                    locate(j, tile_base, o, phys, slot0, dt);
                    const int t = tile_base + o;
                    if (lane % LPT == 0 && t >= rg.lo && t < t1) record(t, phys, slot0 + dt);
                }
            } else {
                const int o = mfma_k_offset(lane);
                locate(j, tile_base, o, phys, slot0, dt);
                const int t = tile_base + o;
                if ((lane >> 4) == 0 && t >= rg.lo && t < t1) record(t, phys, slot0 + dt);
            }
        } else {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int o = mfma_v_offset(lane, rr);
                locate(j, tile_base, o, phys, slot0, dt);
                const int t = tile_base + o;
                if ((lane & 15) == 0 && t >= rg.lo && t < t1) record(t, phys, slot0 + dt);
            }
        }
    }
}

template <int D, int KB, bool ALIGNED, int ROWS>
static hipError_t launch_trace_t(const DecodeParams& p, int batch, hipStream_t stream) {
    // Workgroups are dispatched in grid order, partition by partition: the
    // empty partitions of shorter sequences come after the live partitions of
    // every sequence instead of between them, where each one measured to cost
    // tens of ns of the whole launch (mixed lengths at batch 64: 16% faster).
    const dim3 grid(p.num_kv_heads, batch, p.num_partitions);
    hipLaunchKernelGGL((trace_kernel<D, KB, ALIGNED, ROWS>), grid, dim3(kThreads),
                       (size_t)p.tbl_capacity * sizeof(int32_t), stream, p);
    return hipGetLastError();
}

template <int D, int KB>
static hipError_t launch_trace_d(bool aligned, int rows, const DecodeParams& p, int batch,
                                 hipStream_t s) {
    if (aligned) {
        if (rows == 0) return launch_trace_t<D, KB, true, 0>(p, batch, s);
        if (rows == 1) return launch_trace_t<D, KB, true, 1>(p, batch, s);
        return launch_trace_t<D, KB, true, 2>(p, batch, s);
    }
    if (rows == 0) return launch_trace_t<D, KB, false, 0>(p, batch, s);
    if (rows == 1) return launch_trace_t<D, KB, false, 1>(p, batch, s);
    return launch_trace_t<D, KB, false, 2>(p, batch, s);
}

template <int KB>
static hipError_t launch_trace_kb(int head_size, bool aligned, int rows, const DecodeParams& p,
                                  int batch, hipStream_t stream) {
    switch (head_size) {
        case 64: return launch_trace_d<64, KB>(aligned, rows, p, batch, stream);
        case 128: return launch_trace_d<128, KB>(aligned, rows, p, batch, stream);
        case 256: return launch_trace_d<256, KB>(aligned, rows, p, batch, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_trace(int head_size, int kv_elt_bytes, bool aligned, int rows,
                        const DecodeParams& p, int batch, hipStream_t stream) {
    return kv_elt_bytes == 1 ? launch_trace_kb<1>(head_size, aligned, rows, p, batch, stream)
                             : launch_trace_kb<2>(head_size, aligned, rows, p, batch, stream);
}

}  // namespace pda

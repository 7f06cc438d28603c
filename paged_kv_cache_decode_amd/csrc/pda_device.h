// Device-side building blocks shared by the decode, trace and merge kernels:
// 16-bit element traits, wavefront reductions, and the block-table
// bookkeeping (token -> physical block and slot) that the trace kernel checks
// bit for bit against an independent recomputation.
#pragma once

#include <float.h>
#include <math.h>

#include "pda_common.h"

namespace pda {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

struct BF16 {
    // sum += a.x*b.x + a.y*b.y on packed pairs (v_dot2_f32_bf16)
    __device__ static inline float dot2(uint32_t a, uint32_t b, float sum) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, b), sum, false);
    }
    __device__ static inline float lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ static inline float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
    __device__ static inline uint16_t from_float(float x) {
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));  // round to nearest even
    }
};

struct FP16 {
    __device__ static inline float dot2(uint32_t a, uint32_t b, float sum) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                      __builtin_bit_cast(f16x2_t, b), sum, false);
    }
    __device__ static inline float lo(uint32_t w) {
        return (float)__builtin_bit_cast(f16x2_t, w).x;
    }
    __device__ static inline float hi(uint32_t w) {
        return (float)__builtin_bit_cast(f16x2_t, w).y;
    }
    __device__ static inline uint16_t from_float(float x) {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));  // round to nearest even
    }
};

// ---- DPP lane exchanges (within 16-lane rows) --------------------------
enum : int {
    kDppXor1 = 0xB1,         // quad_perm [1,0,3,2]
    kDppXor2 = 0x4E,         // quad_perm [2,3,0,1]
    kDppRowHalfMirror = 0x141,
    kDppRowMirror = 0x140,
};

template <int CTRL>
__device__ inline float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in 2..64, power of two); every lane
// of a group receives the group's sum.  Within a row the partner patterns are
// xor 1, xor 2, then the half-row and row mirrors (which pair lane i with a
// lane of the other quad / other half); across rows a lane shuffle.
template <int N>
__device__ inline float group_sum(float x) {
    static_assert(N >= 2 && N <= 64 && (N & (N - 1)) == 0, "group size");
    x += dpp<kDppXor1>(x);
    if constexpr (N >= 4) x += dpp<kDppXor2>(x);
    if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}

// ---- VALU tile geometry --------------------------------------------------
// One lane loads 16 bytes (8 elements) of a token row, so a row of D
// elements spans LPT = D/8 lanes and a wavefront covers R = 64/LPT tokens per
// load instruction.  A tile is U such rounds.
template <int D>
struct ValuGeom {
    static constexpr int LPT = D / 8;
    static constexpr int R = kWave / LPT;
    static constexpr int U = (D == 256) ? 4 : kTile / R;
    static constexpr int TT = U * R;   // tokens per tile: 16 (D 64/128) or 8 (D 256)
};

__host__ __device__ constexpr int valu_tile_tokens(int head_size) {
    return head_size == 256 ? 8 : 16;
}

// ---- block-table bookkeeping --------------------------------------------
// The partition's slice of the sequence's block-table row is staged in LDS:
// entries for logical blocks lb0 .. lb1 of tokens [t0, t1).
__device__ inline void stage_table_slice(const DecodeParams& p, int b, int lb0, int lb1,
                                         int32_t* tbl) {
    const int32_t* row = p.block_table + (int64_t)b * p.max_blocks_per_seq;
    for (int j = threadIdx.x; j <= lb1 - lb0; j += blockDim.x) tbl[j] = row[lb0 + j];
}

// Context length of sequence b as the kernels use it: seq_lens[b] clamped to
// [0, max_seq_len], so an out-of-contract length cannot drive an access past
// the block-table row or the workspace.
__device__ inline int context_len(const DecodeParams& p, int b) {
    return max(0, min(p.seq_lens[b], p.max_seq_len));
}

// Physical block and slot of the token that round u, lane-row r of the tile
// starting at tile_base reads.  Tokens at or past t1 (the partition end,
// never past the sequence end) are redirected to token t1-1, so no slot at or
// past seq_len is ever addressed.  Block ids are clamped into the pool, so a
// corrupt table entry gives a wrong row, never an access outside the pool.
//  ALIGNED (block size a multiple of the tile): the whole tile lies in one
//  block, located once per tile; the lane adds its row offset.
//  Otherwise every lane divides its own token index by the block size.
template <int R, bool ALIGNED>
__device__ inline void locate_token(const DecodeParams& p, const int32_t* tbl, int lb0,
                                    int tile_base, int t1, int u, int r, int& phys, int& slot) {
    const int rel = min(u * R + r, t1 - 1 - tile_base);
    if constexpr (ALIGNED) {
        const int lb = (int)fastdiv((uint32_t)tile_base, p.bs_div);
        slot = tile_base - lb * p.block_size + rel;
        phys = __builtin_amdgcn_readfirstlane(tbl[lb - lb0]);
        phys = min(max(phys, 0), p.num_blocks - 1);
    } else {
        const int t = tile_base + rel;
        const int lb = (int)fastdiv((uint32_t)t, p.bs_div);
        slot = t - lb * p.block_size;
        phys = min(max(tbl[lb - lb0], 0), p.num_blocks - 1);
    }
}

}  // namespace pda

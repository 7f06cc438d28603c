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

// 2^x with the hardware instruction (v_exp_f32).  Arguments here are
// differences of scores from a running max, so they are <= 0; -inf gives 0,
// and results below the smallest normal flush to 0, which only drops weights
// under 2^-126 of the largest one.
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16 bytes of a K/V row.  The cache is streamed once per call, so the load
// carries the non-temporal hint (measured ~6% faster on MI355X).
#ifndef PDA_VALU_NT
#define PDA_VALU_NT 1
#endif
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline uint4 load_row16(const char* ptr) {
#if PDA_VALU_NT
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ptr));
#else
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ptr);
#endif
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Device-scope (all XCDs) store and load of fp32 workspace data: the store
// is written through to the device coherence point (sc1), the load reads
// from it, so partials written by one workgroup can be read by another on a
// different XCD without flushing or invalidating the L2.
__device__ inline void store_coherent(float* ptr, float v) {
    __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_coherent(const float* ptr) {
    return __hip_atomic_load(const_cast<float*>(ptr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's outstanding memory operations (its device-scope
// stores included) have completed; also a compiler barrier for memory.
__device__ inline void wait_stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---- DPP lane exchanges (within 16-lane rows) --------------------------
enum : int {
    kDppXor1 = 0xB1,         // quad_perm [1,0,3,2]
    kDppXor2 = 0x4E,         // quad_perm [2,3,0,1]
    kDppRowHalfMirror = 0x141,
    kDppRowMirror = 0x140,
};

// Every lane has a valid source in these patterns, so bound_ctrl is moot;
// setting it lets the compiler fold the move into the consuming add
// (v_add_f32 with a DPP operand).
template <int CTRL>
__device__ inline float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
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
// load instruction (a "round").  A tile is U rounds, TT = U*R tokens.
// Rounds per tile, chosen by measurement on MI355X: two rounds (a 1 KB load
// per wave and tensor per round) with two tiles in flight beat deeper tiles,
// which raise register pressure without raising bandwidth.
#ifndef PDA_VALU_ROUNDS_64
#define PDA_VALU_ROUNDS_64 2
#endif
#ifndef PDA_VALU_ROUNDS_128
#define PDA_VALU_ROUNDS_128 2
#endif
#ifndef PDA_VALU_ROUNDS_256
#define PDA_VALU_ROUNDS_256 2
#endif
template <int D>
struct ValuGeom {
    static constexpr int LPT = D / 8;
    static constexpr int R = kWave / LPT;
    static constexpr int U = D == 64 ? PDA_VALU_ROUNDS_64
                           : D == 128 ? PDA_VALU_ROUNDS_128 : PDA_VALU_ROUNDS_256;
    static constexpr int TT = U * R;
};

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
// starting at tile_base reads: slot = slot0 + dt.  Tokens at or past t1 (the
// partition end, never past the sequence end) are redirected to token t1-1,
// so no slot at or past seq_len is ever addressed.  Block ids are clamped
// into the pool, so a corrupt table entry gives a wrong row, never an access
// outside the pool.
//  ALIGNED (block size a multiple of 16): the round's tokens lie in one block
//  (R divides 16 and rounds start at multiples of R), located once per round
//  from the round's first (clamped) token: phys and slot0 are wave-uniform,
//  dt in [0, R) is the lane's row offset.
//  Otherwise every lane divides its own token index by the block size and
//  dt = 0.
template <int R, bool ALIGNED>
__device__ inline void locate_token(const DecodeParams& p, const int32_t* tbl, int lb0,
                                    int tile_base, int t1, int u, int r, int& phys, int& slot0,
                                    int& dt) {
    const int last = t1 - 1 - tile_base;
    const int t = tile_base + min(u * R + r, last);
    if constexpr (ALIGNED) {
        const int ub = tile_base + min(u * R, last);
        const int lb = (int)fastdiv((uint32_t)ub, p.bs_div);
        slot0 = ub - lb * p.block_size;
        dt = t - ub;
        phys = __builtin_amdgcn_readfirstlane(tbl[lb - lb0]);
        phys = min(max(phys, 0), p.num_blocks - 1);
    } else {
        const int lb = (int)fastdiv((uint32_t)t, p.bs_div);
        slot0 = t - lb * p.block_size;
        dt = 0;
        phys = min(max(tbl[lb - lb0], 0), p.num_blocks - 1);
    }
}

}  // namespace pda

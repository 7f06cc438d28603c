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

// ---- fp8 E4M3 (OCP) KV bytes -------------------------------------------
// Two E4M3 bytes of w (bytes 0 and 1, or 2 and 3 with HI) -> two elements of
// the 16-bit type in one instruction (v_cvt_scalef32_pk_{bf16,f16}_fp8 with
// scale 1), low byte to the low half.  The conversion is exact: every E4M3
// value, subnormals included, is a bf16 and an fp16 value (checked against
// the conversion through fp32 on all 256 codes).
template <typename Elt, bool HI>
__device__ inline uint32_t fp8x2_to_16bit(uint32_t w);
template <>
__device__ inline uint32_t fp8x2_to_16bit<BF16, false>(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
template <>
__device__ inline uint32_t fp8x2_to_16bit<BF16, true>(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
template <>
__device__ inline uint32_t fp8x2_to_16bit<FP16, false>(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
template <>
__device__ inline uint32_t fp8x2_to_16bit<FP16, true>(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// 8 E4M3 bytes -> 8 elements of the 16-bit type, exactly
template <typename Elt>
__device__ inline uint4 fp8x8_to_16bit(uint32_t w0, uint32_t w1) {
    return make_uint4(fp8x2_to_16bit<Elt, false>(w0), fp8x2_to_16bit<Elt, true>(w0),
                      fp8x2_to_16bit<Elt, false>(w1), fp8x2_to_16bit<Elt, true>(w1));
}

// Byte transpose of four 32-bit words: out[e] holds byte e of x0, x1, x2, x3
// in its bytes 0, 1, 2, 3 (v_perm_b32 picks byte k of the 64-bit {hi, lo} for
// selector value k: 0-3 from lo, 4-7 from hi).
__device__ inline void byte_transpose4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                       uint32_t (&out)[4]) {
    const uint32_t a = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // x0.b0 x1.b0 x0.b1 x1.b1
    const uint32_t b = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // x0.b2 x1.b2 x0.b3 x1.b3
    const uint32_t c = __builtin_amdgcn_perm(x3, x2, 0x05010400u);  // x2.b0 x3.b0 x2.b1 x3.b1
    const uint32_t d = __builtin_amdgcn_perm(x3, x2, 0x07030602u);  // x2.b2 x3.b2 x2.b3 x3.b3
    out[0] = __builtin_amdgcn_perm(c, a, 0x05040100u);  // a.b0 a.b1 c.b0 c.b1
    out[1] = __builtin_amdgcn_perm(c, a, 0x07060302u);  // a.b2 a.b3 c.b2 c.b3
    out[2] = __builtin_amdgcn_perm(d, b, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(d, b, 0x07060302u);
}

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

// The same 16 bytes at base + off through a buffer resource.  `base` must be
// wave-uniform (it rides in scalar registers); `off` is the lane's byte
// offset.  With `valid` false the resource holds no records, so the load
// returns zeros without touching memory: the software pipelines use it to
// prefetch "tiles" past the end with no traffic and no extra latency, keeping
// every load in the loop unconditional (a guarded load or an early exit makes
// the compiler drain all outstanding loads at the loop head).
// Word 3 of the resource: 32-bit data format, as raw buffer loads need.
constexpr int kBufferWord3 = 0x00020000;
__device__ inline uint4 load_row16_buf(const char* base, uint32_t off, bool valid) {
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base), (short)0, valid ? 0x7fffffff : 0, kBufferWord3);
#if PDA_VALU_NT
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 2);  // nt
#else
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
#endif
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 8 bytes of a row (an fp8 V chunk), plain and through a buffer resource
// (same contract as load_row16 / load_row16_buf).
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint2 load_row8(const char* ptr) {
#if PDA_VALU_NT
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(ptr));
#else
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(ptr);
#endif
    return make_uint2(v.x, v.y);
}
__device__ inline uint2 load_row8_buf(const char* base, uint32_t off, bool valid) {
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base), (short)0, valid ? 0x7fffffff : 0, kBufferWord3);
#if PDA_VALU_NT
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, off, 0, 2);  // nt
#else
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, off, 0, 0);
#endif
    return make_uint2(v.x, v.y);
}

// 4 bytes of a row (an fp8 V chunk at head size 64), plain and through a
// buffer resource (same contract as load_row16 / load_row16_buf).
__device__ inline uint32_t load_row4(const char* ptr) {
#if PDA_VALU_NT
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ptr));
#else
    return *reinterpret_cast<const uint32_t*>(ptr);
#endif
}
__device__ inline uint32_t load_row4_buf(const char* base, uint32_t off, bool valid) {
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base), (short)0, valid ? 0x7fffffff : 0, kBufferWord3);
#if PDA_VALU_NT
    return __builtin_amdgcn_raw_buffer_load_b32(rsrc, off, 0, 2);  // nt
#else
    return __builtin_amdgcn_raw_buffer_load_b32(rsrc, off, 0, 0);
#endif
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
// A buffer resource over `base`, made wave-uniform with readfirstlane (a
// lane-varying resource would make the compiler loop over the lanes' distinct
// values); `base` must be the same for every lane of the wave.
constexpr int kBufferSc1 = 16;  // cache-policy bit sc1 of a buffer access: device scope
__device__ inline __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    // each half through uint32_t: the builtin returns int, and a low half
    // with bit 31 set would otherwise sign-extend into the high half
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((hi << 32) | lo), (short)0,
                                             0x7fffffff, kBufferWord3);
}
// N = 2 or 4 consecutive floats stored at base + off (byte offset, 8N-byte
// aligned) at device scope in one access: written through to the point where
// every XCD sees them, like store_coherent, but as one 8- or 16-byte store
// rather than N 4-byte ones (each of which costs a memory write of its own).
template <int N>
__device__ inline void store_coherent_vec(float* base, uint32_t off, const float* v) {
    static_assert(N == 2 || N == 4, "8- or 16-byte stores");
    if constexpr (N == 4) {
        const u32x4_t w = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                           __float_as_uint(v[3])};
        __builtin_amdgcn_raw_buffer_store_b128(w, uniform_rsrc(base), off, 0, kBufferSc1);
    } else {
        const u32x2_t w = {__float_as_uint(v[0]), __float_as_uint(v[1])};
        __builtin_amdgcn_raw_buffer_store_b64(w, uniform_rsrc(base), off, 0, kBufferSc1);
    }
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

// ---- exchanges across the four 16-lane rows ------------------------------
// gfx950's v_permlane16_swap / v_permlane32_swap exchange whole 16-lane rows
// between two registers in the VALU, without the LDS round trip of a lane
// shuffle (ds_bpermute).  With both operands x, the pair returned holds in
// every lane x and the value of the lane X apart: first own and second the
// partner's where (lane & X) == 0, the other way round elsewhere.
struct RowPair {
    float a, b;
};
template <int X>
__device__ inline RowPair row_swap(float x) {
    static_assert(X == 16 || X == 32, "row swaps exchange lanes 16 or 32 apart");
    const uint32_t u = __float_as_uint(x);
    if constexpr (X == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return RowPair{__uint_as_float(r[0]), __uint_as_float(r[1])};
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return RowPair{__uint_as_float(r[0]), __uint_as_float(r[1])};
    }
}
// The value of lane (lane ^ X), X = 16 or 32.
template <int X>
__device__ inline float xor_lane(float x) {
    const RowPair r = row_swap<X>(x);
    return (threadIdx.x & X) == 0 ? r.b : r.a;
}
// max and sum over lanes l and l ^ X (the same value in both lanes; a sum is
// own + partner, up to the order of two terms, which does not change it)
template <int X>
__device__ inline float max_xor(float x) {
    const RowPair r = row_swap<X>(x);
    return fmaxf(r.a, r.b);
}
template <int X>
__device__ inline float sum_xor(float x) {
    const RowPair r = row_swap<X>(x);
    return r.a + r.b;
}

// Sum over aligned groups of N lanes (N in 2..64, power of two); every lane
// of a group receives the group's sum.  Within a row the partner patterns are
// xor 1, xor 2, then the half-row and row mirrors (which pair lane i with a
// lane of the other quad / other half); across rows the row swaps.
template <int N>
__device__ inline float group_sum(float x) {
    static_assert(N >= 2 && N <= 64 && (N & (N - 1)) == 0, "group size");
    x += dpp<kDppXor1>(x);
    if constexpr (N >= 4) x += dpp<kDppXor2>(x);
    if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
    if constexpr (N >= 32) x = sum_xor<16>(x);
    if constexpr (N >= 64) x = sum_xor<32>(x);
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
// The block-table view locate_row takes: for ALIGNED kernels the global row
// of sequence b (scalar loads, lb0 = 0); otherwise the LDS slice, which the
// caller stages with stage_table_slice and publishes with a barrier.
template <bool ALIGNED>
__device__ inline const int32_t* table_view(const DecodeParams& p, int b, const int32_t* lds) {
    return ALIGNED ? p.block_table + (int64_t)b * p.max_blocks_per_seq : lds;
}

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

// Tokens of sequence b the decode attends to.  With n = q_len query rows,
// row i attends to [lo_i, e_i), e_i = L - n + i + 1 (causal among the new
// rows; e_{n-1} = L), lo_i = max(0, e_i - W) for a sliding window W > 0,
// else 0.  The unit reads [lo, L) with lo = lo_0, the smallest; its
// partitions tile [base, L) with base = lo rounded down to the 16-token grid,
// so that aligned tiles keep starting on it; rows in [base, lo) are
// redirected to lo (tile_row) and their scores are masked, so no slot before
// the window is ever read.  end0 = e_0 and lo_last = lo_{n-1} bound the
// tiles every row takes whole (full_tile).
// seq_range_of takes the raw seq_lens entry, loaded by the caller.
struct SeqRange {
    int L, lo, base, end0, lo_last;
};
__device__ inline SeqRange seq_range_of(const DecodeParams& p, int raw_len) {
    const int L = max(0, min(raw_len, p.max_seq_len));
    const int end0 = L - p.q_len + 1;
    const int lo = p.window > 0 ? max(0, end0 - p.window) : 0;
    const int lo_last = p.window > 0 ? max(0, L - p.window) : 0;
    return SeqRange{L, lo, lo & ~(kAlignTokens - 1), end0, lo_last};
}
__device__ inline SeqRange seq_range(const DecodeParams& p, int b) {
    return seq_range_of(p, p.seq_lens[b]);
}

// Tokens [lo, end) of query row position i (see SeqRange).
struct RowRange {
    int lo, end;
};
__device__ inline RowRange row_range(const DecodeParams& p, const SeqRange& rg, int i) {
    const int end = rg.end0 + i;
    return RowRange{p.window > 0 ? max(0, end - p.window) : 0, end};
}
// Whether every row attends to every token of [tile_base, tile_base + tt)
// (tokens below t1, the partition end): no score of the tile needs a mask.
__device__ inline bool full_tile(const SeqRange& rg, int tile_base, int tt, int t1) {
    return tile_base >= rg.lo_last && tile_base + tt <= min(t1, rg.end0);
}

// Row r of a unit (b, g) packs query position i = r / G and head h = r % G;
// its index among the [B][q_len][Hq] rows of q, out and the partials.
__device__ inline int64_t row_index(const DecodeParams& p, int b, int g, int r) {
    const int i = r / p.group, h = r - i * p.group;
    return ((int64_t)b * p.q_len + i) * p.num_q_heads + g * p.group + h;
}

// A compiler barrier for memory operations, emitting no instruction and no
// wait: the loads issued before it stay before it.  The decode kernels issue
// their context-independent loads (query rows, first table entries) ahead of
// the branch on the context length with it; left alone, the compiler sinks
// them past that branch, behind the seq_lens round trip.
__device__ inline void issue_fence() { asm volatile("" ::: "memory"); }
// The same for scalar loads of constant memory (table entries), which the
// fence does not hold: a use in place keeps them, together with the seq_lens
// load.  It waits for the three values, as the context-length branch after
// it would wait for seq_lens alone: the scalar loads are in flight together.
__device__ inline void keep_issued(int len, int e0, int e1) {
    asm volatile("" ::"s"(len), "s"(e0), "s"(e1));
}

// Partitions of a unit that hold tokens (the rest are empty).
__device__ inline int live_partitions(const DecodeParams& p, const SeqRange& r) {
    return min(p.num_partitions, (r.L - r.base + p.tokens_per_part - 1) / p.tokens_per_part);
}

// The block of the aligned path's tile that starts at tile_base (a multiple
// of 16 tokens or of the round length, with the block size a multiple of 16):
// every row a wave reads with that tile lies in the tile's 16-token group,
// hence in this block.  `row` is the sequence's block-table row in global
// memory, read with a scalar load (wave-uniform index: no staging, no barrier,
// no vector register).  The index does not depend on the context length, so
// the first tiles' entries can be loaded while the length is still in flight;
// it is clamped into the row, so a tile past the end (a prefetch that loads
// nothing) reads an entry inside the row.  Block ids are clamped into the
// pool, so a corrupt entry gives a wrong row, never an access outside the
// pool.
struct TileBlock {
    int phys, slot0;
};
__device__ inline int tile_table_index(const DecodeParams& p, int tile_base) {
    return min((int)fastdiv((uint32_t)tile_base, p.bs_div), p.max_blocks_per_seq - 1);
}
__device__ inline int table_entry(const int32_t* row, int lb) {
    typedef const __attribute__((address_space(4))) int32_t* const_i32p;
    return ((const_i32p)row)[lb];  // address-space cast: C-style only
}
__device__ inline TileBlock tile_block_of(const DecodeParams& p, int entry, int lb, int tile_base) {
    return TileBlock{min(max(entry, 0), p.num_blocks - 1), tile_base - lb * p.block_size};
}
__device__ inline TileBlock tile_block(const DecodeParams& p, const int32_t* row, int tile_base) {
    const int lb = tile_table_index(p, tile_base);
    return tile_block_of(p, table_entry(row, lb), lb, tile_base);
}

// A wave's first two tiles on the aligned path: tile `wave` and tile
// `wave + kWaves` of partition `part` (tt tokens each).  The decode kernels
// load their table entries together with seq_lens, before the context length
// is known, at the positions the tiles have when the partition grid starts at
// token 0 (first_tile_entries).  Once the length is known, first_tile_blocks
// keeps those entries unless a sliding window moved the grid (base != 0) or,
// without buffer loads, a tile lies past the end (such a prefetch re-reads
// the last tile); otherwise it looks the blocks up again.  The trace kernel
// takes the same two steps, so the bit-exact trace covers the early loads.
struct FirstTiles {
    int lb[2];  // logical block indices (clamped into the row)
    int e[2];   // their table entries
};
__device__ inline FirstTiles first_tile_entries(const DecodeParams& p, const int32_t* row,
                                                int part, int wave, int tt) {
    FirstTiles f;
    const int ts = part * p.tokens_per_part + wave * tt;
    f.lb[0] = tile_table_index(p, ts);
    f.lb[1] = tile_table_index(p, ts + kWaves * tt);
    f.e[0] = table_entry(row, f.lb[0]);
    f.e[1] = table_entry(row, f.lb[1]);
    return f;
}
__device__ inline void first_tile_blocks(const DecodeParams& p, const int32_t* row,
                                         const FirstTiles& f, int part, int wave, int tt,
                                         const SeqRange& rg, int t0, int ntiles, bool buf,
                                         TileBlock (&first)[2]) {
    const int ts = part * p.tokens_per_part + wave * tt;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const int jj = wave + st * kWaves;
        if (rg.base != 0 || (!buf && jj >= ntiles))
            first[st] = tile_block(p, row, t0 + (buf ? jj : min(jj, ntiles - 1)) * tt);
        else
            first[st] = tile_block_of(p, f.e[st], f.lb[st], ts + st * kWaves * tt);
    }
}

// In-tile offset of the row a lane reads for in-tile offset o: tokens at or
// past t1 (the partition end, never past the sequence end) are redirected to
// token t1-1, and tokens before lo (the first token attended to) to lo, so no
// slot past seq_len or before a sliding window is ever addressed.
__device__ inline int tile_row(int tile_base, int lo, int t1, int o) {
    return min(max(o, lo - tile_base), t1 - 1 - tile_base);
}

// Physical block and slot of the row a lane reads, slot = slot0 + dt (rows
// redirected as in tile_row).
//  ALIGNED: phys and slot0 are those of the tile (tile_block), wave-uniform;
//  dt is the lane's row offset.  `tbl` is the sequence's block-table row in
//  global memory (lb0 = 0).
//  Otherwise `tbl` is the LDS copy of the slice starting at block lb0, every
//  lane divides its own token index by the block size and dt = 0.
template <bool ALIGNED>
__device__ inline void locate_row(const DecodeParams& p, const int32_t* tbl, int lb0,
                                  int tile_base, int lo, int t1, int o, int& phys, int& slot0,
                                  int& dt) {
    const int ot = tile_row(tile_base, lo, t1, o);
    if constexpr (ALIGNED) {
        const TileBlock tb = tile_block(p, tbl, tile_base);
        phys = tb.phys;
        slot0 = tb.slot0;
        dt = ot;
    } else {
        const int t = tile_base + ot;
        const int lb = (int)fastdiv((uint32_t)t, p.bs_div);
        slot0 = t - lb * p.block_size;
        dt = 0;
        phys = min(max(tbl[lb - lb0], 0), p.num_blocks - 1);
    }
}

// The VALU kernel's rows: round u of a tile, lane-row r (R rows per round;
// R divides 16 and rounds start at multiples of R).
template <int R, bool ALIGNED>
__device__ inline void locate_token(const DecodeParams& p, const int32_t* tbl, int lb0,
                                    int tile_base, int lo, int t1, int u, int r, int& phys,
                                    int& slot0, int& dt) {
    locate_row<ALIGNED>(p, tbl, lb0, tile_base, lo, t1, u * R + r, phys, slot0, dt);
}

// ---- MFMA tile geometry --------------------------------------------------
// A 16-token tile.  K rows feed the A operand of v_mfma_f32_16x16x32 (S^T =
// K Q^T): lane l holds token l%16, elements 32s + 8(l/16) .. +8 for k-step s.
// V rows feed the A operand of v_mfma_f32_16x16x16 (O^T = V^T P^T): for
// round r lane l reads token 4(l/16) + r, elements dh*128 + VE*(l%16) .. +VE,
// VE = 8 (16 lanes cover a 128-wide half dh) or 4 at D 64 (16 lanes cover
// the row), so the 16 d-rows of every PV product are distinct columns.
template <int D>
struct MfmaGeom {
    static constexpr int KS = D / 32;                 // QK k-steps (16-byte K loads per tile)
    static constexpr int DH = D >= 128 ? D / 128 : 1; // 128-wide halves of V
    static constexpr int VE = D >= 128 ? 8 : 4;       // V elements per lane and round
};
// K rows are loaded whole: a row of RB bytes spans LPT = RB/16 lanes, so load
// s of a tile gives lane l bytes 16*(l % LPT) .. +16 of token s*(64/LPT) +
// l/LPT (every instruction reads whole 128-byte lines).  The tile then moves
// through a per-wave LDS buffer of 16 rows, RB + 16 bytes apart, into the
// A-operand layout above (lane l: token l%16, bytes 64s + 16(l/16) .. +16).
__device__ inline int mfma_k_token(int lane, int s, int lpt) { return s * (64 / lpt) + lane / lpt; }
// The token a lane loads when K is loaded in the operand layout directly
// (mfma_k_whole_rows false): token l%16, bytes 64s + 16(l/16) for load s.
__device__ inline int mfma_k_offset(int lane) { return lane & 15; }
__device__ inline int mfma_v_offset(int lane, int r) { return 4 * (lane >> 4) + r; }


// ---- unit epilogue shared by the decode kernels ------------------------
// Combine the kWaves per-wave states of rows h0 .. h0+hn-1 of unit (b, g),
// staged in LDS as red[w][i][0..D) = unnormalised O, red[w][i][D] = running
// max m (exp2 domain), red[w][i][D+1] = denominator l (red_heads rows per
// wave, hn <= min(red_heads, kThreads / TPR)), in a fixed order, and write
// either the 16-bit output (one partition) or the fp32 partial.  TPR threads
// per row (32: 8 rows at a time; 16: 16 rows at a time); thread j of a row
// takes the element pairs d = 2j + 2*TPR*k (k < D/(2*TPR)), so a row's
// threads read 2*TPR consecutive floats of LDS per pair (8 consecutive
// elements per thread put threads 4 apart on the same banks) and write
// 8*TPR contiguous bytes of output or partials per pair and row.
// All LDS reads of the step are issued before any arithmetic.  WT: partials
// for the merge kernel are written through to the device coherence point
// (device-scope stores), leaving no dirty L2 lines for the end of the launch
// to write back (measured faster for the matrix-core kernel, slightly slower
// for the VALU one).
template <typename Elt, int D, bool WT, int TPR = 32>
__device__ inline void write_unit_rows(const DecodeParams& p, const float* red, int red_heads,
                                       int h0, int hn, int b, int g, int part) {
    constexpr int KP = D / (2 * TPR);  // element pairs per thread
    static_assert((TPR == 16 || TPR == 32) && KP >= 1 && kThreads % TPR == 0, "rows of threads");
    // one pass serves every row its callers stage: up to kHeadChunk rows at
    // 32 threads per row, up to 16 at 16
    static_assert(kThreads / TPR >= (TPR == 32 ? kHeadChunk : 16), "a thread row per staged row");
    const int i = threadIdx.x / TPR, j = threadIdx.x % TPR;
    if (i >= hn) return;
    // every LDS read of the step first: the waves' (m, l) and the row's pairs
    float mw[kWaves], lw[kWaves];
    float2 vw[kWaves][KP];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float* rw = red + (w * red_heads + i) * lds_row_floats(D);
        mw[w] = rw[D];
        lw[w] = rw[D + 1];
#pragma unroll
        for (int k = 0; k < KP; ++k)
            vw[w][k] = *reinterpret_cast<const float2*>(rw + 2 * j + 2 * TPR * k);
    }
    float M = -FLT_MAX;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mw[w]);
    float wt[kWaves], den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        wt[w] = fast_exp2(mw[w] - M);
        den += lw[w] * wt[w];
    }
    // a row with no token in this partition (a causal row ending before it)
    // has den == 0: its normalised partial is 0, and its weight l = 0 keeps
    // it out of the merge.  v_scale (1 for 16-bit KV) dequantises fp8 V; the
    // merge is linear in o, so it applies to partials too.
    const float f = den > 0.f ? p.v_scale / den : 0.f;
    float2 o[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) o[k] = make_float2(0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            o[k].x += vw[w][k].x * wt[w];
            o[k].y += vw[w][k].y * wt[w];
        }
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        o[k].x *= f;
        o[k].y *= f;
    }
    const int64_t row = row_index(p, b, g, h0 + i);
    if (p.num_partitions == 1) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.out) + row * D);
#pragma unroll
        for (int k = 0; k < KP; ++k)
            dst[j + TPR * k] = (uint32_t)Elt::from_float(o[k].x) |
                              ((uint32_t)Elt::from_float(o[k].y) << 16);
        return;
    }
    const int64_t prow = row * p.num_partitions + part;
    if (p.fused_merge || WT) {  // read back by another workgroup of this launch, or written through
        const int64_t row0 = row_index(p, b, g, 0);
        const int64_t span = (row_index(p, b, g, p.rows - 1) - row0 + 1) * p.num_partitions * D * 4;
        if (span < ((int64_t)1 << 31)) {
            const int64_t prel = (row - row0) * p.num_partitions + part;
            float* obase = p.ws_o + row0 * p.num_partitions * D;
            const uint32_t off = (uint32_t)((prel * D + 2 * j) * 4);
#pragma unroll
            for (int k = 0; k < KP; ++k) {
                const float v2[2] = {o[k].x, o[k].y};
                store_coherent_vec<2>(obase, off + 8 * TPR * k, v2);
            }
            if (j == 0) {
                const float mlv[2] = {M, den};
                store_coherent_vec<2>(p.ws_ml + row0 * p.num_partitions * 2, (uint32_t)(prel * 8), mlv);
            }
        } else {
            float* dst = p.ws_o + prow * D;
#pragma unroll
            for (int k = 0; k < KP; ++k) {
                store_coherent(dst + 2 * j + 2 * TPR * k, o[k].x);
                store_coherent(dst + 2 * j + 2 * TPR * k + 1, o[k].y);
            }
            if (j == 0) {
                store_coherent(p.ws_ml + prow * 2, M);
                store_coherent(p.ws_ml + prow * 2 + 1, den);
            }
        }
    } else {              // read by the merge kernel after this launch
        float2* dst = reinterpret_cast<float2*>(p.ws_o + prow * D);
#pragma unroll
        for (int k = 0; k < KP; ++k) dst[j + TPR * k] = o[k];
        if (j == 0) reinterpret_cast<float2*>(p.ws_ml)[prow] = make_float2(M, den);
    }
}

// Log-sum-exp merge of the Pb partials (o_p normalised, m_p, l_p in the exp2
// domain) of the R rows of unit (b, g):
//   out = sum_p l_p 2^(m_p - M) o_p / sum_p l_p 2^(m_p - M),  M = max_p m_p
// (0 for a row with no token at all), partitions summed in index order.
// Every load of a step is issued before any is used: first all (m, l) pairs
// of the unit, from which one thread per row forms the weights in LDS; then
// each thread loads all Pb partials of four consecutive elements of a row
// (16-byte device-scope loads) and sums them.  Up to kMergePairs (row,
// partition) pairs; beyond that, one element per thread and step with a
// running max.
constexpr int kMergePairs = 1024;
constexpr int kMergeUnroll = 16;  // partitions whose loads are in flight together

// 16 bytes of the workspace at base + off (16-byte aligned), read at device
// scope (sc1: not from a possibly stale L2 line) through a buffer resource.
// `base` must be wave-uniform (it is made so: a lane-varying resource would
// make the compiler loop over the lanes' distinct values).
__device__ inline float4 load_coherent16(const float* base, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(uniform_rsrc(base), off, 0, kBufferSc1);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                       __uint_as_float(v.w));
}

// 8 bytes of the workspace at base + off (8-byte aligned), read like
// load_coherent16.
__device__ inline float2 load_coherent8(const float* base, uint32_t off) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(uniform_rsrc(base), off, 0, kBufferSc1);
    return make_float2(__uint_as_float(v.x), __uint_as_float(v.y));
}

#ifndef PDA_FUSED_ONE_TRIP
#define PDA_FUSED_ONE_TRIP 1
#endif

// The fused merge in one memory round trip (up to U = kMergeUnroll partitions):
// each thread takes four consecutive elements of one row and issues the
// loads of every partition's (m, l) pair and of its four partial elements
// together, then forms the weights itself (every thread of a row the same
// ones): M = max over p, w_p = l_p 2^(m_p - M), the sums over p in index
// order, times 1 / sum w_p -- the rule of merge_unit below, with no LDS
// step and no barrier between the two kinds of loads.
template <typename Elt, int D, int U>
__device__ inline void merge_unit_one_trip(const DecodeParams& p, int b, int g, int Pb) {
    constexpr int D4 = D / 4;
    uint16_t* out16 = static_cast<uint16_t*>(p.out);
    const int R = p.rows, P = p.num_partitions;
    const int64_t row0 = row_index(p, b, g, 0);
    const float* obase = p.ws_o + row0 * P * D;
    const float* mbase = p.ws_ml + row0 * P * 2;
    for (int it = threadIdx.x; it < R * D4; it += blockDim.x) {
        const int i = it / D4, c = it - i * D4;
        const int64_t rrel = row_index(p, b, g, i) - row0;
        const uint32_t ooff = (uint32_t)((rrel * P * D + 4 * c) * sizeof(float));
        const uint32_t moff = (uint32_t)(rrel * P * 2 * sizeof(float));
        float2 ml[U];
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = min(u, Pb - 1);  // past Pb: re-read the last, never used
            ml[u] = load_coherent8(mbase, moff + (uint32_t)(q * 2 * sizeof(float)));
            v[u] = load_coherent16(obase, ooff + (uint32_t)(q * D * sizeof(float)));
        }
        float M = -FLT_MAX;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < Pb) M = fmaxf(M, ml[u].x);
        float den = 0.f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = u < Pb ? ml[u].y * fast_exp2(ml[u].x - M) : 0.f;
            if (u < Pb) den += w;
            acc.x += w * v[u].x; acc.y += w * v[u].y;
            acc.z += w * v[u].z; acc.w += w * v[u].w;
        }
        const float f = den > 0.f ? 1.f / den : 0.f;
        uint16_t* dst = out16 + (row0 + rrel) * D + 4 * c;
        dst[0] = Elt::from_float(acc.x * f);
        dst[1] = Elt::from_float(acc.y * f);
        dst[2] = Elt::from_float(acc.z * f);
        dst[3] = Elt::from_float(acc.w * f);
    }
}

template <typename Elt, int D>
__device__ void merge_unit(const DecodeParams& p, int b, int g, int Pb) {
    __shared__ float s_w[kMergePairs];
    __shared__ float s_f[PDA_MAX_ROWS];
    uint16_t* out16 = static_cast<uint16_t*>(p.out);
    const int R = p.rows, P = p.num_partitions;
    // byte span of the unit's partials from its first row: the 16-byte loads
    // take 32-bit offsets from that row
    const int64_t span = (row_index(p, b, g, R - 1) - row_index(p, b, g, 0) + 1) * P * D * 4;
    if (R * Pb > kMergePairs || span >= ((int64_t)1 << 31)) {
        for (int idx = threadIdx.x; idx < R * D; idx += blockDim.x) {
            const int i = idx / D, d = idx - i * D;
            const int64_t row = row_index(p, b, g, i);
            const float* ml = p.ws_ml + row * P * 2;
            const float* po = p.ws_o + row * P * D + d;
            float M = -FLT_MAX, o = 0.f, den = 0.f;
            for (int q = 0; q < Pb; ++q) {
                const float mq = load_coherent(ml + 2 * q), lq = load_coherent(ml + 2 * q + 1);
                const float oq = load_coherent(po + (int64_t)q * D);
                const float mn = fmaxf(M, mq);
                const float sc = fast_exp2(M - mn);
                const float w = lq * fast_exp2(mq - mn);
                o = o * sc + w * oq;
                den = den * sc + w;
                M = mn;
            }
            out16[row * D + d] = Elt::from_float(den > 0.f ? o / den : 0.f);
        }
        return;
    }
    // (m, l) of every (row, partition) pair: s_w holds m, then the weight
    constexpr int KP = (kMergePairs + kThreads - 1) / kThreads;
    float lv[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int idx = threadIdx.x + k * kThreads;
        if (idx < R * Pb) {
            const int i = idx / Pb, q = idx - i * Pb;
            const float* ml = p.ws_ml + (row_index(p, b, g, i) * P + q) * 2;
            s_w[idx] = load_coherent(ml);
            lv[k] = load_coherent(ml + 1);
        }
    }
    __syncthreads();
    if (threadIdx.x < R) {  // the row's max, held in s_f for the next step
        float M = -FLT_MAX;
        for (int q = 0; q < Pb; ++q) M = fmaxf(M, s_w[threadIdx.x * Pb + q]);
        s_f[threadIdx.x] = M;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KP; ++k) {  // each pair's m is read and replaced by its own thread
        const int idx = threadIdx.x + k * kThreads;
        if (idx < R * Pb) s_w[idx] = lv[k] * fast_exp2(s_w[idx] - s_f[idx / Pb]);
    }
    __syncthreads();
    if (threadIdx.x < R) {  // the row's normalisation, sums in partition order
        float den = 0.f;
        for (int q = 0; q < Pb; ++q) den += s_w[threadIdx.x * Pb + q];
        s_f[threadIdx.x] = den > 0.f ? 1.f / den : 0.f;
    }
    __syncthreads();
    constexpr int D4 = D / 4;
    // partials of the unit's first row: the wave-uniform base of the loads
    const int64_t row0 = row_index(p, b, g, 0);
    const float* base = p.ws_o + row0 * P * D;
    for (int it = threadIdx.x; it < R * D4; it += blockDim.x) {
        const int i = it / D4, c = it - i * D4;
        const int64_t row = row_index(p, b, g, i);
        const uint32_t off0 = (uint32_t)(((row - row0) * P * D + 4 * c) * sizeof(float));
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int q0 = 0; q0 < Pb; q0 += kMergeUnroll) {
            float4 v[kMergeUnroll];
#pragma unroll
            for (int u = 0; u < kMergeUnroll; ++u) {
                const int q = min(q0 + u, Pb - 1);  // past Pb: re-read the last, weight 0
                v[u] = load_coherent16(base, off0 + (uint32_t)(q * D * sizeof(float)));
            }
#pragma unroll
            for (int u = 0; u < kMergeUnroll; ++u) {
                const float w = q0 + u < Pb ? s_w[i * Pb + q0 + u] : 0.f;
                acc.x += w * v[u].x; acc.y += w * v[u].y;
                acc.z += w * v[u].z; acc.w += w * v[u].w;
            }
        }
        const float f = s_f[i];
        uint16_t* dst = out16 + row * D + 4 * c;
        dst[0] = Elt::from_float(acc.x * f);
        dst[1] = Elt::from_float(acc.y * f);
        dst[2] = Elt::from_float(acc.z * f);
        dst[3] = Elt::from_float(acc.w * f);
    }
}

// Fused split-KV merge: the unit that finishes last among the Pb non-empty
// partitions of (b, g) merges them.  The partials were stored at device scope
// (write-through to the point where all XCDs see them); each wave waits for
// its stores to be acknowledged before the workgroup barrier, then thread 0
// counts the arrival with a device-scope atomic.  The last arrival resets the
// counter for the next call and reads the partials back with device-scope
// loads.  No L2 write-back or invalidate is needed.
#ifndef PDA_FUSED_ACQREL
#define PDA_FUSED_ACQREL 0
#endif
template <typename Elt, int D>
__device__ inline void fused_merge_tail(const DecodeParams& p, const SeqRange& rg, int b,
                                        int g) {
    __shared__ int s_last;
    wait_stores_done();
    __syncthreads();
    const int Pb = live_partitions(p, rg);
    if (threadIdx.x == 0) {
        int32_t* ctr = p.counters + (int64_t)b * p.num_kv_heads + g;
#if PDA_FUSED_ACQREL
        const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
#else
        const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#endif
        s_last = old == Pb - 1;
        if (s_last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
#if PDA_FUSED_ONE_TRIP
    const int64_t span = (row_index(p, b, g, p.rows - 1) - row_index(p, b, g, 0) + 1) *
                         p.num_partitions * D * 4;
    if (Pb <= kMergeUnroll && span < ((int64_t)1 << 31)) {
        merge_unit_one_trip<Elt, D, kMergeUnroll>(p, b, g, Pb);
        return;
    }

#endif
    merge_unit<Elt, D>(p, b, g, Pb);
}

// Zero output rows of the R rows of (b, g) (an empty context).
template <int D>
__device__ inline void zero_unit_rows(const DecodeParams& p, int b, int g) {
    uint16_t* out16 = static_cast<uint16_t*>(p.out);
    for (int idx = threadIdx.x; idx < p.rows * D; idx += blockDim.x) {
        const int i = idx / D, d = idx - i * D;
        out16[row_index(p, b, g, i) * D + d] = 0;
    }
}

}  // namespace pda

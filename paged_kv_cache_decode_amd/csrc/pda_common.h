// Shared definitions of the gfx950 paged-decode library: kernel parameter
// block, fast division by the (runtime) block size, and the launcher
// declarations the host runtime calls.  Internal to libpda.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pda.h"

namespace pda {

// Unsigned division by a runtime constant d >= 1 for dividends n < 2^31,
// by the round-up multiply-high method of Granlund and Montgomery
// ("Division by invariant integers using multiplication", 1994):
//   l = ceil(log2 d),  m = floor(2^32 * (2^l - d) / d) + 1,
//   n / d = (mulhi(n, m) + n) >> l.
// mulhi(n, m) < n, so the sum fits in 32 bits for n < 2^31.  Used to split a
// token index into (logical block, slot) for any block size, including ones
// that are not powers of two (784 = 16 x 49).
struct FastDiv {
    uint32_t d;
    uint32_t mul;
    uint32_t shift;
};

__host__ __device__ inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    f.shift = l;
    f.mul = (uint32_t)((((1ull << l) - d) << 32) / d + 1ull);
    return f;
}

__host__ __device__ inline uint32_t fastdiv(uint32_t n, const FastDiv& f) {
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t hi = __umulhi(n, f.mul);
#else
    uint32_t hi = (uint32_t)(((uint64_t)n * f.mul) >> 32);
#endif
    return (hi + n) >> f.shift;
}

// Everything one decode launch needs; passed by value as the kernel argument.
struct DecodeParams {
    // what a decode workgroup needs first (its first table entries and the
    // context length) fills the first 64 bytes, which one scalar load brings
    const void* q;             // [B][q_len][Hq][D]
    const int32_t* block_table;// [B][MBS]
    const int32_t* seq_lens;   // [B]
    int32_t tokens_per_part;   // T_p
    int32_t max_blocks_per_seq;// MBS
    FastDiv bs_div;
    int32_t group;             // G = Hq / Hkv
    int32_t num_q_heads;       // Hq
    int32_t max_seq_len;       // host bound on seq_lens (also the trace row length)
    int32_t window;            // sliding window W (0: whole context)
    int32_t q_len;             // query rows per sequence (1: plain decode)
    const void* k_cache;       // [NB][Hkv][bs][D]
    const void* v_cache;       // [NB][Hkv][bs][D]
    void* out;                 // [B][q_len][Hq][D]
    float* ws_o;               // [B][q_len][Hq][P][D]    (P > 1 only)
    float* ws_ml;              // [B][q_len][Hq][P][2]    (P > 1 only)
    int32_t* counters;         // arrival counters (fused merge), entry b * Hkv + g
    int32_t* trace_slot;       // trace kernel only
    int32_t* trace_part;
    int32_t* trace_range;
    float scale_log2;          // scale * log2(e): scores live in the exp2 domain
    int32_t num_kv_heads;      // Hkv
    int32_t block_size;        // bs
    int32_t num_partitions;    // P
    int32_t tbl_capacity;      // LDS entries reserved for the block-table slice
    int32_t fused_merge;       // 1: the last unit of each (b, g) merges the partials
    int32_t num_blocks;        // NB: block ids are clamped into [0, NB)
    int32_t rows;              // R = q_len * G rows per unit
    float v_scale;             // fp8 V scale (1 for 16-bit KV); k_scale is in scale_log2
    int32_t lds_floor;         // dynamic LDS of the decode launch is at least this (bytes)
    int64_t block_stride;      // Hkv * bs * D elements
    int32_t head_stride;       // bs * D elements
};
static_assert(offsetof(DecodeParams, q_len) + sizeof(int32_t) <= 64,
              "the start-up fields fit one 64-byte scalar load");

constexpr int kWave = 64;
// Wavefronts per workgroup of the decode kernels (tiles of a partition are
// dealt to them round-robin).
#ifndef PDA_KERNEL_WAVES
#define PDA_KERNEL_WAVES 4
#endif
constexpr int kWaves = PDA_KERNEL_WAVES;
constexpr int kTile = PDA_TILE;
constexpr int kAlignTokens = 16;
constexpr int kThreads = kWave * kWaves;

// Heads are combined in chunks of at most this many through LDS at the end
// of a unit.
constexpr int kHeadChunk = 8;

// Launchers (one translation unit per element type and head size).
// `aligned` selects the path for block sizes that are multiples of the tile.
// start/stop: optional events bracketing the decode kernel (hipExtLaunchKernel)
hipError_t launch_decode_valu(int dtype, int head_size, int group_pad, bool aligned,
                              const DecodeParams& p, int batch, hipStream_t stream,
                              hipEvent_t start, hipEvent_t stop);
hipError_t launch_decode_mfma(int dtype, int head_size, bool aligned, const DecodeParams& p,
                              int batch, hipStream_t stream, hipEvent_t start, hipEvent_t stop);
hipError_t launch_merge(int dtype, int head_size, const DecodeParams& p, int batch,
                        hipStream_t stream);
// zero `bytes` at device pointer `dst` with a fill kernel on `stream`
hipError_t launch_zero_fill(void* dst, int64_t bytes, hipStream_t stream);
// rows: 0 = the VALU kernel's rows, 1 = the MFMA kernel's K rows, 2 = its V
// rows; kv_elt_bytes (1 for fp8 KV, else 2) sets the MFMA K rows' lane map
hipError_t launch_trace(int head_size, int kv_elt_bytes, bool aligned, int rows,
                        const DecodeParams& p, int batch, hipStream_t stream);

// The decode step behind every decode entry point: validates the shape and
// plan, lays the plan's workspace out in `workspace` (workspace_bytes long),
// launches the split-KV kernel (with the optional events around it) and the
// merge kernel when the plan needs one.  Returns a PDA_* status.
int run_decode(const pda_shape_t* s, const pda_plan_t* pl, const void* q, const void* k_cache,
               const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
               float scale, void* out, void* workspace, int64_t workspace_bytes, void* stream,
               hipEvent_t ev0, hipEvent_t ev1);

// Floats per staged row of the unit epilogue in LDS: D values, the running
// max m and the denominator l, and two floats of padding, so that rows start
// 16 bytes apart (with the 16-byte aligned LDS base, every 8- and 16-byte
// access is aligned) and the matrix-core layout's 16-byte row writes of up to
// 8 rows fall on distinct banks (D + 2 put two rows' writes on each bank).
__host__ __device__ constexpr int lds_row_floats(int head_size) { return head_size + 4; }

// Rows the MFMA kernel stages in LDS at once at the end of a unit: 16 (a
// whole 16-row matrix-core chunk, one barrier) up to head size 128, 8 at 256
// (LDS).
__host__ __device__ constexpr int mfma_row_chunk(int head_size) {
    return head_size <= 128 ? 16 : kHeadChunk;
}

// Whether the MFMA kernel loads K in whole rows and moves each tile through
// an LDS buffer into the matrix-core operand layout (otherwise it loads the
// operand layout directly: 64 bytes of each of 16 rows per instruction).  By
// measurement: whole rows at head sizes 64 and 256, for fp8 KV, for
// partitions of at most 512 tokens (a call's first loads are then a large
// part of it) and over more than 128 units (B * Hkv; many rounds of
// workgroups); the direct loads for 16-bit KV at head size 128 with longer
// partitions over few units, where the LDS round trip measured 0.2-0.3 us
// slower per call.
__host__ __device__ inline bool mfma_k_whole_rows(int head_size, int kv_elt_bytes,
                                                  int tokens_per_part, int64_t units) {
    return head_size != 128 || kv_elt_bytes != 2 || tokens_per_part <= 512 || units > 128;
}

// Bytes of the MFMA kernel's per-wave LDS buffers through which a K tile
// moves from whole-row loads into the matrix-core operand layout: 16 rows of
// kv_elt_bytes * head_size bytes, each padded by 16 bytes.
__host__ __device__ constexpr int mfma_kstage_bytes(int head_size, int kv_elt_bytes) {
    return kWaves * 16 * (kv_elt_bytes * head_size + 16);
}

// Bytes of dynamic LDS the MFMA kernel uses: the K staging buffers (whole-row
// K loads only), the epilogue's rows (staged mfma_row_chunk at a time), the
// block-table slice.
inline size_t mfma_lds_bytes(int head_size, int kv_elt_bytes, bool k_whole_rows,
                             int tbl_capacity) {
    return (size_t)(k_whole_rows ? mfma_kstage_bytes(head_size, kv_elt_bytes) : 0) +
           (size_t)kWaves * mfma_row_chunk(head_size) * lds_row_floats(head_size) * sizeof(float) +
           (size_t)tbl_capacity * sizeof(int32_t);
}

// Padded group sizes the VALU kernel is compiled for.
inline int valu_group_pad(int g) {
    if (g <= 4) return g;
    if (g <= 6) return 6;
    if (g <= 8) return 8;
    if (g <= 12) return 12;
    return 16;
}

// Bytes of dynamic LDS the decode kernel uses for a block-table slice of
// `tbl_capacity` entries plus the cross-wave merge of `gpad` heads.
inline size_t decode_lds_bytes(int head_size, int gpad, int tbl_capacity) {
    size_t merge = (size_t)kWaves * gpad * lds_row_floats(head_size) * sizeof(float);
    return merge + (size_t)tbl_capacity * sizeof(int32_t);
}

}  // namespace pda

// Paged-attention decode, matrix-core variant, for gfx950.
//
// Same unit of work as the VALU variant -- one workgroup of 4 wavefronts per
// (partition p, KV head g, sequence b), all rows of the unit packed (the G
// query heads of the group, for each of the q_len query positions), every
// K/V byte read once -- but both contractions run on MFMA, with the packed
// rows padded to 16 per chunk:
//
//   QK^T  S^T = K Q^T on v_mfma_f32_16x16x32_{bf16,f16}: a 16-token tile of K
//         rows is the A operand (lane l holds 16 bytes of token l%16 per
//         k-step), Q^T the B operand.  Where it measured faster
//         (mfma_k_whole_rows) K is loaded in whole rows (each load
//         instruction reads whole 128-byte lines, where the operand layout
//         reads 64 bytes of each of 16 rows) and moved into the operand
//         layout through the wave's own LDS buffer; elsewhere (16-bit KV at
//         head size 128, long partitions, few units) it is loaded straight
//         into the operand layout.  The 16x16 result leaves
//         each lane the scores of one row (l%16) for four tokens (4(l/16) +
//         r, r = 0..3).
//   mask  scores of tokens at or past the partition end, outside a sliding
//         window or after the row's causal end become -inf by select; tail
//         slots and slots before a window are never addressed (see tile_row).
//   softmax  online, exp2 domain; the running max per head is shared by the
//         four lanes that hold that head; the accumulator is rescaled only
//         when some max grew.
//   PV    O^T = V^T P^T on v_mfma_f32_16x16x16_{bf16,f16}, one MFMA per
//         element e of the lanes' VE-element V chunks (VE = 8, or 4 at head
//         size 64 so that the 16 d-rows stay distinct): round r of V loads
//         token 4(l/16) + r, elements d = VE*(l%16) + e, so element e of the
//         lane's four rounds is exactly its A operand (d-row l%16, tokens
//         4(l/16) .. +4), and the exp'd scores the lane holds (row l%16,
//         the same four tokens) are exactly its B operand.  Neither V nor P
//         moves between lanes; the weights are rounded to the 16-bit type
//         (V is exact), and the denominator sums the rounded weights, so the
//         output stays a convex combination of V rows.
//
// VALU work per tile is reduced to the repacking of V halves and the softmax
// bookkeeping, independent of the row count.
//
// fp8 KV (F8): K and V rows are OCP E4M3 bytes.  A lane's 16-byte K load
// then holds 16 elements, d = 64*s2 + 16*q4 .. +16, decoded exactly to the
// 16-bit type as the A operands of k-steps 2*s2 and 2*s2 + 1; the query
// elements of each k-step are loaded in the same permuted order of d (a dot
// product does not depend on the order of its terms).  V chunks are VE-byte
// loads, byte-transposed across the four rounds and decoded exactly to the
// 16-bit type.  k_scale is folded into the score scale and v_scale
// into the output (write_unit_rows).
//
// Compiled once per (element type, head size, KV type): PDA_DTYPE (0 bf16,
// 1 fp16), PDA_HEAD (64, 128, 256) and PDA_KV_FP8 (0: 16-bit KV, 1: fp8).
#include <hip/hip_ext.h>

#include <type_traits>

#include "pda_device.h"

#ifndef PDA_DTYPE
#error "PDA_DTYPE must be defined"
#endif
#ifndef PDA_HEAD
#error "PDA_HEAD must be defined"
#endif
#ifndef PDA_KV_FP8
#define PDA_KV_FP8 0
#endif
// Register-buffer stages of the tile pipeline, chosen by measurement (the
// kernel takes four for K+V tiles under 4 KiB per wave, see below)
#ifndef PDA_MFMA_STAGES
#define PDA_MFMA_STAGES 2
#endif
#ifndef PDA_MFMA_STAGES_FP8
#define PDA_MFMA_STAGES_FP8 2
#endif

namespace pda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename Elt>
struct MfmaQK;
template <>
struct MfmaQK<BF16> {
    __device__ static inline f32x4_t run(uint4 a, uint4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
};
template <>
struct MfmaQK<FP16> {
    __device__ static inline f32x4_t run(uint4 a, uint4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
};

template <typename Elt>
struct MfmaPV;
template <>
struct MfmaPV<BF16> {
    typedef short i16x4_t __attribute__((ext_vector_type(4)));
    __device__ static inline f32x4_t run(uint2 a, uint2 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                         __builtin_bit_cast(i16x4_t, b), c, 0, 0,
                                                         0);
    }
};
template <>
struct MfmaPV<FP16> {
    typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
    __device__ static inline f32x4_t run(uint2 a, uint2 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                     __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
    }
};

// 32-bit word i of a 16- or 8-byte chunk (i a compile-time constant after
// unrolling)
__device__ inline uint32_t word_of(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ inline uint32_t word_of(const uint2& v, int i) { return i == 0 ? v.x : v.y; }

// A lane's V chunk of one round: VE elements, 16, 8 or 4 bytes
template <int BYTES>
struct VChunk;
template <>
struct VChunk<16> {
    typedef uint4 type;
    __device__ static type load(const char* p) { return load_row16(p); }
    __device__ static type load_buf(const char* b, uint32_t off, bool v) { return load_row16_buf(b, off, v); }
};
template <>
struct VChunk<8> {
    typedef uint2 type;
    __device__ static type load(const char* p) { return load_row8(p); }
    __device__ static type load_buf(const char* b, uint32_t off, bool v) { return load_row8_buf(b, off, v); }
};
template <>
struct VChunk<4> {
    typedef uint32_t type;
    __device__ static type load(const char* p) { return load_row4(p); }
    __device__ static type load_buf(const char* b, uint32_t off, bool v) { return load_row4_buf(b, off, v); }
};

// The element type and head size are template parameters of the kernel so
// that every instantiation has its own symbol across translation units.
// The unit's R = q_len * G rows (row r: query position r / G, head r % G)
// are packed in RC chunks of 16 (RC = 2 for R > 16): each K tile feeds RC
// QK and RC PV products, and each chunk keeps its own softmax state and
// accumulators.  KWR: K is loaded in whole rows and moved into the operand
// layout through the wave's LDS buffer (mfma_k_whole_rows picks it per call).
template <typename Elt, int D, bool ALIGNED, bool BUF, int RC, bool F8, bool KWR>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(DecodeParams p) {
    static_assert(RC == 1 || RC == 2, "one or two 16-row chunks");
    using Geo = MfmaGeom<D>;
    constexpr int KS = Geo::KS, DH = Geo::DH, VE = Geo::VE, TT = 16;
    constexpr int EB = F8 ? 1 : 2;             // KV bytes per element
    // tiles in register buffers (fp8 tiles are half the bytes and registers);
    // a wave's K+V tile under 4 KiB (fp8 at head size 64) takes four, which
    // keep enough bytes in flight (two: 6 % slower per call)
    constexpr int S = 2 * TT * D * EB < 4096 ? 4 : F8 ? PDA_MFMA_STAGES_FP8 : PDA_MFMA_STAGES;
    static_assert(S >= 2 && S <= 6, "stages");
    constexpr int KL = F8 ? KS / 2 : KS;       // 16-byte K loads per lane and tile
    using VC = VChunk<VE * EB>;
    using VRaw = typename VC::type;            // a lane's VE V elements of one round
    // 16-byte aligned: the static LDS of the merge tail (4228 bytes) comes
    // first, and a 4-byte aligned base made every 8- and 16-byte access of
    // the epilogue a misaligned one
    extern __shared__ __attribute__((aligned(16))) float smem[];
    // K rows: RB bytes, LPT lanes per row in a whole-row load, staged KSB apart
    constexpr int RB = EB * D, LPT = RB / 16, KSB = RB + 16;
    constexpr int KSTAGE = KWR ? mfma_kstage_bytes(D, EB) : 0;
    static_assert(KSTAGE % 16 == 0, "the epilogue rows stay 16-byte aligned");
    char* kst = reinterpret_cast<char*>(smem);  // [kWaves][16][KSB]: each wave's K tile (KWR)
    float* red = smem + KSTAGE / 4;  // [kWaves][HC][lds_row_floats(D)]: the epilogue's rows
    constexpr int HC = mfma_row_chunk(D);  // rows staged in LDS at a time
    int32_t* tbl = reinterpret_cast<int32_t*>(red + kWaves * HC * lds_row_floats(D));

    // grid (Hkv, B, P): the partition index varies slowest (see the launcher)
    const int g = blockIdx.x, b = blockIdx.y, part = blockIdx.z;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int q4 = lane >> 4, c16 = lane & 15;
    const int R = p.rows;

    // Loads that do not depend on the context length leave together with the
    // seq_lens load, so the first K/V loads wait for one round trip, not three:
    // Q^T, the B operand of chunk c (row 16c + c16 of the unit, elements
    // 32s + 8*q4 .. +8 for k-step s; lanes past R read row R-1 again, and the
    // results of those padding rows are never written), and on the aligned
    // path the table entries of the wave's first two tiles at the partition's
    // start without a sliding window.
    const int raw_len = p.seq_lens[b];
    int lrow[RC];  // the lane's row in each chunk (clamped to a real row)
    uint4 qb[RC][KS];
#pragma unroll
    for (int c = 0; c < RC; ++c) {
        lrow[c] = min(16 * c + c16, R - 1);
        const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + row_index(p, b, g, lrow[c]) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            // elements of k-step s in the lane's K operand (see the file comment)
            const int e0 = F8 ? 64 * (s / 2) + 16 * q4 + 8 * (s % 2) : 32 * s + 8 * q4;
            qb[c][s] = *reinterpret_cast<const uint4*>(qrow + e0);
        }
    }
    const int32_t* trow = p.block_table + (int64_t)b * p.max_blocks_per_seq;
    FirstTiles ft{{0, 0}, {0, 0}};
    if constexpr (ALIGNED) {
        ft = first_tile_entries(p, trow, part, wave, TT);
        keep_issued(raw_len, ft.e[0], ft.e[1]);
    }
    issue_fence();

    const SeqRange rg = seq_range_of(p, raw_len);
    const int L = rg.L;
    const int t0 = rg.base + part * p.tokens_per_part;
    const bool direct = p.num_partitions == 1;

    if (t0 >= L) {  // empty partition; the first one of an empty context writes zeros
        if (part == 0) zero_unit_rows<D>(p, b, g);
        return;
    }
    RowRange rr[RC];  // tokens the lane's row of each chunk attends to
#pragma unroll
    for (int c = 0; c < RC; ++c) rr[c] = row_range(p, rg, lrow[c] / p.group);
    const int t1 = min(t0 + p.tokens_per_part, L);
    const int lb0 = (int)fastdiv((uint32_t)t0, p.bs_div);
    const int lb1 = (int)fastdiv((uint32_t)(t1 - 1), p.bs_div);
    if (!ALIGNED) stage_table_slice(p, b, lb0, lb1, tbl);
    const int32_t* tv = table_view<ALIGNED>(p, b, tbl);
    const int tlb0 = ALIGNED ? 0 : lb0;
    if (!ALIGNED) __syncthreads();  // publish the staged table slice

    const char* kc = static_cast<const char*>(p.k_cache);
    const char* vc = static_cast<const char*>(p.v_cache);
    const int64_t head_off = (int64_t)g * p.head_stride;               // elements
    const uint32_t v_lane = (uint32_t)(VE * c16 * EB);                  // bytes
    const int ntiles = (t1 - t0 + TT - 1) / TT;

    // Tile jj >= ntiles is a prefetch past the end: with buffer loads (BUF)
    // it loads nothing (zeros, no memory access); otherwise it re-reads the
    // last tile.  Either way process() never sees it.  Buffer loads need a
    // wave-uniform block base: the launcher uses them on the aligned path.
    static_assert(ALIGNED || !BUF, "buffer loads need the aligned path");
    constexpr bool kBuf = BUF;
    auto tile_start = [&](int jj) { return t0 + (kBuf ? jj : min(jj, ntiles - 1)) * TT; };
    TileBlock first[2] = {{0, 0}, {0, 0}};
    if constexpr (ALIGNED)
        first_tile_blocks(p, trow, ft, part, wave, TT, rg, t0, ntiles, kBuf, first);
    // `tb` is the tile's block on the aligned path (tile_block of tile_start)
    auto load_tile = [&](int jj, const TileBlock& tb, uint4 (&kr)[KL], VRaw (&vr)[4][DH]) {
        const bool valid = jj < ntiles;
        const int tile_base = tile_start(jj);
        int phys = tb.phys, slot0 = tb.slot0, dt;
        if constexpr (KWR) {
            // whole rows: load s gives the lane 16 bytes of token mfma_k_token
#pragma unroll
            for (int s = 0; s < KL; ++s) {
                const int tok = mfma_k_token(lane, s, LPT);
                if constexpr (ALIGNED) {
                    dt = tile_row(tile_base, rg.lo, t1, tok);
                } else {
                    locate_row<false>(p, tv, tlb0, tile_base, rg.lo, t1, tok, phys, slot0, dt);
                }
                const int64_t base =
                    EB * ((int64_t)phys * p.block_stride + head_off + (int64_t)slot0 * D);
                const uint32_t off = (uint32_t)dt * RB + 16 * (lane % LPT);
                kr[s] = kBuf ? load_row16_buf(kc + base, off, valid) : load_row16(kc + base + off);
            }
        } else {
            // the operand layout: token l%16, bytes 64s + 16(l/16) for load s
            if constexpr (ALIGNED) {
                dt = tile_row(tile_base, rg.lo, t1, mfma_k_offset(lane));
            } else {
                locate_row<false>(p, tv, tlb0, tile_base, rg.lo, t1, mfma_k_offset(lane), phys,
                                  slot0, dt);
            }
            const int64_t base =
                EB * ((int64_t)phys * p.block_stride + head_off + (int64_t)slot0 * D);
            const uint32_t off = (uint32_t)dt * RB + 16 * q4;
#pragma unroll
            for (int s = 0; s < KL; ++s)
                kr[s] = kBuf ? load_row16_buf(kc + base, off + 64 * s, valid)
                             : load_row16(kc + base + off + 64 * s);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (ALIGNED) {
                dt = tile_row(tile_base, rg.lo, t1, mfma_v_offset(lane, r));
            } else {
                locate_row<false>(p, tv, tlb0, tile_base, rg.lo, t1, mfma_v_offset(lane, r), phys,
                                  slot0, dt);
            }
            const int64_t base =
                EB * ((int64_t)phys * p.block_stride + head_off + (int64_t)slot0 * D);
            const uint32_t off = (uint32_t)dt * (EB * D) + v_lane;
#pragma unroll
            for (int dh = 0; dh < DH; ++dh)
                vr[r][dh] = kBuf ? VC::load_buf(vc + base, off + 128 * EB * dh, valid)
                                 : VC::load(vc + base + off + 128 * EB * dh);
        }
    };
    auto block_of = [&](int jj) {
        return ALIGNED ? tile_block(p, trow, tile_start(jj)) : TileBlock{0, 0};
    };

    // oacc[c][dh][e][i] = O[row 16c + c16][d = dh*128 + VE*(4*q4 + i) + e]
    f32x4_t oacc[RC][DH][VE];
#pragma unroll
    for (int a = 0; a < RC; ++a)
#pragma unroll
        for (int dh = 0; dh < DH; ++dh)
#pragma unroll
            for (int e = 0; e < VE; ++e) oacc[a][dh][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m[RC], l[RC];
#pragma unroll
    for (int c = 0; c < RC; ++c) {
        m[c] = -FLT_MAX;  // running max of row 16c + c16 (finite floor: exp2(-inf - m) = 0)
        l[c] = 0.f;       // this lane's share of that row's denominator
    }

    auto process = [&](int j, const uint4 (&kr)[KL], const VRaw (&vr)[4][DH]) {
        const int tile_base = t0 + j * TT;
        const bool full = full_tile(rg, tile_base, TT, t1);
        // the whole-row K loads through the wave's LDS buffer into the operand
        // layout (the wave's LDS operations complete in order, so each read
        // sees this tile's writes, and the next tile's writes follow these
        // reads); rows KSB apart keep both the writes and the reads free of
        // bank conflicts
        uint4 kx[KL];
        if constexpr (KWR) {
            char* kb = kst + wave * 16 * KSB;
#pragma unroll
            for (int s = 0; s < KL; ++s)
                *reinterpret_cast<uint4*>(kb + mfma_k_token(lane, s, LPT) * KSB +
                                          16 * (lane % LPT)) = kr[s];
#pragma unroll
            for (int s = 0; s < KL; ++s)
                kx[s] = *reinterpret_cast<const uint4*>(kb + c16 * KSB + 64 * s + 16 * q4);
        } else {
#pragma unroll
            for (int s = 0; s < KL; ++s) kx[s] = kr[s];
        }
        // the A operands of the k-steps (fp8 bytes decoded to the 16-bit type)
        uint4 ka[KS];
#pragma unroll
        for (int s = 0; s < KL; ++s) {
            if constexpr (F8) {
                ka[2 * s] = fp8x8_to_16bit<Elt>(kx[s].x, kx[s].y);
                ka[2 * s + 1] = fp8x8_to_16bit<Elt>(kx[s].z, kx[s].w);
            } else {
                ka[s] = kx[s];
            }
        }
        float sc[RC][4];
#pragma unroll
        for (int c = 0; c < RC; ++c) {
            f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) sacc = MfmaQK<Elt>::run(ka[s], qb[c][s], sacc);
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[c][r] = sacc[r] * p.scale_log2;
        }
        if (!full) {
#pragma unroll
            for (int c = 0; c < RC; ++c)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = tile_base + mfma_v_offset(lane, r);
                    sc[c][r] = (t >= rr[c].lo && t < min(t1, rr[c].end)) ? sc[c][r] : -INFINITY;
                }
        }
        float mn[RC];
        bool grew = false;
#pragma unroll
        for (int c = 0; c < RC; ++c) {
            float mt = fmaxf(fmaxf(sc[c][0], sc[c][1]), fmaxf(sc[c][2], sc[c][3]));
            mt = max_xor<16>(mt);
            mt = max_xor<32>(mt);
            mn[c] = fmaxf(m[c], mt);
            grew |= mn[c] > m[c];
        }
        if (__builtin_amdgcn_ballot_w64(grew)) {
#pragma unroll
            for (int c = 0; c < RC; ++c) {
                // every accumulator register of the lane belongs to its own row
                const float alpha = fast_exp2(m[c] - mn[c]);
                l[c] *= alpha;
#pragma unroll
                for (int dh = 0; dh < DH; ++dh)
#pragma unroll
                    for (int e = 0; e < VE; ++e) oacc[c][dh][e] *= alpha;
                m[c] = mn[c];
            }
        }
        // B operand: the lane's four weights of row 16c + c16 (tokens
        // 4*q4 + r), rounded to the 16-bit type; the denominator sums the
        // rounded values, in token order
        uint2 pb[RC];
#pragma unroll
        for (int c = 0; c < RC; ++c) {
            uint32_t h[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) h[r] = Elt::from_float(fast_exp2(sc[c][r] - m[c]));
            pb[c].x = h[0] | (h[1] << 16);
            pb[c].y = h[2] | (h[3] << 16);
            l[c] += Elt::lo(pb[c].x);
            l[c] += Elt::hi(pb[c].x);
            l[c] += Elt::lo(pb[c].y);
            l[c] += Elt::hi(pb[c].y);
        }
#pragma unroll
        for (int dh = 0; dh < DH; ++dh) {
            if constexpr (F8) {
                // byte e of the four rounds (tokens 4*q4 + r, in order) into
                // one word, which two packed conversions turn into the A
                // operand of element e
                uint32_t tb[VE];
                if constexpr (VE == 8) {
                    byte_transpose4(vr[0][dh].x, vr[1][dh].x, vr[2][dh].x, vr[3][dh].x,
                                    *reinterpret_cast<uint32_t(*)[4]>(&tb[0]));
                    byte_transpose4(vr[0][dh].y, vr[1][dh].y, vr[2][dh].y, vr[3][dh].y,
                                    *reinterpret_cast<uint32_t(*)[4]>(&tb[4]));
                } else {
                    byte_transpose4(vr[0][dh], vr[1][dh], vr[2][dh], vr[3][dh],
                                    *reinterpret_cast<uint32_t(*)[4]>(&tb[0]));
                }
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const uint2 a = make_uint2(fp8x2_to_16bit<Elt, false>(tb[e]),
                                               fp8x2_to_16bit<Elt, true>(tb[e]));
#pragma unroll
                    for (int c = 0; c < RC; ++c)
                        oacc[c][dh][e] = MfmaPV<Elt>::run(a, pb[c], oacc[c][dh][e]);
                }
            } else {
                // A operand: element e of the lane's four V rounds (tokens
                // 4*q4 + r), tokens in order
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const int wi = e / 2;
                    uint2 a;
                    if (e % 2 == 0) {
                        a.x = (word_of(vr[0][dh], wi) & 0xffffu) | (word_of(vr[1][dh], wi) << 16);
                        a.y = (word_of(vr[2][dh], wi) & 0xffffu) | (word_of(vr[3][dh], wi) << 16);
                    } else {
                        a.x = (word_of(vr[0][dh], wi) >> 16) | (word_of(vr[1][dh], wi) & 0xffff0000u);
                        a.y = (word_of(vr[2][dh], wi) >> 16) | (word_of(vr[3][dh], wi) & 0xffff0000u);
                    }
#pragma unroll
                    for (int c = 0; c < RC; ++c)
                        oacc[c][dh][e] = MfmaPV<Elt>::run(a, pb[c], oacc[c][dh][e]);
                }
            }
        }
    };

    // Register buffers in rotation.  The loop has a single exit and its loads
    // are unconditional (past the end they load nothing, see load_tile): an
    // exit or a guarded load in the middle of the body makes the compiler
    // drain every outstanding load (vmcnt(0)) at the loop head, which leaves
    // one tile in flight instead of more.
    int j = wave;
    if constexpr (S == 2) {
        // two buffers, loop rotated so that its head waits for buffer a
        // while buffer b is in flight
        uint4 ka[KL], kb[KL];
        VRaw va[4][DH], vb[4][DH];
        if (j < ntiles) {
            load_tile(j, first[0], ka, va);
            load_tile(j + kWaves, first[1], kb, vb);
        }
        for (; j < ntiles; j += 2 * kWaves) {
            process(j, ka, va);
            load_tile(j + 2 * kWaves, block_of(j + 2 * kWaves), ka, va);
            if (j + kWaves < ntiles) process(j + kWaves, kb, vb);
            load_tile(j + 3 * kWaves, block_of(j + 3 * kWaves), kb, vb);
        }
    } else {
        // S buffers: each step refills the buffer freed by the previous step,
        // then processes the oldest, so S-1 tiles are in flight meanwhile
        uint4 kbuf[S][KL];
        VRaw vbuf[S][4][DH];
        if (j < ntiles) {
            load_tile(j, first[0], kbuf[0], vbuf[0]);
            load_tile(j + kWaves, first[1], kbuf[1], vbuf[1]);
#pragma unroll
            for (int st = 2; st < S - 1; ++st)
                load_tile(j + st * kWaves, block_of(j + st * kWaves), kbuf[st], vbuf[st]);
        }
        for (; j < ntiles; j += S * kWaves) {
#pragma unroll
            for (int st = 0; st < S; ++st) {
                const int jn = j + (st + S - 1) * kWaves;
                load_tile(jn, block_of(jn), kbuf[(st + S - 1) % S], vbuf[(st + S - 1) % S]);
                if (j + st * kWaves < ntiles) process(j + st * kWaves, kbuf[st], vbuf[st]);
            }
        }
    }

    // full denominator of each lane row (all four lane groups hold the same m)
#pragma unroll
    for (int c = 0; c < RC; ++c) {
        l[c] = sum_xor<16>(l[c]);
        l[c] = sum_xor<32>(l[c]);
    }

    // merge the wavefronts and write the unit's result, rows in chunks
    for (int h0 = 0; h0 < R; h0 += HC) {
        const int hn = min(HC, R - h0);
#pragma unroll
        for (int c = 0; c < RC; ++c) {
            const int hi = 16 * c + c16 - h0;
            if (hi < 0 || hi >= hn) continue;
            float* row = red + (wave * HC + hi) * lds_row_floats(D);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int dh = 0; dh < DH; ++dh)
#pragma unroll
                    for (int e = 0; e < VE; ++e)
                        row[dh * 128 + VE * (4 * q4 + i) + e] = oacc[c][dh][e][i];
        }
        if (q4 == 0) {
#pragma unroll
            for (int c = 0; c < RC; ++c) {
                const int hi = 16 * c + c16 - h0;
                if (hi < 0 || hi >= hn) continue;
                float* row = red + (wave * HC + hi) * lds_row_floats(D);
                row[D] = m[c];
                row[D + 1] = l[c];
            }
        }
        __syncthreads();
        // the combine: up to 8 rows in one pass of 32 threads per row, 9 to
        // 16 rows in one pass of 16 threads per row
        bool done = false;
        if constexpr (HC > kHeadChunk) {
            if (hn > kHeadChunk) {
                write_unit_rows<Elt, D, true, 16>(p, red, HC, h0, hn, b, g, part);
                done = true;
            }
        }
        if (!done) write_unit_rows<Elt, D, true>(p, red, HC, h0, hn, b, g, part);
        if (h0 + HC < R) __syncthreads();  // before the next chunk reuses red
    }
    if (!direct && p.fused_merge) fused_merge_tail<Elt, D>(p, rg, b, g);
}

#if PDA_DTYPE == 0
using EltT = BF16;
#else
using EltT = FP16;
#endif
constexpr int kHead = PDA_HEAD;

constexpr bool kF8 = PDA_KV_FP8 != 0;

template <bool ALIGNED, bool BUF, int RC, bool KWR>
static hipError_t launch_one(const DecodeParams& p, int batch, hipStream_t stream,
                             hipEvent_t start, hipEvent_t stop) {
    // Workgroups are dispatched in grid order, partition by partition: the
    // empty partitions of shorter sequences come after the live partitions of
    // every sequence instead of between them, where each one measured to cost
    // tens of ns of the whole launch (mixed lengths at batch 64: 16% faster).
    const dim3 grid(p.num_kv_heads, batch, p.num_partitions);
    const size_t own = mfma_lds_bytes(kHead, kF8 ? 1 : 2, KWR, p.tbl_capacity);
    const uint32_t lds = (uint32_t)(own > (size_t)p.lds_floor ? own : (size_t)p.lds_floor);
    if (start || stop)
        hipExtLaunchKernelGGL((decode_mfma_kernel<EltT, kHead, ALIGNED, BUF, RC, kF8, KWR>), grid,
                              dim3(kThreads), lds, stream, start, stop, 0, p);
    else
        hipLaunchKernelGGL((decode_mfma_kernel<EltT, kHead, ALIGNED, BUF, RC, kF8, KWR>), grid,
                           dim3(kThreads), lds, stream, p);
    return hipGetLastError();
}

// Whole-row K loads where they measured faster (mfma_k_whole_rows); the
// direct operand-layout loads are compiled only where they can be chosen.
template <bool ALIGNED, bool BUF, int RC>
static hipError_t launch_kwr(const DecodeParams& p, int batch, hipStream_t stream,
                             hipEvent_t start, hipEvent_t stop) {
    if constexpr (kHead == 128 && !kF8) {
        if (!mfma_k_whole_rows(kHead, 2, p.tokens_per_part, (int64_t)p.num_kv_heads * batch))
            return launch_one<ALIGNED, BUF, RC, false>(p, batch, stream, start, stop);
    }
    return launch_one<ALIGNED, BUF, RC, true>(p, batch, stream, start, stop);
}

// One 16-row chunk for up to 16 rows per unit, two beyond.
template <bool ALIGNED, bool BUF>
static hipError_t launch_pv(const DecodeParams& p, int batch, hipStream_t stream,
                            hipEvent_t start, hipEvent_t stop) {
    if (p.rows <= 16) return launch_kwr<ALIGNED, BUF, 1>(p, batch, stream, start, stop);
    return launch_kwr<ALIGNED, BUF, 2>(p, batch, stream, start, stop);
}

#define PDA_CAT2(a, b, c) a##_##b##_##c
#define PDA_CAT(a, b, c) PDA_CAT2(a, b, c)
#if PDA_KV_FP8
#define PDA_MFMA_LAUNCHER launch_decode_mfma8
#else
#define PDA_MFMA_LAUNCHER launch_decode_mfma
#endif
hipError_t PDA_CAT(PDA_MFMA_LAUNCHER, PDA_DTYPE, PDA_HEAD)(bool aligned, const DecodeParams& p,
                                                           int batch, hipStream_t stream,
                                                           hipEvent_t e0, hipEvent_t e1) {
    // The aligned path uses buffer loads (past-the-end prefetches load
    // nothing); they measured faster at every head size (at 256 since the
    // 16x16x16 PV: 29.7 -> 28.7 us at the low-parallelism layer).
    if (!aligned) return launch_pv<false, false>(p, batch, stream, e0, e1);
    return launch_pv<true, true>(p, batch, stream, e0, e1);
}

}  // namespace pda

// Paged-attention decode, VALU variant, for gfx950.
//
// One workgroup (4 wavefronts) per unit (partition p, KV head g, sequence b).
// All rows of the unit are packed (the G query heads of the KV group, for
// each of the q_len query positions), so every K/V byte of the partition is
// read from HBM once.  Each lane loads 16 contiguous
// bytes of a token row; a row spans D/8 lanes, so a wavefront load covers
// whole rows and consecutive lanes touch consecutive addresses.
//
// Per tile and lane:
//   QK^T   packed dot2 over the lane's 8 elements, then a DPP sum over the
//          token row's lanes -> one score per packed row;
//   mask   scores of tokens at or past the partition end, outside a sliding
//          window or after a row's causal end are replaced by -inf with a
//          select (tail slots are not even addressed: see tile_row), so NaN
//          or garbage there cannot reach a score;
//   online softmax in the exp2 domain, per lane sub-stream, with a rescale
//          only when some lane's running max grew;
//   PV     fp32 FMAs of the lane's 8 V elements.
// At the end the sub-streams of a wavefront and then the 4 wavefronts are
// merged with the log-sum-exp rule, in a fixed order (run-to-run identical).
// With one partition the unit writes the 16-bit output; otherwise it writes
// the fp32 partial (o, m, l) that the merge kernel combines.
//
// This translation unit is compiled once per (element type, head size):
// PDA_DTYPE (0 bf16, 1 fp16) and PDA_HEAD (64, 128, 256).
#include <hip/hip_ext.h>

#include "pda_device.h"

#ifndef PDA_DTYPE
#error "PDA_DTYPE must be defined"
#endif
#ifndef PDA_HEAD
#error "PDA_HEAD must be defined"
#endif

// Tiles in flight per wave (register buffers in rotation): 3 measured best.
#ifndef PDA_VALU_STAGES
#define PDA_VALU_STAGES 3
#endif

namespace pda {

// The element type and head size are template parameters of the kernel (not
// only of this translation unit) so that every instantiation has its own
// symbol name across the six translation units.
template <typename Elt, int D, int GP, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(DecodeParams p) {
    using Geo = ValuGeom<D>;
    constexpr int LPT = Geo::LPT, RT = Geo::R, U = Geo::U, TT = Geo::TT;
    // 16-byte aligned: the static LDS of the merge tail (4228 bytes) comes
    // first, and a 4-byte aligned base made every 8- and 16-byte access of
    // the epilogue a misaligned one
    extern __shared__ __attribute__((aligned(16))) float smem[];
    float* red = smem;  // [kWaves][GP][lds_row_floats(D)]: the unit epilogue's staging
    int32_t* tbl = reinterpret_cast<int32_t*>(smem + kWaves * GP * lds_row_floats(D));

    // grid (Hkv, B, P): the partition index varies slowest (see the launcher)
    const int g = blockIdx.x, b = blockIdx.y, part = blockIdx.z;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int c = lane % LPT, r = lane / LPT;
    const int R = p.rows;  // rows of the unit: q_len positions x G heads
    constexpr int S = PDA_VALU_STAGES;
    static_assert(S >= 2 && S <= 8, "stages");

    // Loads that do not depend on the context length leave together with the
    // seq_lens load, so the first K/V loads wait for one round trip, not
    // three: the packed query rows of this unit (8 elements per lane and row;
    // padding rows past R read row R-1 again, and their results are never
    // written), and on the aligned path the table entries of the wave's
    // first S-1 tiles at the partition's start without a sliding window.
    const int raw_len = p.seq_lens[b];
    uint4 qv[GP];
#pragma unroll
    for (int i = 0; i < GP; ++i) {
        const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                               row_index(p, b, g, min(i, R - 1)) * D + c * 8;
        qv[i] = *reinterpret_cast<const uint4*>(qrow);
    }
    const int32_t* trow = p.block_table + (int64_t)b * p.max_blocks_per_seq;
    static_assert(S == 3, "the first-tile table entries are kept for S - 1 = 2 tiles");
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
    RowRange rr[GP];  // tokens each row attends to
#pragma unroll
    for (int i = 0; i < GP; ++i) rr[i] = row_range(p, rg, min(i, R - 1) / p.group);
    const int t1 = min(t0 + p.tokens_per_part, L);
    const int lb0 = (int)fastdiv((uint32_t)t0, p.bs_div);
    const int lb1 = (int)fastdiv((uint32_t)(t1 - 1), p.bs_div);
    if (!ALIGNED) stage_table_slice(p, b, lb0, lb1, tbl);
    const int32_t* tv = table_view<ALIGNED>(p, b, tbl);
    const int tlb0 = ALIGNED ? 0 : lb0;
    if (!ALIGNED) __syncthreads();  // publish the staged table slice

    const char* kc = static_cast<const char*>(p.k_cache);
    const char* vc = static_cast<const char*>(p.v_cache);
    const int64_t head_off = (int64_t)g * p.head_stride;   // elements
    const uint32_t lane_off = (uint32_t)c * 16;            // bytes
    const int ntiles = (t1 - t0 + TT - 1) / TT;

    // Address of a round's row: a block base (wave-uniform on the aligned
    // path, so it stays in scalar registers) plus a 32-bit per-lane byte
    // offset, the form of a global load with a scalar base.
    // Tile jj >= ntiles is a prefetch past the end: with buffer loads it
    // loads nothing (zeros, no memory access); otherwise it re-reads the last
    // tile.  Either way process() never sees it.  Buffer loads need a
    // wave-uniform block base (the aligned path); they are used where they
    // measured faster, a group of one head (with more heads the compiler's
    // schedule of the buffer form loses ~1%).
    constexpr bool kBuf = ALIGNED && GP == 1;
    auto tile_start = [&](int jj) { return t0 + (kBuf ? jj : min(jj, ntiles - 1)) * TT; };
    TileBlock first[S - 1] = {{0, 0}, {0, 0}};
    if constexpr (ALIGNED)
        first_tile_blocks(p, trow, ft, part, wave, TT, rg, t0, ntiles, kBuf, first);
    // `tb` is the tile's block on the aligned path (tile_block of tile_start)
    auto load_tile = [&](int jj, const TileBlock& tb, uint4 (&kr)[U], uint4 (&vr)[U]) {
        const bool valid = jj < ntiles;
        const int tile_base = tile_start(jj);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int phys = tb.phys, slot0 = tb.slot0, dt;
            if constexpr (ALIGNED)
                dt = tile_row(tile_base, rg.lo, t1, u * RT + r);
            else
                locate_token<RT, false>(p, tv, tlb0, tile_base, rg.lo, t1, u, r, phys, slot0, dt);
            const int64_t base = 2 * ((int64_t)phys * p.block_stride + head_off + (int64_t)slot0 * D);
            const uint32_t off = (uint32_t)dt * (2 * D) + lane_off;
            if constexpr (kBuf) {
                kr[u] = load_row16_buf(kc + base, off, valid);
                vr[u] = load_row16_buf(vc + base, off, valid);
            } else {
                kr[u] = load_row16(kc + base + off);
                vr[u] = load_row16(vc + base + off);
            }
        }
    };
    auto block_of = [&](int jj) {
        return ALIGNED ? tile_block(p, trow, tile_start(jj)) : TileBlock{0, 0};
    };

    float m[GP], l[GP], acc[GP][8];
#pragma unroll
    for (int i = 0; i < GP; ++i) {
        m[i] = -FLT_MAX;  // finite floor: exp2(-inf - m) stays 0, never NaN
        l[i] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
    }

    // One tile of QK^T, masking, online softmax and PV for this lane.
    auto process = [&](int j, const uint4 (&kr)[U], const uint4 (&vr)[U]) {
        const int tile_base = t0 + j * TT;
        const bool full = full_tile(rg, tile_base, TT, t1);
        float s[U][GP];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int i = 0; i < GP; ++i) {
                float d = Elt::dot2(qv[i].x, kr[u].x, 0.f);
                d = Elt::dot2(qv[i].y, kr[u].y, d);
                d = Elt::dot2(qv[i].z, kr[u].z, d);
                d = Elt::dot2(qv[i].w, kr[u].w, d);
                s[u][i] = group_sum<LPT>(d) * p.scale_log2;
            }
        }
        if (!full) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int t = tile_base + u * RT + r;
#pragma unroll
                for (int i = 0; i < GP; ++i)
                    s[u][i] = (t >= rr[i].lo && t < min(t1, rr[i].end)) ? s[u][i] : -INFINITY;
            }
        }
        bool grew = false;
        float mn[GP];
#pragma unroll
        for (int i = 0; i < GP; ++i) {
            float mt = s[0][i];
#pragma unroll
            for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u][i]);
            mn[i] = fmaxf(m[i], mt);
            grew |= mn[i] > m[i];
        }
        if (__builtin_amdgcn_ballot_w64(grew)) {
#pragma unroll
            for (int i = 0; i < GP; ++i) {
                const float alpha = fast_exp2(m[i] - mn[i]);
                l[i] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[i][e] *= alpha;
                m[i] = mn[i];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[8];
            vf[0] = Elt::lo(vr[u].x); vf[1] = Elt::hi(vr[u].x);
            vf[2] = Elt::lo(vr[u].y); vf[3] = Elt::hi(vr[u].y);
            vf[4] = Elt::lo(vr[u].z); vf[5] = Elt::hi(vr[u].z);
            vf[6] = Elt::lo(vr[u].w); vf[7] = Elt::hi(vr[u].w);
#pragma unroll
            for (int i = 0; i < GP; ++i) {
                const float pw = fast_exp2(s[u][i] - m[i]);
                l[i] += pw;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(pw, vf[e], acc[i][e]);
            }
        }
    };

    // Register buffers in rotation: while one tile is processed the wave's
    // next tile(s) are already in flight, and no buffer is ever copied (a copy
    // would force a wait for the in-flight loads).
    uint4 kbuf[S][U], vbuf[S][U];
    int j = wave;
    if (j < ntiles) {
#pragma unroll
        for (int st = 0; st < S - 1; ++st) load_tile(j + st * kWaves, first[st], kbuf[st], vbuf[st]);
    }
    // Each step refills the buffer freed S-1 steps ago and then processes the
    // oldest one, so S-1 tiles are in flight while one is processed.  One
    // exit, unconditional loads (past the end they load nothing): see the
    // note at load_row16_buf.
    for (; j < ntiles; j += S * kWaves) {
#pragma unroll
        for (int st = 0; st < S; ++st) {
            const int jn = j + (st + S - 1) * kWaves;
            load_tile(jn, block_of(jn), kbuf[(st + S - 1) % S], vbuf[(st + S - 1) % S]);
            if (j + st * kWaves < ntiles) process(j + st * kWaves, kbuf[st], vbuf[st]);
        }
    }

    // merge the RT lane sub-streams (lanes c, c+LPT, ...) of the wavefront
#pragma unroll
    for (int x = LPT; x < kWave; x <<= 1) {
#pragma unroll
        for (int i = 0; i < GP; ++i) {
            // the partner lane's values: row swaps across 16-lane rows,
            // a lane shuffle within a row
            auto partner = [&](float v) {
                return x == 16 ? xor_lane<16>(v) : x == 32 ? xor_lane<32>(v) : __shfl_xor(v, x);
            };
            const float mo = partner(m[i]);
            const float lo = partner(l[i]);
            const float mm = fmaxf(m[i], mo);
            const float wa = fast_exp2(m[i] - mm), wb = fast_exp2(mo - mm);
            l[i] = l[i] * wa + lo * wb;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float ao = partner(acc[i][e]);
                acc[i][e] = acc[i][e] * wa + ao * wb;
            }
            m[i] = mm;
        }
    }
    if (r == 0) {
#pragma unroll
        for (int i = 0; i < GP; ++i) {
            float* row = red + (wave * GP + i) * lds_row_floats(D);
#pragma unroll
            for (int e = 0; e < 8; ++e) row[c * 8 + e] = acc[i][e];
            if (c == 0) { row[D] = m[i]; row[D + 1] = l[i]; }
        }
    }
    __syncthreads();

    // merge the wavefronts and write the unit's result
    write_unit_rows<Elt, D, false>(p, red, GP, 0, R, b, g, part);
    if (!direct && p.fused_merge) fused_merge_tail<Elt, D>(p, rg, b, g);
}

#if PDA_DTYPE == 0
using EltT = BF16;
#else
using EltT = FP16;
#endif
constexpr int kHead = PDA_HEAD;

template <int GP, bool ALIGNED>
static hipError_t launch_one(const DecodeParams& p, int batch, hipStream_t stream,
                             hipEvent_t start, hipEvent_t stop) {
    // Workgroups are dispatched in grid order, partition by partition: the
    // empty partitions of shorter sequences come after the live partitions of
    // every sequence instead of between them, where each one measured to cost
    // tens of ns of the whole launch (mixed lengths at batch 64: 16% faster).
    const dim3 grid(p.num_kv_heads, batch, p.num_partitions);
    const size_t own = decode_lds_bytes(kHead, GP, p.tbl_capacity);
    const uint32_t lds = (uint32_t)(own > (size_t)p.lds_floor ? own : (size_t)p.lds_floor);
    if (start || stop)
        hipExtLaunchKernelGGL((decode_valu_kernel<EltT, kHead, GP, ALIGNED>), grid, dim3(kThreads),
                              lds, stream, start, stop, 0, p);
    else
        hipLaunchKernelGGL((decode_valu_kernel<EltT, kHead, GP, ALIGNED>), grid, dim3(kThreads),
                           lds, stream, p);
    return hipGetLastError();
}

template <bool ALIGNED>
static hipError_t launch_gp(int gpad, const DecodeParams& p, int batch, hipStream_t s,
                            hipEvent_t e0, hipEvent_t e1) {
    switch (gpad) {
        case 1: return launch_one<1, ALIGNED>(p, batch, s, e0, e1);
        case 2: return launch_one<2, ALIGNED>(p, batch, s, e0, e1);
        case 3: return launch_one<3, ALIGNED>(p, batch, s, e0, e1);
        case 4: return launch_one<4, ALIGNED>(p, batch, s, e0, e1);
        case 6: return launch_one<6, ALIGNED>(p, batch, s, e0, e1);
        case 8: return launch_one<8, ALIGNED>(p, batch, s, e0, e1);
        default: return hipErrorInvalidValue;
    }
}

#define PDA_CAT2(a, b, c) a##_##b##_##c
#define PDA_CAT(a, b, c) PDA_CAT2(a, b, c)
hipError_t PDA_CAT(launch_decode_valu, PDA_DTYPE, PDA_HEAD)(int gpad, bool aligned,
                                                            const DecodeParams& p, int batch,
                                                            hipStream_t stream, hipEvent_t e0,
                                                            hipEvent_t e1) {
    return aligned ? launch_gp<true>(gpad, p, batch, stream, e0, e1)
                   : launch_gp<false>(gpad, p, batch, stream, e0, e1);
}

}  // namespace pda

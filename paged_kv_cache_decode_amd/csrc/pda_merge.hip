// Log-sum-exp merge of split-KV partials, for gfx950.
//
// The context of a (sequence, KV head) is split into P partitions (the
// split-KV decode of page "Hybrid-SSM decode rate on dual Radeon cards": the
// KV range is split over more workgroups and reduced afterwards).  Partition
// p of query head h left a normalised fp32 output o_p, its max score m_p (exp2
// domain) and its denominator l_p.  The exact softmax over the union is
//     M = max_p m_p,   w_p = l_p * 2^(m_p - M),   out = sum_p w_p o_p / sum_p w_p
// over the partitions that hold tokens (p < ceil((L - base) / T_p)); the
// stale workspace entries of empty partitions may be loaded but never enter
// the sums.  A partition in which a causal row has no token left l_p = 0,
// so it weighs nothing; a row with no token at all (L == 0, or L < q_len)
// gives zeros.
//
// One workgroup of 256 threads per (64-element chunk of D, query head,
// query row position and sequence): 16 lanes x 4 elements cover the chunk,
// 16 partition groups stride over p.  Each thread merges its partitions with a running max, a
// batch of loads at a time; the 16 groups are then combined in a fixed order
// through LDS, so the result does not depend on timing.
#include "pda_device.h"

namespace pda {

template <typename Elt, int D, bool AHEAD>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p) {
    constexpr int kBatch = 8;  // partitions per thread and memory round trip
    __shared__ float4 red_o[16][16];
    __shared__ float2 red_mw[16][16];
    const int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;  // bi = b * q_len + i
    const int b = bi / p.q_len;
    const int tid = threadIdx.x, d4 = tid & 15, pg = tid >> 4;
    const int64_t row = (int64_t)bi * p.num_q_heads + h;
    uint16_t* out = static_cast<uint16_t*>(p.out) + row * D + chunk * 64 + d4 * 4;
    const float2* ml = reinterpret_cast<const float2*>(p.ws_ml) + row * p.num_partitions;
    const float* po = p.ws_o + row * p.num_partitions * D + chunk * 64 + d4 * 4;

    // AHEAD (few rows, latency-bound): the first batch of this thread's
    // partitions (pg, pg+16, ... below P) is loaded before the context length
    // is known, so the loads leave together with the seq_lens load and the
    // kernel pays one memory round trip instead of two; entries of partitions
    // past the live ones hold stale data and are never used.  Otherwise (many
    // rows, bandwidth-bound) only the live partitions are loaded.
    float2 mlv[kBatch];
    float4 ov[kBatch];
    if constexpr (AHEAD) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int q = pg + 16 * k;
            if (q < p.num_partitions) {
                mlv[k] = ml[q];
                ov[k] = *reinterpret_cast<const float4*>(po + (int64_t)q * D);
            }
        }
    }
    const int Pb = live_partitions(p, seq_range(p, b));
    if constexpr (!AHEAD) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int q = pg + 16 * k;
            if (q < Pb) {
                mlv[k] = ml[q];
                ov[k] = *reinterpret_cast<const float4*>(po + (int64_t)q * D);
            }
        }
    }
    if (Pb == 0) {
        if (pg == 0) { out[0] = 0; out[1] = 0; out[2] = 0; out[3] = 0; }
        return;
    }

    // Combine with a running max (exp2 domain), batch by batch.
    float M = -FLT_MAX, W = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q0 = pg;;) {
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (q0 + 16 * k >= Pb) break;
            const float mn = fmaxf(M, mlv[k].x);
            const float sc = fast_exp2(M - mn);
            const float w = mlv[k].y * fast_exp2(mlv[k].x - mn);
            O.x = O.x * sc + w * ov[k].x; O.y = O.y * sc + w * ov[k].y;
            O.z = O.z * sc + w * ov[k].z; O.w = O.w * sc + w * ov[k].w;
            W = W * sc + w;
            M = mn;
        }
        q0 += 16 * kBatch;
        if (q0 >= Pb) break;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int q = q0 + 16 * k;
            if (q < Pb) {
                mlv[k] = ml[q];
                ov[k] = *reinterpret_cast<const float4*>(po + (int64_t)q * D);
            }
        }
    }
    red_o[pg][d4] = O;
    red_mw[pg][d4] = make_float2(M, W);
    __syncthreads();
    if (pg == 0) {
        // combine the 16 partition groups in a fixed order
        float Mg = -FLT_MAX;
#pragma unroll
        for (int k = 0; k < 16; ++k) Mg = fmaxf(Mg, red_mw[k][d4].x);
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        float ws = 0.f;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const float2 mw = red_mw[k][d4];
            const float4 t = red_o[k][d4];
            const float f = fast_exp2(mw.x - Mg);
            s.x += f * t.x; s.y += f * t.y; s.z += f * t.z; s.w += f * t.w;
            ws += f * mw.y;
        }
        // a row with no token at all has ws == 0: zeros
        out[0] = Elt::from_float(ws > 0.f ? s.x / ws : 0.f);
        out[1] = Elt::from_float(ws > 0.f ? s.y / ws : 0.f);
        out[2] = Elt::from_float(ws > 0.f ? s.z / ws : 0.f);
        out[3] = Elt::from_float(ws > 0.f ? s.w / ws : 0.f);
    }
}

// batch: B * q_len (grid z runs over sequences and their query positions)
template <typename Elt, int D>
static hipError_t launch_merge_t(const DecodeParams& p, int batch, hipStream_t stream) {
    const dim3 grid(D / 64, p.num_q_heads, batch);
    // loading ahead of seq_lens pays when the merge is latency-bound (few
    // rows); with many rows it would read every partition slot, live or not
    if ((int64_t)batch * p.num_q_heads <= 256)
        hipLaunchKernelGGL((merge_kernel<Elt, D, true>), grid, dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((merge_kernel<Elt, D, false>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_merge(int dtype, int head_size, const DecodeParams& p, int batch,
                        hipStream_t stream) {
    if (dtype == PDA_BF16) {
        switch (head_size) {
            case 64: return launch_merge_t<BF16, 64>(p, batch, stream);
            case 128: return launch_merge_t<BF16, 128>(p, batch, stream);
            case 256: return launch_merge_t<BF16, 256>(p, batch, stream);
        }
    } else {
        switch (head_size) {
            case 64: return launch_merge_t<FP16, 64>(p, batch, stream);
            case 128: return launch_merge_t<FP16, 128>(p, batch, stream);
            case 256: return launch_merge_t<FP16, 256>(p, batch, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace pda

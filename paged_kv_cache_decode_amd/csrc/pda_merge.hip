// Log-sum-exp merge of split-KV partials, for gfx950.
//
// The context of a (sequence, KV head) is split into P partitions (the
// split-KV decode of page "Hybrid-SSM decode rate on dual Radeon cards": the
// KV range is split over more workgroups and reduced afterwards).  Partition
// p of query head h left a normalised fp32 output o_p, its max score m_p (exp2
// domain) and its denominator l_p.  The exact softmax over the union is
//     M = max_p m_p,   w_p = l_p * 2^(m_p - M),   out = sum_p w_p o_p / sum_p w_p
// over the partitions that hold tokens (p < ceil(L / T_p)); empty partitions
// are never read.  L == 0 gives a zero row.
//
// One workgroup of 256 threads per (64-element chunk of D, query head,
// sequence): 16 lanes x 4 elements cover the chunk, 16 partition groups
// stride over p, and the groups are summed in a fixed order through LDS.
#include "pda_device.h"

namespace pda {

template <typename Elt, int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p) {
    __shared__ float red_m[4];
    __shared__ float4 red_o[16][16];
    __shared__ float red_w[16][16];
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, d4 = tid & 15, pg = tid >> 4;
    const int L = context_len(p, b);
    const int Pb = min(p.num_partitions, (L + p.tokens_per_part - 1) / p.tokens_per_part);
    const int64_t row = (int64_t)b * p.num_q_heads + h;
    uint16_t* out = static_cast<uint16_t*>(p.out) + row * D + chunk * 64 + d4 * 4;

    if (Pb == 0) {
        if (pg == 0) { out[0] = 0; out[1] = 0; out[2] = 0; out[3] = 0; }
        return;
    }
    const float* ml = p.ws_ml + row * p.num_partitions * 2;
    const float* po = p.ws_o + row * p.num_partitions * D + chunk * 64 + d4 * 4;

    // M = max over non-empty partitions
    float mloc = -INFINITY;
    for (int q = tid; q < Pb; q += 256) mloc = fmaxf(mloc, ml[2 * q]);
#pragma unroll
    for (int x = 1; x < 64; x <<= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, x));
    if ((tid & 63) == 0) red_m[tid >> 6] = mloc;
    __syncthreads();
    const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));

    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float wsum = 0.f;
#pragma unroll 4
    for (int q = pg; q < Pb; q += 16) {
        const float w = ml[2 * q + 1] * exp2f(ml[2 * q] - M);
        const float4 v = *reinterpret_cast<const float4*>(po + (int64_t)q * D);
        o.x += w * v.x; o.y += w * v.y; o.z += w * v.z; o.w += w * v.w;
        wsum += w;
    }
    red_o[pg][d4] = o;
    red_w[pg][d4] = wsum;
    __syncthreads();
    if (pg == 0) {
        float4 s = red_o[0][d4];
        float ws = red_w[0][d4];
#pragma unroll
        for (int k = 1; k < 16; ++k) {
            const float4 t = red_o[k][d4];
            s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
            ws += red_w[k][d4];
        }
        out[0] = Elt::from_float(s.x / ws);
        out[1] = Elt::from_float(s.y / ws);
        out[2] = Elt::from_float(s.z / ws);
        out[3] = Elt::from_float(s.w / ws);
    }
}

template <typename Elt, int D>
static hipError_t launch_merge_t(const DecodeParams& p, int batch, hipStream_t stream) {
    const dim3 grid(D / 64, p.num_q_heads, batch);
    hipLaunchKernelGGL((merge_kernel<Elt, D>), grid, dim3(256), 0, stream, p);
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

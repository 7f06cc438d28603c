// A decode step driven through the C ABI alone (include/pda.h): device
// buffers from hipMalloc, the library's plan and workspace queries, the call,
// and the result checked against the fp32 CPU oracle (oracle/liboracle.so,
// test infrastructure).  No Python and no torch anywhere on the path.
//
// Inputs are seeded and synthetic: q, K and V uniform in [-2, 2) rounded to
// bf16 (nearest even), a random permutation of the pool's block ids dealt out
// in sequence order, NaN in every unwritten tail slot and unreferenced block
// (the unwritten-tail fault test of page "vLLM's custom ROCm paged-attention
// kernel wins all sixty cells", section 5: no NaN may reach the output).
//
//   decode_from_c              GPU run: every case under the device plan and
//                              forced plans; exit 0 when all pass
//   decode_from_c --host-only  the host-side validation paths only (no GPU)
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "pda.h"

extern "C" int oracle_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                             const int32_t* seq_lens, const int64_t* kv_off, const float* q,
                             const float* k, const float* v, float scale, float* out,
                             int32_t nthreads);

namespace {

// splitmix64: a counter-based generator, the inputs' only source of randomness
struct Rng {
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9e3779b97f4a7c15ull);
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        return z ^ (z >> 31);
    }
    float uniform(float lo, float hi) {  // 24 random bits
        return lo + (hi - lo) * (float)(next() >> 40) * (1.0f / 16777216.0f);
    }
};

uint16_t to_bf16(float x) {  // round to nearest even (finite inputs)
    uint32_t u;
    std::memcpy(&u, &x, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
float from_bf16(uint16_t h) {
    const uint32_t u = (uint32_t)h << 16;
    float x;
    std::memcpy(&x, &u, 4);
    return x;
}
constexpr uint16_t kBf16NaN = 0x7fc0;

#define HIP_OK(call)                                                          \
    do {                                                                      \
        hipError_t e_ = (call);                                               \
        if (e_ != hipSuccess) {                                               \
            std::printf("HIP error %s at %s\n", hipGetErrorString(e_), #call); \
            return false;                                                     \
        }                                                                     \
    } while (0)

struct Case {
    const char* name;
    int B, Hq, Hkv, D, bs;
    std::vector<int> lens;
};

// One case: build the paged inputs, decode under each plan, compare.
bool run_case(const Case& c, uint64_t seed) {
    const int B = c.B, Hq = c.Hq, Hkv = c.Hkv, D = c.D, bs = c.bs;
    int max_len = 0, used = 0, mbs = 1;
    for (int L : c.lens) {
        max_len = L > max_len ? L : max_len;
        used += (L + bs - 1) / bs;
        mbs = (L + bs - 1) / bs > mbs ? (L + bs - 1) / bs : mbs;
    }
    const int NB = used + 2;  // two blocks nobody references
    Rng rng{seed};

    // q, and the contiguous K/V the oracle reads ([Hkv][L_b][D] per sequence)
    std::vector<uint16_t> q16((size_t)B * Hq * D);
    std::vector<float> qf(q16.size());
    for (size_t i = 0; i < q16.size(); ++i) {
        q16[i] = to_bf16(rng.uniform(-2.f, 2.f));
        qf[i] = from_bf16(q16[i]);
    }
    std::vector<int64_t> kv_off(B);
    int64_t total = 0;
    for (int b = 0; b < B; ++b) {
        kv_off[b] = total;
        total += (int64_t)Hkv * c.lens[b] * D;
    }
    std::vector<float> kf(total), vf(total);

    // the pool, NaN everywhere first, and the permuted table
    const size_t pool = (size_t)NB * Hkv * bs * D;
    std::vector<uint16_t> k16(pool, kBf16NaN), v16(pool, kBf16NaN);
    std::vector<int> perm(NB);
    for (int i = 0; i < NB; ++i) perm[i] = i;
    for (int i = NB - 1; i > 0; --i) {
        const int j = (int)(rng.next() % (uint64_t)(i + 1));
        const int t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
    std::vector<int32_t> table((size_t)B * mbs, 0), lens(c.lens.begin(), c.lens.end());
    int next = 0;
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < (c.lens[b] + bs - 1) / bs; ++j) table[(size_t)b * mbs + j] = perm[next++];
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < Hkv; ++g)
            for (int t = 0; t < c.lens[b]; ++t)
                for (int d = 0; d < D; ++d) {
                    const int64_t o = kv_off[b] + ((int64_t)g * c.lens[b] + t) * D + d;
                    const uint16_t kh = to_bf16(rng.uniform(-2.f, 2.f));
                    const uint16_t vh = to_bf16(rng.uniform(-2.f, 2.f));
                    kf[o] = from_bf16(kh);
                    vf[o] = from_bf16(vh);
                    const int blk = table[(size_t)b * mbs + t / bs];
                    const size_t p = (((size_t)blk * Hkv + g) * bs + t % bs) * D + d;
                    k16[p] = kh;
                    v16[p] = vh;
                }

    const float scale = 1.0f / std::sqrt((float)D);
    std::vector<float> ref((size_t)B * Hq * D);
    if (oracle_decode(B, Hq, Hkv, D, lens.data(), kv_off.data(), qf.data(), kf.data(), vf.data(),
                      scale, ref.data(), 0) != 0) {
        std::printf("%s: oracle failed\n", c.name);
        return false;
    }
    float ref_max = 0.f;
    for (float x : ref) ref_max = std::fabs(x) > ref_max ? std::fabs(x) : ref_max;

    pda_shape_t s{};
    s.num_seqs = B;
    s.num_q_heads = Hq;
    s.num_kv_heads = Hkv;
    s.head_size = D;
    s.block_size = bs;
    s.num_blocks = NB;
    s.max_blocks_per_seq = mbs;
    s.max_seq_len = max_len;
    s.dtype = PDA_BF16;
    s.q_len = 1;
    s.kv_dtype = PDA_KV_SAME;
    if (pda_check_shape(&s) != PDA_OK) {
        std::printf("%s: shape refused\n", c.name);
        return false;
    }

    void *dq, *dk, *dv, *dtab, *dlen, *dout;
    HIP_OK(hipMalloc(&dq, q16.size() * 2));
    HIP_OK(hipMalloc(&dk, pool * 2));
    HIP_OK(hipMalloc(&dv, pool * 2));
    HIP_OK(hipMalloc(&dtab, table.size() * 4));
    HIP_OK(hipMalloc(&dlen, lens.size() * 4));
    HIP_OK(hipMalloc(&dout, ref.size() * 2));
    HIP_OK(hipMemcpy(dq, q16.data(), q16.size() * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dk, k16.data(), pool * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dv, v16.data(), pool * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dtab, table.data(), table.size() * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dlen, lens.data(), lens.size() * 4, hipMemcpyHostToDevice));

    // the device plan, then forced ones: one partition, three with the merge
    // kernel, three with the fused merge
    pda_plan_t dev{};
    if (paged_decode_attn_plan(&s, &dev) != PDA_OK) {
        std::printf("%s: no device plan\n", c.name);
        return false;
    }
    const int span = (max_len + PDA_TP_ALIGN - 1) / PDA_TP_ALIGN * PDA_TP_ALIGN;
    const int t3 = ((max_len + 2) / 3 + PDA_TP_ALIGN - 1) / PDA_TP_ALIGN * PDA_TP_ALIGN;
    const pda_plan_t plans[4] = {dev,
                                 {1, span, dev.variant, PDA_MERGE_KERNEL, 0, 0},
                                 {3, t3, dev.variant, PDA_MERGE_KERNEL, 0, 0},
                                 {3, t3, dev.variant, PDA_MERGE_FUSED, 0, 0}};
    bool ok = true;
    std::vector<uint16_t> out16(ref.size());
    for (int k = 0; k < 4; ++k) {
        const pda_plan_t& pl = plans[k];
        const int64_t wsb = pda_workspace_bytes(&s, &pl);
        void* ws = nullptr;
        if (wsb > 0) {
            HIP_OK(hipMalloc(&ws, (size_t)wsb));
            if (paged_decode_attn_workspace_init(ws, wsb, nullptr) != PDA_OK) return false;
        }
        const int rc = k == 0 ? paged_decode_attn(&s, dq, dk, dv, (const int32_t*)dtab,
                                                  (const int32_t*)dlen, scale, dout, ws, wsb,
                                                  nullptr)
                              : paged_decode_attn_with_plan(&s, &pl, dq, dk, dv,
                                                            (const int32_t*)dtab,
                                                            (const int32_t*)dlen, scale, dout,
                                                            ws, wsb, nullptr);
        if (rc != PDA_OK) {
            std::printf("%s plan %d: %s\n", c.name, k, pda_status_string(rc));
            return false;
        }
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(out16.data(), dout, out16.size() * 2, hipMemcpyDeviceToHost));
        if (ws) HIP_OK(hipFree(ws));
        float err = 0.f;
        int nonfinite = 0;
        for (size_t i = 0; i < ref.size(); ++i) {
            const float g = from_bf16(out16[i]);
            if (!std::isfinite(g)) ++nonfinite;
            err = std::fabs(g - ref[i]) > err ? std::fabs(g - ref[i]) : err;
        }
        const float rel = ref_max > 0.f ? err / ref_max : err;
        const bool pass = nonfinite == 0 && rel <= 1e-2f;
        std::printf("%s plan %d (P=%d T_p=%d variant=%d merge=%d): rel-Linf %.3e, non-finite %d %s\n",
                    c.name, k, pl.num_partitions, pl.tokens_per_partition, pl.variant, pl.merge,
                    rel, nonfinite, pass ? "ok" : "FAIL");
        ok = ok && pass;
    }
    HIP_OK(hipFree(dq));
    HIP_OK(hipFree(dk));
    HIP_OK(hipFree(dv));
    HIP_OK(hipFree(dtab));
    HIP_OK(hipFree(dlen));
    HIP_OK(hipFree(dout));
    return ok;
}

// Validation on the host: each bad argument gives its status and nothing is
// launched (no device is touched on these paths).
bool host_only() {
    pda_shape_t s{};
    s.num_seqs = 2;
    s.num_q_heads = 8;
    s.num_kv_heads = 4;
    s.head_size = 128;
    s.block_size = 16;
    s.num_blocks = 8;
    s.max_blocks_per_seq = 3;
    s.max_seq_len = 40;
    s.dtype = PDA_BF16;
    s.q_len = 1;
    bool ok = pda_check_shape(&s) == PDA_OK;
    pda_shape_t bad = s;
    bad.head_size = 96;
    ok = ok && pda_check_shape(&bad) == PDA_ERR_UNSUPPORTED;
    bad = s;
    bad.num_q_heads = 6;  // not a multiple of Hkv
    ok = ok && pda_check_shape(&bad) == PDA_ERR_INVALID;
    pda_plan_t pl{};
    ok = ok && pda_plan_for_cus(&s, 256, &pl) == PDA_OK && pl.num_partitions >= 1;
    char dummy[64];  // non-null host addresses: these calls stop before any launch
    ok = ok && paged_decode_attn_with_plan(&s, &pl, nullptr, dummy, dummy, (int32_t*)dummy,
                                           (int32_t*)dummy, 1.f, dummy, dummy, 1 << 20,
                                           nullptr) == PDA_ERR_INVALID;
    pda_plan_t p3{3, 64, PDA_VARIANT_MFMA, PDA_MERGE_KERNEL, 0, 0};
    ok = ok && pda_workspace_bytes(&s, &p3) > 0;
    ok = ok && paged_decode_attn_with_plan(&s, &p3, dummy, dummy, dummy, (int32_t*)dummy,
                                           (int32_t*)dummy, 1.f, dummy, dummy, 16,
                                           nullptr) == PDA_ERR_WORKSPACE;
    pda_plan_t p0{0, 64, PDA_VARIANT_MFMA, PDA_MERGE_KERNEL, 0, 0};
    ok = ok && paged_decode_attn_with_plan(&s, &p0, dummy, dummy, dummy, (int32_t*)dummy,
                                           (int32_t*)dummy, 1.f, dummy, dummy, 1 << 20,
                                           nullptr) == PDA_ERR_INVALID;
    std::printf("host-only validation: %s (%s)\n", ok ? "ok" : "FAIL", pda_build_id());
    return ok;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc > 1 && std::strcmp(argv[1], "--host-only") == 0) return host_only() ? 0 : 1;
    const Case cases[] = {
        {"tiny 8/4 heads, D 128, block 16", 2, 8, 4, 128, 16, {17, 40}},
        {"24/4 heads, D 256, block 784", 3, 24, 4, 256, 784, {500, 1568, 785}},
        {"8/8 heads, D 64, block 5", 2, 8, 8, 64, 5, {1, 333}},
    };
    bool ok = true;
    uint64_t seed = 20261202;
    for (const Case& c : cases) {
        std::printf("== %s\n", c.name);
        std::fflush(stdout);
        ok = run_case(c, seed++) && ok;
    }
    std::printf("%s\n", ok ? "all ok" : "FAILED");
    return ok ? 0 : 1;
}

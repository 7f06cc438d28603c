// CPU harness for the library's host runtime (pda_host.cpp: validation, the
// partition plan, the workspace layout and the launch sequence), built with
// g++ under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py.  No GPU: the kernel launchers and the two HIP
// device queries the runtime makes are stubs defined here.
//
// The launcher stubs replay, on the host, every workspace, output, query and
// block-table index the kernels of a launch address (one workgroup per
// (KV head, sequence, partition), R = q_len * G rows per unit), against
// buffers allocated with exactly the sizes the caller is told to provide:
// the output and query [B][q_len][Hq][D], the table [B][MBS], and a workspace
// of exactly pda_workspace_bytes(shape, plan).  Any index outside those
// buffers is a heap overflow that AddressSanitizer reports, so the host's
// workspace sizing and layout are checked against the kernels' indexing.
// A fuzz pass then feeds random, mostly invalid shapes and plans to every
// pure entry point; UndefinedBehaviorSanitizer (signed overflow, division by
// zero, shifts) aborts on any undefined arithmetic.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "pda_common.h"

static int g_cu_count = 256;
static long g_launches = 0, g_merges = 0, g_fused_units = 0;

extern "C" hipError_t hipGetDevice(int* dev) {
    *dev = 0;
    return hipSuccess;
}
extern "C" hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
    *value = g_cu_count;
    return hipSuccess;
}
// "device" buffers are host memory here
extern "C" hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind,
                                     hipStream_t) {
    memcpy(dst, src, bytes);
    return hipSuccess;
}
extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

namespace pda {

// row index of unit (b, g), row r (query position r / G, head r % G) among
// the [B][q_len][Hq] rows, as the kernels compute it
static int64_t row_of(const DecodeParams& p, int b, int g, int r) {
    const int i = r / p.group, h = r % p.group;
    return ((int64_t)b * p.q_len + i) * p.num_q_heads + g * p.group + h;
}

static volatile float g_sink;

// Every address the decode kernel of this launch touches outside the KV pools.
static hipError_t replay_decode(const DecodeParams& p, int batch, int head_size) {
    ++g_launches;
    const int D = head_size, P = p.num_partitions;
    const uint16_t* q = static_cast<const uint16_t*>(p.q);
    uint16_t* out = static_cast<uint16_t*>(p.out);
    float acc = 0.f;
    for (int b = 0; b < batch; ++b) {
        acc += (float)p.seq_lens[b];
        // the aligned kernels read table entries anywhere in the row
        acc += (float)p.block_table[(int64_t)b * p.max_blocks_per_seq + p.max_blocks_per_seq - 1];
        for (int g = 0; g < p.num_kv_heads; ++g) {
            for (int r = 0; r < p.rows; ++r) {
                const int64_t row = row_of(p, b, g, r);
                acc += (float)q[row * D] + (float)q[row * D + D - 1];
                if (P == 1) {
                    out[row * D] = 0;
                    out[row * D + D - 1] = 0;
                    continue;
                }
                for (int part = 0; part < P; ++part) {
                    const int64_t prow = row * P + part;
                    p.ws_o[prow * D] = 0.f;
                    p.ws_o[prow * D + D - 1] = 0.f;
                    p.ws_ml[prow * 2] = 0.f;
                    p.ws_ml[prow * 2 + 1] = 0.f;
                }
                if (p.fused_merge) {  // the last workgroup of the unit writes out
                    out[row * D] = 0;
                    out[row * D + D - 1] = 0;
                }
            }
            if (P > 1 && p.fused_merge) {
                ++g_fused_units;
                p.counters[(int64_t)b * p.num_kv_heads + g] = 0;
            }
        }
    }
    g_sink = acc;
    return hipSuccess;
}

#define PDA_STUB_VALU(DT, HD)                                                                  \
    hipError_t launch_decode_valu_##DT##_##HD(int, bool, const DecodeParams& p, int batch,     \
                                              hipStream_t, hipEvent_t, hipEvent_t) {           \
        return replay_decode(p, batch, HD);                                                    \
    }
#define PDA_STUB_MFMA(NAME, DT, HD)                                                            \
    hipError_t NAME##_##DT##_##HD(bool, const DecodeParams& p, int batch, hipStream_t,         \
                                  hipEvent_t, hipEvent_t) {                                    \
        return replay_decode(p, batch, HD);                                                    \
    }
PDA_STUB_VALU(0, 64) PDA_STUB_VALU(0, 128) PDA_STUB_VALU(0, 256)
PDA_STUB_VALU(1, 64) PDA_STUB_VALU(1, 128) PDA_STUB_VALU(1, 256)
PDA_STUB_MFMA(launch_decode_mfma, 0, 64) PDA_STUB_MFMA(launch_decode_mfma, 0, 128)
PDA_STUB_MFMA(launch_decode_mfma, 0, 256) PDA_STUB_MFMA(launch_decode_mfma, 1, 64)
PDA_STUB_MFMA(launch_decode_mfma, 1, 128) PDA_STUB_MFMA(launch_decode_mfma, 1, 256)
PDA_STUB_MFMA(launch_decode_mfma8, 0, 64) PDA_STUB_MFMA(launch_decode_mfma8, 0, 128)
PDA_STUB_MFMA(launch_decode_mfma8, 0, 256) PDA_STUB_MFMA(launch_decode_mfma8, 1, 64)
PDA_STUB_MFMA(launch_decode_mfma8, 1, 128) PDA_STUB_MFMA(launch_decode_mfma8, 1, 256)

// the merge kernel: grid (D/64, Hq, B * q_len); reads every partition slot
// of its row, writes the row
hipError_t launch_merge(int, int head_size, const DecodeParams& p, int batch, hipStream_t) {
    ++g_merges;
    const int D = head_size, P = p.num_partitions;
    uint16_t* out = static_cast<uint16_t*>(p.out);
    float acc = 0.f;
    for (int bi = 0; bi < batch; ++bi) {
        acc += (float)p.seq_lens[bi / p.q_len];
        for (int h = 0; h < p.num_q_heads; ++h) {
            const int64_t row = (int64_t)bi * p.num_q_heads + h;
            for (int part = 0; part < P; ++part) {
                acc += p.ws_o[(row * P + part) * D + D - 1] + p.ws_ml[(row * P + part) * 2 + 1];
            }
            out[row * D + D - 1] = 0;
        }
    }
    g_sink = acc;
    return hipSuccess;
}

hipError_t launch_zero_fill(void* dst, int64_t bytes, hipStream_t) {
    memset(dst, 0, (size_t)bytes);
    return hipSuccess;
}

hipError_t launch_trace(int, int, bool, int, const DecodeParams& p, int batch, hipStream_t) {
    // trace_range [B][Hkv][P][2]
    for (int b = 0; b < batch; ++b)
        for (int g = 0; g < p.num_kv_heads; ++g)
            for (int part = 0; part < p.num_partitions; ++part) {
                const int64_t u = ((int64_t)b * p.num_kv_heads + g) * p.num_partitions + part;
                p.trace_range[2 * u] = 0;
                p.trace_range[2 * u + 1] = 0;
            }
    return hipSuccess;
}

}  // namespace pda

// ---- driver -------------------------------------------------------------
static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {  // splitmix64
    uint64_t z = (g_rng += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int rnd(int lo, int hi) { return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)); }
static int pick(const std::vector<int>& v) { return v[next_u64() % v.size()]; }

static int failures = 0;
#define EXPECT(c)                                                                \
    do {                                                                         \
        if (!(c)) {                                                              \
            fprintf(stderr, "FAILED %s at line %d\n", #c, __LINE__);             \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

// One decode call under `plan` with caller buffers of exactly the documented
// sizes (fake K/V pool pointers: the stubs never touch the pools).  Returns
// the call's status; a workspace one byte short must be refused before any
// launch.  Plans whose buffers would exceed 256 MiB are skipped (-100).
static int call_with_plan(const pda_shape_t& s, const pda_plan_t& plan, bool device_plan) {
    const int64_t need = pda_workspace_bytes(&s, &plan);
    if (need < 0) return (int)need;
    const int64_t qlen = s.q_len > 1 ? s.q_len : 1;
    const int64_t rows = (int64_t)s.num_seqs * qlen * s.num_q_heads;
    if (need > ((int64_t)1 << 28) || rows * s.head_size > ((int64_t)1 << 26)) return -100;
    std::vector<uint16_t> q(rows * s.head_size), out(rows * s.head_size);
    std::vector<int32_t> table((int64_t)s.num_seqs * s.max_blocks_per_seq, 0);
    std::vector<int32_t> lens(s.num_seqs, s.max_seq_len);
    // the workspace exactly as large as the plan says (malloc'd: ASan guards it)
#ifdef PDA_HARNESS_PLANT_SHORT_WORKSPACE
    // a planted mistake, for the test that the instrument sees it: the
    // caller's workspace 4 bytes short of what the runtime was told
    char* ws = need > 0 ? static_cast<char*>(calloc(1, (size_t)need - 4)) : nullptr;
#else
    char* ws = need > 0 ? static_cast<char*>(calloc(1, (size_t)need)) : nullptr;
#endif
    static char pool[64];
    int rc;
    if (device_plan)
        rc = paged_decode_attn(&s, q.data(), pool, pool, table.data(), lens.data(), 0.1f,
                               out.data(), ws, need, nullptr);
    else
        rc = paged_decode_attn_with_plan(&s, &plan, q.data(), pool, pool, table.data(),
                                         lens.data(), 0.1f, out.data(), ws, need, nullptr);
    if (rc == PDA_OK && need > 0) {
        const long before = g_launches;
        const int rc2 = paged_decode_attn_with_plan(&s, &plan, q.data(), pool, pool, table.data(),
                                                    lens.data(), 0.1f, out.data(), ws, need - 1,
                                                    nullptr);
        EXPECT(rc2 == PDA_ERR_WORKSPACE);
        EXPECT(g_launches == before);
    }
    free(ws);
    return rc;
}

static pda_shape_t valid_shape() {
    pda_shape_t s{};
    const int G = pick({1, 2, 3, 4, 5, 6, 7, 8, 11, 12, 16});
    s.num_kv_heads = pick({1, 2, 4, 8, 16});
    s.num_q_heads = G * s.num_kv_heads;
    s.num_seqs = pick({1, 2, 3, 8, 64});
    s.head_size = pick({64, 128, 256});
    s.block_size = pick({1, 5, 16, 48, 784});
    s.dtype = rnd(0, 1);
    s.q_len = rnd(0, 3) == 0 ? rnd(1, 32 / G > 0 ? 32 / G : 1) : 1;
    s.sliding_window = rnd(0, 3) == 0 ? rnd(1, 4096) : 0;
    s.kv_dtype = rnd(0, 3) == 0 ? PDA_KV_FP8_E4M3 : PDA_KV_SAME;
    s.k_scale = 0.5f;
    s.v_scale = 0.25f;
    s.max_seq_len = pick({0, 1, 17, 500, 4096, 32768});
    s.max_blocks_per_seq = s.max_seq_len / s.block_size + 1 + rnd(0, 2);
    s.num_blocks = s.max_blocks_per_seq * s.num_seqs + 1;
    return s;
}

int main(int argc, char** argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 2000;

    // 1. the five workload shapes and the device plan at several CU counts
    struct Named { const char* name; pda_shape_t s; };
    std::vector<Named> named;
    auto mk = [](int B, int Hq, int Hkv, int D, int bs, int L) {
        pda_shape_t s{};
        s.num_seqs = B; s.num_q_heads = Hq; s.num_kv_heads = Hkv; s.head_size = D;
        s.block_size = bs; s.max_seq_len = L; s.max_blocks_per_seq = (L + bs - 1) / bs;
        s.num_blocks = s.max_blocks_per_seq * B + 1; s.dtype = PDA_BF16; s.q_len = 1;
        s.k_scale = s.v_scale = 1.f;
        return s;
    };
    named.push_back({"tiny", mk(2, 8, 4, 128, 16, 40)});
    named.push_back({"sweep", mk(1, 32, 8, 128, 16, 32768)});
    named.push_back({"gemma B8", mk(8, 32, 16, 128, 16, 32768)});
    named.push_back({"low-parallelism", mk(1, 24, 4, 256, 784, 32768)});
    named.push_back({"mixed B64", mk(64, 32, 8, 128, 16, 32767)});
    // the device's CU count is queried once and cached: the stub's 256
    for (auto& n : named) {
        pda_plan_t plan;
        EXPECT(paged_decode_attn_plan(&n.s, &plan) == PDA_OK);
        EXPECT(plan.cu_count == 256);
        EXPECT(call_with_plan(n.s, plan, true) == PDA_OK);
    }
    for (int cus : {1, 80, 256, 304, 1024}) {
        for (auto& n : named) {
            pda_plan_t plan;
            EXPECT(pda_plan_for_cus(&n.s, cus, &plan) == PDA_OK);
            EXPECT(plan.cu_count == cus);
            for (int merge : {PDA_MERGE_FUSED, PDA_MERGE_KERNEL}) {
                pda_plan_t p2 = plan;
                p2.merge = merge;
                const int rc = call_with_plan(n.s, p2, false);
                // the fused merge is refused only beyond its counter block
                EXPECT(rc == PDA_OK || (merge == PDA_MERGE_FUSED && rc == PDA_ERR_UNSUPPORTED));
            }
        }
    }
    // the workspace check counts the counters left non-zero, within the
    // counter block and the buffer's own size only
    {
        std::vector<int32_t> ws(16384 + 64, 0);
        int32_t nz = -1;
        EXPECT(paged_decode_attn_workspace_check(ws.data(), (int64_t)ws.size() * 4, nullptr, &nz) ==
               PDA_OK && nz == 0);
        ws[7] = 3;
        ws[16383] = -1;
        ws[16384] = 5;  // past the counter block: partial data, not counted
        EXPECT(paged_decode_attn_workspace_check(ws.data(), (int64_t)ws.size() * 4, nullptr, &nz) ==
               PDA_OK && nz == 2);
        EXPECT(paged_decode_attn_workspace_check(ws.data(), 28, nullptr, &nz) == PDA_OK && nz == 0);
        EXPECT(paged_decode_attn_workspace_check(ws.data(), 32, nullptr, &nz) == PDA_OK && nz == 1);
        EXPECT(paged_decode_attn_workspace_check(ws.data(), -4, nullptr, &nz) == PDA_ERR_INVALID);
        EXPECT(paged_decode_attn_workspace_check(nullptr, 4, nullptr, &nz) == PDA_ERR_INVALID);
        EXPECT(paged_decode_attn_workspace_check(ws.data(), 4, nullptr, nullptr) == PDA_ERR_INVALID);
        EXPECT(paged_decode_attn_workspace_check(nullptr, 0, nullptr, &nz) == PDA_OK && nz == 0);
    }
    // 2. random valid shapes under their plan, and under random forced plans
    int forced_ok = 0;
    for (int it = 0; it < iters; ++it) {
        pda_shape_t s = valid_shape();
        if (pda_check_shape(&s) != PDA_OK) continue;
        pda_plan_t plan;
        EXPECT(pda_plan_for_cus(&s, rnd(1, 512), &plan) == PDA_OK);
        const int rc = call_with_plan(s, plan, false);
        EXPECT(rc == PDA_OK || rc == -100);
        pda_plan_t forced = plan;
        forced.tokens_per_partition = PDA_TP_ALIGN * rnd(1, 40);
        forced.num_partitions = s.max_seq_len / forced.tokens_per_partition + 1 + rnd(0, 3);
        forced.merge = rnd(0, 1);
        forced.variant = rnd(1, 2);
        const int rc2 = call_with_plan(s, forced, false);
        EXPECT(rc2 == PDA_OK || rc2 == PDA_ERR_UNSUPPORTED || rc2 == -100);
        forced_ok += rc2 == PDA_OK;
        // null buffers are refused whatever the plan
        EXPECT(paged_decode_attn_with_plan(&s, &forced, nullptr, nullptr, nullptr, nullptr,
                                           nullptr, 0.f, nullptr, nullptr, 0, nullptr) < 0);
    }
    EXPECT(forced_ok > iters / 4);

    // 3. fuzz: arbitrary field values through every pure entry point
    const std::vector<int> wild = {INT32_MIN, -65536, -1, 0, 1, 2, 3, 7, 16, 64, 128, 256, 784,
                                   1000, 4096, 32768, 65535, 65536, 1 << 20, 1 << 30,
                                   INT32_MAX - 1, INT32_MAX};
    for (int it = 0; it < 20 * iters; ++it) {
        pda_shape_t s{};
        int32_t* f = &s.num_seqs;
        for (int k = 0; k < 12; ++k) f[k] = rnd(0, 2) == 0 ? pick(wild) : rnd(-3, 300);
        if (rnd(0, 1)) { s.head_size = pick({64, 128, 256}); s.dtype = rnd(0, 1); }
        if (rnd(0, 1)) { s.kv_dtype = rnd(0, 1); s.q_len = rnd(0, 4); }
        s.k_scale = rnd(0, 1) ? 1.f : -1.f;
        s.v_scale = 1.f;
        pda_check_shape(&s);
        pda_plan_t plan{};
        pda_plan_for_cus(&s, rnd(0, 2) ? rnd(1, 2048) : pick(wild), &plan);
        paged_decode_attn_plan(&s, &plan);
        paged_decode_attn_workspace_size(&s);
        pda_plan_t wp{};
        int32_t* pf = &wp.num_partitions;
        for (int k = 0; k < 5; ++k) pf[k] = rnd(0, 2) == 0 ? pick(wild) : rnd(-3, 300);
        pda_workspace_bytes(&s, &wp);
        pda_workspace_bytes(&s, &plan);
        paged_decode_attn_with_plan(&s, &wp, nullptr, nullptr, nullptr, nullptr, nullptr, 0.f,
                                    nullptr, nullptr, 0, nullptr);
    }
    EXPECT(pda_workspace_bytes(nullptr, nullptr) < 0);
    EXPECT(pda_check_shape(nullptr) == PDA_ERR_INVALID);
    EXPECT(pda_status_string(-99) != nullptr);
    EXPECT(pda_build_id() != nullptr);

    printf("launches %ld merges %ld fused units %ld failures %d\n", g_launches, g_merges,
           g_fused_units, failures);
    return failures == 0 ? 0 : 1;
}

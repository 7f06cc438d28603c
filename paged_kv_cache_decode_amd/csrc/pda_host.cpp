// Host runtime of libpda.so: argument validation, the partition plan, the
// workspace layout and the kernel launches behind the C ABI of pda.h.
#include <algorithm>
#include <atomic>
#include <math.h>
#include <stdint.h>
#include <vector>

#include "pda_common.h"

namespace pda {
// one definition per (element type, head size) translation unit
hipError_t launch_decode_valu_0_64(int, bool, const DecodeParams&, int, hipStream_t,
                                       hipEvent_t, hipEvent_t);
hipError_t launch_decode_valu_0_128(int, bool, const DecodeParams&, int, hipStream_t,
                                       hipEvent_t, hipEvent_t);
hipError_t launch_decode_valu_0_256(int, bool, const DecodeParams&, int, hipStream_t,
                                       hipEvent_t, hipEvent_t);
hipError_t launch_decode_valu_1_64(int, bool, const DecodeParams&, int, hipStream_t,
                                       hipEvent_t, hipEvent_t);
hipError_t launch_decode_valu_1_128(int, bool, const DecodeParams&, int, hipStream_t,
                                       hipEvent_t, hipEvent_t);
hipError_t launch_decode_valu_1_256(int, bool, const DecodeParams&, int, hipStream_t,
                                       hipEvent_t, hipEvent_t);

hipError_t launch_decode_mfma_0_64(bool, const DecodeParams&, int, hipStream_t, hipEvent_t,
                                       hipEvent_t);
hipError_t launch_decode_mfma_0_128(bool, const DecodeParams&, int, hipStream_t, hipEvent_t,
                                       hipEvent_t);
hipError_t launch_decode_mfma_0_256(bool, const DecodeParams&, int, hipStream_t, hipEvent_t,
                                       hipEvent_t);
hipError_t launch_decode_mfma_1_64(bool, const DecodeParams&, int, hipStream_t, hipEvent_t,
                                       hipEvent_t);
hipError_t launch_decode_mfma_1_128(bool, const DecodeParams&, int, hipStream_t, hipEvent_t,
                                       hipEvent_t);
hipError_t launch_decode_mfma_1_256(bool, const DecodeParams&, int, hipStream_t, hipEvent_t,
                                       hipEvent_t);

hipError_t launch_decode_mfma8_0_64(bool, const DecodeParams&, int, hipStream_t, hipEvent_t,
                                    hipEvent_t);
hipError_t launch_decode_mfma8_0_128(bool, const DecodeParams&, int, hipStream_t, hipEvent_t,
                                     hipEvent_t);
hipError_t launch_decode_mfma8_0_256(bool, const DecodeParams&, int, hipStream_t, hipEvent_t,
                                     hipEvent_t);
hipError_t launch_decode_mfma8_1_64(bool, const DecodeParams&, int, hipStream_t, hipEvent_t,
                                    hipEvent_t);
hipError_t launch_decode_mfma8_1_128(bool, const DecodeParams&, int, hipStream_t, hipEvent_t,
                                     hipEvent_t);
hipError_t launch_decode_mfma8_1_256(bool, const DecodeParams&, int, hipStream_t, hipEvent_t,
                                     hipEvent_t);

// fp8 KV: the translation units built with PDA_KV_FP8
static hipError_t launch_decode_mfma_fp8(int dtype, int head_size, bool aligned,
                                         const DecodeParams& p, int batch, hipStream_t s,
                                         hipEvent_t e0, hipEvent_t e1) {
    if (dtype == PDA_BF16) {
        if (head_size == 64) return launch_decode_mfma8_0_64(aligned, p, batch, s, e0, e1);
        if (head_size == 128) return launch_decode_mfma8_0_128(aligned, p, batch, s, e0, e1);
        if (head_size == 256) return launch_decode_mfma8_0_256(aligned, p, batch, s, e0, e1);
    } else {
        if (head_size == 64) return launch_decode_mfma8_1_64(aligned, p, batch, s, e0, e1);
        if (head_size == 128) return launch_decode_mfma8_1_128(aligned, p, batch, s, e0, e1);
        if (head_size == 256) return launch_decode_mfma8_1_256(aligned, p, batch, s, e0, e1);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(int dtype, int head_size, bool aligned, const DecodeParams& p,
                              int batch, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    if (dtype == PDA_BF16) {
        if (head_size == 64) return launch_decode_mfma_0_64(aligned, p, batch, s, e0, e1);
        if (head_size == 128) return launch_decode_mfma_0_128(aligned, p, batch, s, e0, e1);
        if (head_size == 256) return launch_decode_mfma_0_256(aligned, p, batch, s, e0, e1);
    } else {
        if (head_size == 64) return launch_decode_mfma_1_64(aligned, p, batch, s, e0, e1);
        if (head_size == 128) return launch_decode_mfma_1_128(aligned, p, batch, s, e0, e1);
        if (head_size == 256) return launch_decode_mfma_1_256(aligned, p, batch, s, e0, e1);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode_valu(int dtype, int head_size, int gpad, bool aligned,
                              const DecodeParams& p, int batch, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1) {
    if (dtype == PDA_BF16) {
        if (head_size == 64) return launch_decode_valu_0_64(gpad, aligned, p, batch, s, e0, e1);
        if (head_size == 128) return launch_decode_valu_0_128(gpad, aligned, p, batch, s, e0, e1);
        if (head_size == 256) return launch_decode_valu_0_256(gpad, aligned, p, batch, s, e0, e1);
    } else {
        if (head_size == 64) return launch_decode_valu_1_64(gpad, aligned, p, batch, s, e0, e1);
        if (head_size == 128) return launch_decode_valu_1_128(gpad, aligned, p, batch, s, e0, e1);
        if (head_size == 256) return launch_decode_valu_1_256(gpad, aligned, p, batch, s, e0, e1);
    }
    return hipErrorInvalidValue;
}

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int32_t> g_cu_count[kMaxDevices];
constexpr int64_t kMaxLdsBytes = 160 * 1024;  // a gfx950 workgroup may take all of a CU's LDS
constexpr int32_t kMaxSeqLen = 1 << 30;
constexpr int32_t kMaxGridYZ = 65535;
// LDS of one decode workgroup when the launch spans several rounds: with
// 160 KiB of LDS per CU, at most two such workgroups share a CU.  Two
// streaming workgroups per CU measured faster than three or four (mixed
// batch 64: 3% less time), the way one streaming read per CU beats several.
constexpr int32_t kLdsTwoPerCu = 56 * 1024;
// the VALU kernel is compiled for packed groups up to 8 heads
constexpr int kValuMaxGroup = 8;

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool kv_fp8(const pda_shape_t* s) { return s->kv_dtype == PDA_KV_FP8_E4M3; }
int64_t round256(int64_t x) { return cdiv64(x, 256) * 256; }
// the fixed block of arrival counters at the start of a workspace
constexpr int64_t kCounterBytes = (int64_t)PDA_FUSED_MAX_UNITS * 4;
static_assert(kCounterBytes % 256 == 0, "the partials after the counters stay 256-byte aligned");

// block sizes that are multiples of 16 tokens take the one-lookup-per-round
// path of the kernels (kAlignTokens)
bool block_aligned(const pda_shape_t* s) { return s->block_size % kAlignTokens == 0; }

int64_t table_capacity(const pda_shape_t* s, const pda_plan_t* pl) {
    return (int64_t)pl->tokens_per_partition / s->block_size + 2;
}

// Query rows per sequence (0 is read as 1) and rows per unit.
int64_t q_len_of(const pda_shape_t* s) { return s->q_len > 1 ? s->q_len : 1; }
int64_t rows_of(const pda_shape_t* s) {
    return q_len_of(s) * (s->num_q_heads / s->num_kv_heads);
}

// Tokens a partition grid must cover: the whole context, or the union of
// the rows' sliding windows rounded out to the 16-token grid its partitions
// start on.
int64_t plan_span(const pda_shape_t* s) {
    if (s->sliding_window > 0)
        return std::min<int64_t>(s->max_seq_len, (int64_t)s->sliding_window + q_len_of(s) - 1 +
                                                     kAlignTokens - 1);
    return s->max_seq_len;
}

int check_plan(const pda_shape_t* s, const pda_plan_t* pl) {
    if (!pl) return PDA_ERR_INVALID;
    if (pl->num_partitions < 1 || pl->tokens_per_partition < PDA_TP_ALIGN ||
        pl->tokens_per_partition % PDA_TP_ALIGN != 0)
        return PDA_ERR_INVALID;
    if ((int64_t)pl->num_partitions * pl->tokens_per_partition < plan_span(s))
        return PDA_ERR_INVALID;
    if ((int64_t)pl->num_partitions * pl->tokens_per_partition > (int64_t)2 * kMaxSeqLen ||
        pl->num_partitions > kMaxGridYZ)
        return PDA_ERR_UNSUPPORTED;
    if (pl->merge != PDA_MERGE_FUSED && pl->merge != PDA_MERGE_KERNEL) return PDA_ERR_INVALID;
    // the fused merge counts arrivals in the workspace's fixed counter block
    if (pl->merge == PDA_MERGE_FUSED && pl->num_partitions > 1 &&
        (int64_t)s->num_seqs * s->num_kv_heads > PDA_FUSED_MAX_UNITS)
        return PDA_ERR_UNSUPPORTED;
    const int R = (int)rows_of(s);
    if (pl->variant == PDA_VARIANT_VALU) {
        if (R > kValuMaxGroup || kv_fp8(s)) return PDA_ERR_UNSUPPORTED;
        const int64_t lds = (int64_t)decode_lds_bytes(s->head_size, valu_group_pad(R),
                                                      (int)table_capacity(s, pl));
        if (lds > kMaxLdsBytes) return PDA_ERR_UNSUPPORTED;
    } else if (pl->variant == PDA_VARIANT_MFMA) {
        const int eb = kv_fp8(s) ? 1 : 2;
        const int64_t lds = (int64_t)mfma_lds_bytes(
            s->head_size, eb,
            mfma_k_whole_rows(s->head_size, eb, pl->tokens_per_partition,
                              (int64_t)s->num_seqs * s->num_kv_heads),
            (int)table_capacity(s, pl));
        if (lds > kMaxLdsBytes) return PDA_ERR_UNSUPPORTED;
    } else {
        return PDA_ERR_INVALID;
    }
    return PDA_OK;
}

int device_cu_count(int32_t* cu) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PDA_ERR_DEVICE;
    if (dev < 0 || dev >= kMaxDevices) return PDA_ERR_DEVICE;
    int32_t c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c <= 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            return PDA_ERR_DEVICE;
        c = v;
        g_cu_count[dev].store(c, std::memory_order_relaxed);
    }
    *cu = c;
    return PDA_OK;
}

DecodeParams make_params(const pda_shape_t* s, const pda_plan_t* pl, float scale) {
    DecodeParams p{};
    // fp8 KV: q.(k_scale * K) = k_scale * (q.K), folded into the score scale
    p.scale_log2 = (kv_fp8(s) ? scale * s->k_scale : scale) * 1.4426950408889634f;
    p.v_scale = kv_fp8(s) ? s->v_scale : 1.0f;
    p.num_q_heads = s->num_q_heads;
    p.num_kv_heads = s->num_kv_heads;
    p.group = s->num_q_heads / s->num_kv_heads;
    p.block_size = s->block_size;
    p.max_blocks_per_seq = s->max_blocks_per_seq;
    p.max_seq_len = s->max_seq_len;
    p.window = s->sliding_window;
    p.q_len = (int32_t)q_len_of(s);
    p.rows = (int32_t)rows_of(s);
    p.num_blocks = s->num_blocks;
    p.num_partitions = pl->num_partitions;
    p.tokens_per_part = pl->tokens_per_partition;
    p.tbl_capacity = (int32_t)table_capacity(s, pl);
    p.bs_div = make_fastdiv((uint32_t)s->block_size);
    p.head_stride = s->block_size * s->head_size;
    p.block_stride = (int64_t)s->num_kv_heads * p.head_stride;
    return p;
}

}  // namespace

int run_decode(const pda_shape_t* s, const pda_plan_t* pl, const void* q,
                      const void* k_cache, const void* v_cache, const int32_t* block_table,
                      const int32_t* seq_lens, float scale, void* out, void* workspace,
                      int64_t workspace_bytes, void* stream, hipEvent_t ev0, hipEvent_t ev1) {
    int rc = pda_check_shape(s);
    if (rc != PDA_OK) return rc;
    rc = check_plan(s, pl);
    if (rc != PDA_OK) return rc;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return PDA_ERR_INVALID;
    const int64_t need = pda_workspace_bytes(s, pl);
    if (need > 0 && (!workspace || workspace_bytes < need)) return PDA_ERR_WORKSPACE;

    DecodeParams p = make_params(s, pl, scale);
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_table = block_table;
    p.seq_lens = seq_lens;
    p.out = out;
    if (need > 0) {
        const int64_t rows =
            (int64_t)s->num_seqs * q_len_of(s) * s->num_q_heads * pl->num_partitions;
        char* ws = static_cast<char*>(workspace);
        const int64_t o_bytes = round256(rows * s->head_size * 4);
        p.counters = reinterpret_cast<int32_t*>(ws);
        p.ws_o = reinterpret_cast<float*>(ws + kCounterBytes);
        p.ws_ml = reinterpret_cast<float*>(ws + kCounterBytes + o_bytes);
        p.fused_merge = pl->merge == PDA_MERGE_FUSED;
    }
    // more than two workgroups per CU in all: at most two resident at a time
    int32_t cu = 0;
    const int64_t wgs = (int64_t)pl->num_partitions * s->num_kv_heads * s->num_seqs;
    if (device_cu_count(&cu) == PDA_OK && wgs > 2 * (int64_t)cu) p.lds_floor = kLdsTwoPerCu;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool aligned = block_aligned(s);
    hipError_t e;
    if (pl->variant == PDA_VARIANT_MFMA)
        e = kv_fp8(s) ? launch_decode_mfma_fp8(s->dtype, s->head_size, aligned, p, s->num_seqs,
                                               st, ev0, ev1)
                      : launch_decode_mfma(s->dtype, s->head_size, aligned, p, s->num_seqs, st,
                                           ev0, ev1);
    else
        e = launch_decode_valu(s->dtype, s->head_size, valu_group_pad(p.rows), aligned, p,
                               s->num_seqs, st, ev0, ev1);
    if (e != hipSuccess) return PDA_ERR_LAUNCH;
    if (pl->num_partitions > 1 && pl->merge == PDA_MERGE_KERNEL) {
        e = launch_merge(s->dtype, s->head_size, p, (int)(s->num_seqs * q_len_of(s)), st);
        if (e != hipSuccess) return PDA_ERR_LAUNCH;
    }
    return PDA_OK;
}

}  // namespace pda

using namespace pda;

extern "C" {

int pda_check_shape(const pda_shape_t* s) {
    if (!s) return PDA_ERR_INVALID;
    if (s->num_seqs < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1 || s->block_size < 1 ||
        s->num_blocks < 1 || s->max_blocks_per_seq < 1 || s->max_seq_len < 0 ||
        s->sliding_window < 0 || s->q_len < 0)
        return PDA_ERR_INVALID;
    if (s->num_q_heads % s->num_kv_heads != 0) return PDA_ERR_INVALID;
    if (s->head_size != 64 && s->head_size != 128 && s->head_size != 256)
        return PDA_ERR_UNSUPPORTED;
    if (s->dtype != PDA_BF16 && s->dtype != PDA_FP16) return PDA_ERR_UNSUPPORTED;
    if (s->kv_dtype != PDA_KV_SAME && s->kv_dtype != PDA_KV_FP8_E4M3) return PDA_ERR_UNSUPPORTED;
    if (kv_fp8(s) && !(s->k_scale > 0.f && s->k_scale < INFINITY && s->v_scale > 0.f &&
                       s->v_scale < INFINITY))
        return PDA_ERR_INVALID;
    if (s->num_q_heads / s->num_kv_heads > PDA_MAX_GROUP) return PDA_ERR_UNSUPPORTED;
    if (s->q_len > PDA_MAX_ROWS || rows_of(s) > PDA_MAX_ROWS) return PDA_ERR_UNSUPPORTED;
    if ((int64_t)s->max_seq_len > (int64_t)s->max_blocks_per_seq * s->block_size)
        return PDA_ERR_INVALID;
    // one (block, KV head) slab of the pool, in elements, is a 32-bit kernel
    // parameter (the head stride)
    if ((int64_t)s->block_size * s->head_size > INT32_MAX) return PDA_ERR_UNSUPPORTED;
    if (s->max_seq_len > kMaxSeqLen) return PDA_ERR_UNSUPPORTED;
    if (s->num_seqs > kMaxGridYZ || s->num_kv_heads > kMaxGridYZ ||
        s->num_q_heads > kMaxGridYZ || (int64_t)s->num_seqs * q_len_of(s) > kMaxGridYZ)
        return PDA_ERR_UNSUPPORTED;
    return PDA_OK;
}

int pda_plan_for_cus(const pda_shape_t* s, int32_t cu_count, pda_plan_t* plan) {
    int rc = pda_check_shape(s);
    if (rc != PDA_OK) return rc;
    if (!plan || cu_count < 1) return PDA_ERR_INVALID;
    // the rule documented in pda.h
    const int64_t R = rows_of(s);
    const int64_t units = (int64_t)s->num_seqs * s->num_kv_heads;
    const bool mfma = kv_fp8(s) || R >= PDA_MFMA_MIN_GROUP;
    const int64_t bpt = (kv_fp8(s) ? 2 : 4) * (int64_t)s->head_size;
    const int64_t align = PDA_TP_ALIGN;
    const int64_t t_min = std::max(align, (PDA_WG_MIN_BYTES / bpt / align) * align);
    const int64_t t_many = std::max(t_min, (PDA_WG_MANY_BYTES / bpt / align) * align);
    const int64_t t_one = std::max(t_many, (PDA_WG_ONE_BYTES / bpt / align) * align);
    const int64_t p_fill = cdiv64(cu_count, units);
    int64_t tp = t_min;
    const int64_t span = plan_span(s);
    if (span > 0) {
        const int64_t t_fill = std::max(t_min, cdiv64(cdiv64(span, p_fill), align) * align);
        tp = t_fill <= t_one ? t_fill : t_many;
        // at most kMaxGridYZ partitions (a grid dimension)
        tp = std::max(tp, cdiv64(cdiv64(span, kMaxGridYZ), align) * align);
    }
    int64_t P = cdiv64(span, tp);
    if (P < 1) P = 1;
    plan->num_partitions = (int32_t)P;
    plan->tokens_per_partition = (int32_t)tp;
    plan->variant = mfma ? PDA_VARIANT_MFMA : PDA_VARIANT_VALU;
    // fused merge while the unit's partials are small enough for its last
    // workgroup to read them in one round of loads
    plan->merge = P > 1 && P <= PDA_FUSED_MAX_PARTS && units <= PDA_FUSED_MAX_UNITS &&
                          P * R * s->head_size * 4 <= PDA_FUSED_MAX_BYTES
                      ? PDA_MERGE_FUSED
                      : PDA_MERGE_KERNEL;
    plan->cu_count = cu_count;
    plan->workspace_bytes = pda_workspace_bytes(s, plan);
    return PDA_OK;
}

int64_t pda_workspace_bytes(const pda_shape_t* s, const pda_plan_t* pl) {
    if (!s || !pl) return PDA_ERR_INVALID;
    const int rc = pda_check_shape(s);
    if (rc != PDA_OK) return rc;
    // a valid shape has B * q_len <= 65535 and Hq <= 65535, so with at most
    // 65535 partitions the byte count below stays far inside int64
    if (pl->num_partitions < 1) return PDA_ERR_INVALID;
    if (pl->num_partitions > kMaxGridYZ) return PDA_ERR_UNSUPPORTED;
    if (pl->num_partitions == 1) return 0;
    const int64_t rows = (int64_t)s->num_seqs * q_len_of(s) * s->num_q_heads * pl->num_partitions;
    return kCounterBytes + round256(rows * s->head_size * 4) + round256(rows * 2 * 4);
}

int paged_decode_attn_workspace_init(void* workspace, int64_t bytes, void* stream) {
    if (bytes < 0 || (bytes > 0 && !workspace)) return PDA_ERR_INVALID;
    if (bytes == 0) return PDA_OK;
    // a fill kernel, not a memset: a caller may capture this into a HIP graph
    hipError_t e = launch_zero_fill(workspace, bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PDA_OK : PDA_ERR_LAUNCH;
}

int paged_decode_attn_workspace_check(const void* workspace, int64_t bytes, void* stream,
                                      int32_t* nonzero) {
    if (!nonzero || bytes < 0 || (bytes > 0 && !workspace)) return PDA_ERR_INVALID;
    *nonzero = 0;
    const int64_t n = std::min<int64_t>(bytes, kCounterBytes) / 4;
    if (n == 0) return PDA_OK;
    std::vector<int32_t> host((size_t)n);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(host.data(), workspace, (size_t)n * 4, hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return PDA_ERR_LAUNCH;
    int32_t count = 0;
    for (int32_t v : host) count += v != 0;
    *nonzero = count;
    return PDA_OK;
}

int paged_decode_attn_plan(const pda_shape_t* s, pda_plan_t* plan) {
    int rc = pda_check_shape(s);
    if (rc != PDA_OK) return rc;
    if (!plan) return PDA_ERR_INVALID;
    int32_t cu = 0;
    rc = device_cu_count(&cu);
    if (rc != PDA_OK) return rc;
    return pda_plan_for_cus(s, cu, plan);
}

int64_t paged_decode_attn_workspace_size(const pda_shape_t* s) {
    pda_plan_t pl;
    int rc = paged_decode_attn_plan(s, &pl);
    if (rc != PDA_OK) return rc;
    return pl.workspace_bytes;
}

int paged_decode_attn_with_plan(const pda_shape_t* s, const pda_plan_t* pl, const void* q,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* seq_lens,
                                float scale, void* out, void* workspace,
                                int64_t workspace_bytes, void* stream) {
    return run_decode(s, pl, q, k_cache, v_cache, block_table, seq_lens, scale, out, workspace,
                      workspace_bytes, stream, nullptr, nullptr);
}

int paged_decode_attn_timed(const pda_shape_t* s, const pda_plan_t* pl, const void* q,
                            const void* k_cache, const void* v_cache,
                            const int32_t* block_table, const int32_t* seq_lens, float scale,
                            void* out, void* workspace, int64_t workspace_bytes,
                            void* start_event, void* stop_event, void* stream) {
    pda_plan_t own;
    if (!pl) {
        int rc = paged_decode_attn_plan(s, &own);
        if (rc != PDA_OK) return rc;
        pl = &own;
    }
    return run_decode(s, pl, q, k_cache, v_cache, block_table, seq_lens, scale, out, workspace,
                      workspace_bytes, stream, static_cast<hipEvent_t>(start_event),
                      static_cast<hipEvent_t>(stop_event));
}

int paged_decode_attn(const pda_shape_t* s, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                      float scale, void* out, void* workspace, int64_t workspace_bytes,
                      void* stream) {
    int rc = pda_check_shape(s);
    if (rc != PDA_OK) return rc;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return PDA_ERR_INVALID;
    pda_plan_t pl;
    rc = paged_decode_attn_plan(s, &pl);
    if (rc != PDA_OK) return rc;
    return paged_decode_attn_with_plan(s, &pl, q, k_cache, v_cache, block_table, seq_lens, scale,
                                       out, workspace, workspace_bytes, stream);
}

int paged_decode_attn_trace(const pda_shape_t* s, const pda_plan_t* pl, int32_t rows,
                            const int32_t* block_table, const int32_t* seq_lens,
                            int32_t* trace_slot, int32_t* trace_part, int32_t* trace_range,
                            void* stream) {
    int rc = pda_check_shape(s);
    if (rc != PDA_OK) return rc;
    rc = check_plan(s, pl);
    if (rc != PDA_OK) return rc;
    if (!block_table || !seq_lens || !trace_slot || !trace_part || !trace_range)
        return PDA_ERR_INVALID;
    if (rows != 0 && rows != 1) return PDA_ERR_INVALID;
    // the recorded physical slot, block_id * bs + t % bs, is an int32
    if ((int64_t)s->num_blocks * s->block_size > INT32_MAX) return PDA_ERR_UNSUPPORTED;
    const int pattern = pl->variant == PDA_VARIANT_MFMA ? 1 + rows : 0;
    DecodeParams p = make_params(s, pl, 1.0f);
    p.block_table = block_table;
    p.seq_lens = seq_lens;
    p.trace_slot = trace_slot;
    p.trace_part = trace_part;
    p.trace_range = trace_range;
    const bool aligned = block_aligned(s);
    hipError_t e = launch_trace(s->head_size, kv_fp8(s) ? 1 : 2, aligned, pattern, p, s->num_seqs,
                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PDA_OK : PDA_ERR_LAUNCH;
}

const char* pda_status_string(int status) {
    switch (status) {
        case PDA_OK: return "ok";
        case PDA_ERR_INVALID: return "invalid argument";
        case PDA_ERR_UNSUPPORTED: return "unsupported shape or type";
        case PDA_ERR_WORKSPACE: return "workspace too small";
        case PDA_ERR_LAUNCH: return "kernel launch failed";
        case PDA_ERR_DEVICE: return "device query failed";
        default: return "unknown status";
    }
}

#ifndef PDA_BUILD_FLAGS
#define PDA_BUILD_FLAGS "unknown"
#endif
const char* pda_build_id(void) {
    return "libpda 0.4.0; target gfx950; variants valu|mfma; kv bf16|fp16|fp8e4m3; merge fused|kernel; flags " PDA_BUILD_FLAGS;
}

}  // extern "C"

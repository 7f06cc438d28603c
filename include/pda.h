/*
 * pda.h -- C ABI of the gfx950 paged-attention decode library (libpda.so).
 *
 * The operation (page "vLLM's custom ROCm paged-attention kernel wins all
 * sixty cells", section 1 "What is being measured"; page "Hybrid-SSM decode
 * rate on dual Radeon cards", the split-KV passage): pure decode, one query
 * token per sequence attending over that sequence's whole cached context,
 * where the context's K and V rows live in a block-paged cache addressed
 * through a per-sequence block table, with grouped-query attention (G = Hq/Hkv
 * query heads share one KV head).  For sequence b and query head h, with
 * L = seq_lens[b] and g = floor(h / G):
 *
 *     out[b,h,:] = softmax_t( scale * q[b,h,:] . K[b,g,t,:] ) @ V[b,g,t,:]
 *
 * over t in [0, L), where row t of sequence b lives in physical block
 * block_table[b][t / block_size] at slot t % block_size.  Slots at or past L
 * in the final block (the "unwritten tail" the first page's section 5 and
 * Figure 4 are about) never influence the output, whatever they hold: the
 * score of such a slot is excluded by a select, and its V row is never read.
 * The context of one (sequence, KV head) is split over P partitions of
 * T_p tokens (the split-KV decode of the second page), each partition yields
 * a partial (o, m, l), and a log-sum-exp merge combines them.
 *
 * Conventions for every entry point below:
 *  - All array arguments of paged_decode_attn* are DEVICE pointers on the
 *    current HIP device; shape and plan structs are HOST pointers.
 *  - The caller owns every buffer.  The library allocates no device memory,
 *    keeps no pointer after returning and has no global state except a
 *    per-device cache of the compute-unit count.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream).  No entry point synchronises the device, so a call can be
 *    captured into a HIP graph.
 *  - The return value is a status from host-side validation (PDA_OK or a
 *    negative PDA_ERR_*).  On an error nothing is launched.
 *
 * Sliding window (pda_shape_t.sliding_window = W > 0): the softmax runs over
 * the last W tokens only, t in [max(0, L - W), L) -- the sliding-window
 * layers of page "vLLM's custom ROCm paged-attention kernel wins all sixty
 * cells" (section 4, Figure 3: 1024-token scans).  Slots before the window
 * are never read, like the unwritten tail: their rows are redirected to the
 * window's first token and their scores are excluded by a select.  The
 * partitions then tile [base, L) with base = max(0, L - W) rounded down to a
 * multiple of 16, and the plan is sized for that span (see below).
 *
 * Multi-row decode (pda_shape_t.q_len = n > 1): each sequence brings n new
 * query rows at once -- the speculative or multi-token decode whose extra
 * rows the pages ask about (first page, section 6, "One machine, and the
 * model runner question") -- whose K and V are already in the cache as its
 * last n tokens.  Row i (0 <= i < n) sits at position L - n + i and attends
 * causally, to t in [lo_i, e_i) with e_i = L - n + i + 1 and lo_i = 0, or
 * max(0, e_i - W) with a sliding window; row n-1 is the plain decode over
 * the whole context.  q and out are then [B][n][Hq][D]; a unit (b, g) packs
 * R = n * G rows (row r = query position r / G, head r % G of the group), and
 * the kernels read every K/V byte once for all R rows.  A row whose range is
 * empty (L < n) yields zeros.
 *
 * fp8 KV cache (pda_shape_t.kv_dtype = PDA_KV_FP8_E4M3): k_cache and v_cache
 * hold one byte per element in the OCP FP8 E4M3 format (sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; subnormals; no infinity; S.1111.111 is
 * NaN; largest finite 448), with one scale per tensor: the element's value is
 * decode(byte) * k_scale (resp. v_scale).  This halves the KV bytes per token
 * (the fp8 KV the first page lists as untested, section 6).  q and out keep
 * the 16-bit type of `dtype`.  The kernels decode the bytes exactly (every
 * E4M3 value is a 16-bit and an fp32 value), fold k_scale into the score
 * scale and v_scale into the output; arithmetic is the same fp32 as for
 * 16-bit KV.  Only the MFMA variant serves fp8 KV.
 *
 * Device-data contract (not checked on the hot path; violating it is
 * undefined behaviour):
 *  - 0 <= seq_lens[b] <= max_seq_len <= max_blocks_per_seq * block_size;
 *  - block_table[b][j] is in [0, num_blocks) for j < ceil(seq_lens[b] / block_size);
 *    the whole row [b][0, max_blocks_per_seq) must be readable memory: the
 *    kernels may load entries at or past that index (the first tiles'
 *    entries are loaded before the length is known, and prefetches past a
 *    partition's end load clamped entries), but such an entry never
 *    addresses K or V, and block ids are clamped into [0, num_blocks);
 *  - K/V slots at or past seq_lens[b] may hold anything (NaN, Inf, garbage);
 *  - seq_lens[b] == 0 yields a zero output row.
 */
#ifndef PDA_H
#define PDA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PDA_OK                0
#define PDA_ERR_INVALID      -1  /* null pointer, non-positive size, Hq % Hkv != 0, bad plan */
#define PDA_ERR_UNSUPPORTED  -2  /* head size not 64/128/256, G > PDA_MAX_GROUP, bad dtype,
                                    block_size * head_size > INT32_MAX */
#define PDA_ERR_WORKSPACE    -3  /* workspace_bytes smaller than the plan needs */
#define PDA_ERR_LAUNCH       -4  /* a kernel launch failed (hipGetLastError) */
#define PDA_ERR_DEVICE       -5  /* the HIP device query failed */

/* ---- element types ----------------------------------------------------- */
/* q and out share one 16-bit type (dtype); k_cache and v_cache have it too
 * (kv_dtype PDA_KV_SAME) or are fp8 E4M3 bytes with per-tensor scales
 * (kv_dtype PDA_KV_FP8_E4M3).  Arithmetic is fp32 and the output is rounded
 * to nearest-even. */
#define PDA_BF16 0
#define PDA_FP16 1
#define PDA_KV_SAME      0
#define PDA_KV_FP8_E4M3  1

/* Largest supported query-to-KV head ratio G, and largest number of rows
 * R = q_len * G one unit packs (two 16-row matrix-core tiles). */
#define PDA_MAX_GROUP 16
#define PDA_MAX_ROWS  32

/* ---- kernel variants --------------------------------------------------- */
/* PDA_VARIANT_VALU: QK^T with packed dot2 and wavefront DPP reductions, PV
 *   with per-lane fp32 FMAs and fp32 weights; G <= PDA_VALU_MAX_GROUP.
 * PDA_VARIANT_MFMA: QK^T on v_mfma_f32_16x16x32 and PV on
 *   v_mfma_f32_16x16x16 (bf16/fp16 inputs, the packed rows padded to 16 per
 *   chunk, fp32 accumulation); the softmax weights enter PV rounded to the
 *   16-bit type (round to nearest even), and the denominator sums those
 *   rounded weights; R <= PDA_MAX_ROWS.
 * R = q_len * G is the number of rows a unit packs (G for plain decode);
 * the VALU variant serves R <= PDA_VALU_MAX_GROUP. */
#define PDA_VARIANT_VALU 1
#define PDA_VARIANT_MFMA 2
#define PDA_VALU_MAX_GROUP 8

/* ---- the plan -------------------------------------------------------------
 * A pure integer function of (num_seqs B, num_kv_heads Hkv, rows per unit
 * R = q_len * G, head_size D, span Lmax, compute-unit count C), where the
 * span is max_seq_len, or min(max_seq_len, W + q_len - 1 + 15) with a
 * sliding window W > 0 (the union of the rows' windows, rounded out to the
 * 16-token grid the partitions start on):
 *
 * Variant: MFMA for fp8 KV or if R >= PDA_MFMA_MIN_GROUP (the matrix cores
 *   take the per-row arithmetic, at any number of units and rounds); VALU
 *   for one row per unit, where the VALU kernel has the least to do.
 *   Measured against the VALU kernel over many units: 3.8 % faster for the
 *   mixed batch-64 layer (4 rows, 512 units), 9 % for 32 sequences of 4K
 *   tokens, 20 % at 6 rows and head size 256, 32 % at 8 rows.
 * Partition size, with ALIGN = PDA_TP_ALIGN and bpt = 4*D, or 2*D for fp8 KV
 *   (K and V bytes per token of one KV head):
 *   T_min  = max(ALIGN, floor(PDA_WG_MIN_BYTES  / bpt / ALIGN) * ALIGN)
 *   T_many = max(T_min, floor(PDA_WG_MANY_BYTES / bpt / ALIGN) * ALIGN)
 *   T_one  = max(T_many, floor(PDA_WG_ONE_BYTES / bpt / ALIGN) * ALIGN)
 *   P_fill = ceil(C / (B * Hkv))
 *   T_fill = max(T_min, roundup(ceil(Lmax / P_fill), ALIGN))
 *   T_p    = T_fill if T_fill <= T_one else T_many, raised if needed to
 *            roundup(ceil(Lmax / 65535), ALIGN) (at most 65535 partitions)
 *   P      = max(1, ceil(Lmax / T_p))
 *   i.e. when one round of C workgroups, one per compute unit, covers the
 *   job at <= 1 MiB each, use exactly that round (the split-KV partition
 *   count comes from the CU count); otherwise cut the job into 1 MiB
 *   workgroups and let the hardware dispatcher balance them over many
 *   rounds (1 MiB measured faster than 256 and 512 KiB for the batched
 *   shapes).  (Every extra round, and every second workgroup on a CU, exposes
 *   a workgroup's start-up and epilogue again and doubles the partials the
 *   merge reads; one workgroup per CU measured fastest for both variants.)
 * Partition p of (b, g) covers tokens [base + p*T_p, min(base + (p+1)*T_p,
 * seq_lens[b])), base = 0 without a window, else lo_0 (the first row's
 * window start) rounded down to a multiple of 16; it is empty when that
 * range is.  The grid of the main kernel is (Hkv, B, P), the partition
 * index slowest, so that the empty partitions of short sequences are
 * dispatched after every live one; a plan has at most 65535 partitions
 * (PDA_ERR_UNSUPPORTED otherwise).  When P == 1 the main kernel writes `out` directly and no
 * workspace is used; otherwise it writes fp32 partials that are merged with
 * the log-sum-exp rule, either
 *   PDA_MERGE_FUSED  by the last workgroup of each (b, g) to finish, found
 *                    with an atomic counter in the workspace (one launch;
 *                    that workgroup alone reads the unit's P x R x D fp32
 *                    partials), or
 *   PDA_MERGE_KERNEL by a separate merge kernel on the same stream (spread
 *                    over D/64 x Hq x B*q_len workgroups).
 * The plan picks PDA_MERGE_FUSED when 1 < P <= PDA_FUSED_MAX_PARTS,
 * B * Hkv <= PDA_FUSED_MAX_UNITS and P * R * D * 4 <= PDA_FUSED_MAX_BYTES
 * (the last workgroup then reads all of
 * them in one round of loads, and saving the second launch pays: measured
 * 1.6-2.8 us per call at 1K-2K tokens), PDA_MERGE_KERNEL otherwise (with
 * more partitions the fused tail takes more round trips than the merge
 * kernel's launch costs).
 * The workspace (P > 1) holds PDA_FUSED_MAX_UNITS int32 arrival counters
 * first (unit (b, g) uses entry b * Hkv + g), then partial outputs
 * [B][q_len][Hq][P][D] fp32, then (m, l) pairs [B][q_len][Hq][P][2] fp32,
 * each part aligned to 256 bytes.  The counters must be zero when a fused
 * call starts; every fused call leaves them zero again, and they sit at the
 * same place for every shape, so a workspace zeroed once
 * (paged_decode_attn_workspace_init, or any zero fill) before its first use
 * serves any sequence of calls, of any shapes and either merge, that it is
 * large enough for.  Calls that run concurrently need separate workspaces. */
#define PDA_TILE            16
#define PDA_TP_ALIGN        64
#define PDA_MFMA_MIN_GROUP  2
#define PDA_WG_MIN_BYTES    (64 * 1024)
#define PDA_WG_MANY_BYTES   (1024 * 1024)
#define PDA_WG_ONE_BYTES    (1024 * 1024)

#define PDA_MERGE_FUSED   0
#define PDA_MERGE_KERNEL  1
#define PDA_FUSED_MAX_PARTS  16
#define PDA_FUSED_MAX_BYTES  (32 * 1024)
#define PDA_FUSED_MAX_UNITS  16384

typedef struct pda_shape {
    int32_t num_seqs;            /* B >= 1 */
    int32_t num_q_heads;         /* Hq >= 1, multiple of num_kv_heads */
    int32_t num_kv_heads;        /* Hkv >= 1 */
    int32_t head_size;           /* D: 64, 128 or 256 */
    int32_t block_size;          /* bs >= 1 (any value, e.g. 16 or 784); bs * D <= INT32_MAX */
    int32_t num_blocks;          /* NB >= 1: blocks in each of k_cache, v_cache */
    int32_t max_blocks_per_seq;  /* MBS >= 1: row length of block_table */
    int32_t max_seq_len;         /* >= every seq_lens[b], <= MBS * bs; sizes the plan */
    int32_t dtype;               /* PDA_BF16 or PDA_FP16 */
    int32_t sliding_window;      /* W >= 0; 0: attend to the whole context (see above) */
    int32_t q_len;               /* query rows per sequence, 1..; 0 is read as 1 (see above) */
    int32_t kv_dtype;            /* PDA_KV_SAME or PDA_KV_FP8_E4M3 (see above) */
    float k_scale, v_scale;      /* fp8 KV: per-tensor scales, finite and > 0; else unused */
} pda_shape_t;

typedef struct pda_plan {
    int32_t num_partitions;        /* P >= 1 */
    int32_t tokens_per_partition;  /* T_p, a positive multiple of PDA_TP_ALIGN */
    int32_t variant;               /* PDA_VARIANT_VALU or PDA_VARIANT_MFMA */
    int32_t merge;                 /* PDA_MERGE_FUSED or PDA_MERGE_KERNEL (rule above) */
    int32_t cu_count;              /* the C the plan was made for */
    int64_t workspace_bytes;       /* 0 when P == 1 */
} pda_plan_t;

/* Validate a shape: PDA_OK, PDA_ERR_INVALID or PDA_ERR_UNSUPPORTED.  Pure. */
int pda_check_shape(const pda_shape_t* shape);

/* The plan above for an explicit compute-unit count.  Pure and host-only:
 * it needs no GPU.  Writes *plan and returns PDA_OK, or an error status. */
int pda_plan_for_cus(const pda_shape_t* shape, int32_t cu_count, pda_plan_t* plan);

/* The plan for the current HIP device (its compute-unit count is queried
 * once per device and cached).  Returns PDA_ERR_DEVICE if the query fails. */
int paged_decode_attn_plan(const pda_shape_t* shape, pda_plan_t* plan);

/* Workspace bytes paged_decode_attn needs on the current device (0 when the
 * plan has a single partition).  Returns a negative status on error. */
int64_t paged_decode_attn_workspace_size(const pda_shape_t* shape);

/* Workspace bytes a given plan needs (0 when plan->num_partitions == 1), or
 * a negative status for an invalid shape (as pda_check_shape) or a partition
 * count outside [1, 65535]. */
int64_t pda_workspace_bytes(const pda_shape_t* shape, const pda_plan_t* plan);

/* Zero `bytes` of a device workspace on `stream` (asynchronously): the state
 * a workspace must be in before its first fused call.  Call it once after
 * allocating a workspace.  It is a kernel launch (not a memset), so it may
 * also be captured into a HIP graph. */
int paged_decode_attn_workspace_init(void* workspace, int64_t bytes, void* stream);

/* Check a workspace's arrival counters (validation, not for the hot path):
 * waits for the work queued on `stream`, copies the counter block (the first
 * min(bytes, 4 * PDA_FUSED_MAX_UNITS) bytes) to the host and stores in
 * *nonzero the number of counters that are not zero.  Once the calls that
 * used the workspace have completed, every counter is zero; a non-zero count
 * means a fused call started on counters that were not (a workspace not
 * zeroed before its first use, or calls overlapping on one workspace), and
 * that call's merge may not have run.  PDA_ERR_INVALID for a null pointer or
 * a negative size, PDA_ERR_LAUNCH if the copy fails. */
int paged_decode_attn_workspace_check(const void* workspace, int64_t bytes, void* stream,
                                      int32_t* nonzero);

/* The decode step, under the device's own plan.
 *   q            [B][q_len][Hq][D]    16-bit, the query rows of each sequence
 *   k_cache      [NB][Hkv][bs][D]     16-bit or fp8 (kv_dtype), the paged K pool
 *   v_cache      [NB][Hkv][bs][D]     the paged V pool (same type and layout)
 *   block_table  [B][MBS]             int32 physical block ids, row-major
 *   seq_lens     [B]                  int32 context lengths
 *   scale        multiplies q.k before the softmax (usually 1/sqrt(D))
 *   out          [B][q_len][Hq][D]    16-bit, written in full
 *   workspace    device scratch of workspace_bytes (may be NULL if the plan
 *                needs none), zeroed once before its first use (see above)
 * Returns PDA_OK once the kernels are enqueued on `stream`. */
int paged_decode_attn(const pda_shape_t* shape,
                      const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* seq_lens,
                      float scale, void* out,
                      void* workspace, int64_t workspace_bytes,
                      void* stream);

/* The same step under a caller-chosen plan (a partition count and size that
 * cover max_seq_len, and a variant).  Tests use it to force P == 1 or a
 * variant; results differ from the planned call only by fp32 rounding order. */
int paged_decode_attn_with_plan(const pda_shape_t* shape, const pda_plan_t* plan,
                                const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* seq_lens,
                                float scale, void* out,
                                void* workspace, int64_t workspace_bytes,
                                void* stream);

/* Instrumented decode step for benchmarks: identical to
 * paged_decode_attn_with_plan (plan may be NULL for the device's own plan),
 * but the split-KV kernel is launched with hipExtLaunchKernel so that the
 * caller's events `start_event` / `stop_event` (hipEvent_t, created by the
 * caller, may be NULL) record that kernel's own start and end on `stream`.
 * The merge kernel, if any, follows on the same stream untimed. */
int paged_decode_attn_timed(const pda_shape_t* shape, const pda_plan_t* plan,
                            const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_table, const int32_t* seq_lens,
                            float scale, void* out,
                            void* workspace, int64_t workspace_bytes,
                            void* start_event, void* stop_event, void* stream);

/* Bookkeeping trace.  Runs the main kernel's own partitioning, tiling and
 * address generation (the same device functions) under `plan` -- for the
 * plan's variant, the rows its K loads (rows == 0) or its V loads (rows == 1)
 * read -- but instead of loading K/V it records, for every token t consumed:
 *   trace_slot [B][Hkv][max_seq_len]  physical slot  block_id * bs + (t % bs)
 *   trace_part [B][Hkv][max_seq_len]  the partition p that consumed t
 * and for every unit trace_range [B][Hkv][P][2] = (t0, t1) (t1 <= t0 when the
 * partition is empty).  PDA_ERR_UNSUPPORTED when num_blocks * bs exceeds
 * INT32_MAX (a slot id would not fit).  Entries for t >= seq_lens[b], and for t before a
 * sliding window, are left untouched.
 * Device pointers; the caller pre-fills them with a sentinel. */
int paged_decode_attn_trace(const pda_shape_t* shape, const pda_plan_t* plan, int32_t rows,
                            const int32_t* block_table, const int32_t* seq_lens,
                            int32_t* trace_slot, int32_t* trace_part,
                            int32_t* trace_range, void* stream);

/* HBM streaming-read probe (a measurement aid, not part of the decode):
 * reads the `bytes` (a positive multiple of 16) at device pointer `src`
 * once, with the decode kernels' non-temporal 16-byte loads, in a
 * grid-stride loop over `workgroups` workgroups of 256 threads, and XORs the
 * 32-bit words of the buffer into the device word `sink` (which the caller
 * zeroes first: the result is then the XOR of all words, independent of the
 * schedule).  Timing it over a buffer far larger than the 256 MB MALL gives
 * the achievable read bandwidth the decode's roofline fraction can be set
 * against.  Asynchronous on `stream`; PDA_ERR_INVALID for a null pointer, a
 * bad size or 0 / more than 2^20 workgroups. */
int pda_read_probe(const void* src, int64_t bytes, void* sink, int32_t workgroups, void* stream);

/* The decode step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Arguments, layouts, plan and results are those of
 * paged_decode_attn (the same kernels under the device's own plan, bit-
 * identical output); the workspace is not an argument: the library keeps one
 * static device array of PDA_NOALLOC_MAX_WORKSPACE bytes per GPU (held until
 * the process ends) and uses it as the workspace.  The call allocates
 * nothing.  Its first call on a device resolves the array's address and
 * zeroes its counter block with a fill kernel on `stream`; every completed
 * call leaves the counters zero again.
 *  - PDA_ERR_WORKSPACE when the plan's workspace exceeds
 *    PDA_NOALLOC_MAX_WORKSPACE (nothing is launched);
 *  - every call on one GPU shares that GPU's array: calls that overlap on
 *    one GPU (concurrent streams, or host threads) race and must not be
 *    issued; calls queued one after another on a stream are safe. */
#define PDA_NOALLOC_MAX_WORKSPACE (64 * 1024 * 1024)
int paged_decode_attn_noalloc(const pda_shape_t* shape,
                              const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              float scale, void* out, void* stream);

/* Human-readable text of a status code (static storage). */
const char* pda_status_string(int status);

/* Build identification: library version, target and compile flags. */
const char* pda_build_id(void);

#ifdef __cplusplus
}
#endif
#endif /* PDA_H */

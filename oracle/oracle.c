/*
 * CPU oracle for single-token paged-attention decode.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke entry
 * point and the CPU-baseline leg of the benchmark may load this library.  It
 * shares no code, header, table or constant with the GPU library: it never
 * sees the paged KV pool, only the contiguous, pre-paging K/V tensors.
 *
 * What it computes (page "vLLM's custom ROCm paged-attention kernel wins all
 * sixty cells", section 1 "What is being measured"): the reference is an fp32
 * attention over the pre-paging KV tensors of a pure-decode step, i.e. one
 * query token per sequence over its whole cached context.  For one output row
 * (sequence b, query head h) with context length L = seq_lens[b], group size
 * G = Hq / Hkv and KV head g = floor(h / G):
 *
 *   s[t]  = scale * sum_d q[b,h,d] * K_b[g,t,d]     t in [0, L)
 *   m     = max_t s[t]
 *   e[t]  = expf(s[t] - m)
 *   l     = sum_t e[t]
 *   o[d]  = (sum_t e[t] * V_b[g,t,d]) / l
 *
 * i.e. softmax(q K^T * scale) V written out as a plain two-pass softmax.  All
 * arithmetic is fp32 (the pages fix the reference's precision at fp32); sums
 * run in index order; the library is built with -ffp-contract=off so every
 * product and every sum is rounded once, as written.  L = 0 gives a zero row
 * (an empty softmax has no value; zeros is the defined, NaN-free choice).
 *
 * Layout of the inputs (all fp32, exact upcasts of the bf16/fp16 data):
 *   q      [B][Hq][D]
 *   k, v   concatenation over b of [Hkv][L_b][D]; kv_off[b] is the element
 *          offset of sequence b's block inside k and v.
 * Parallelism: optional OpenMP over output rows.  Each row is computed by one
 * thread in the order above, so the thread count never changes a result.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One output row over the token sub-range [t0, t1) of sequence b.
 * Writes o[D] (normalised), and the row's max score *m_out and
 * denominator *l_out (natural-exp domain).  Returns 0, or -1 on allocation
 * failure.  An empty range writes zeros, m = -inf, l = 0. */
static int row_range(int32_t Hq, int32_t Hkv, int32_t D,
                     const int32_t* seq_lens, const int64_t* kv_off,
                     const float* q, const float* k, const float* v, float scale,
                     int32_t b, int32_t h, int32_t t0, int32_t t1,
                     float* o, float* m_out, float* l_out)
{
    const int32_t G = Hq / Hkv;
    const int32_t g = h / G;
    const int32_t L = seq_lens[b];
    const float* qv = q + ((int64_t)b * Hq + h) * D;
    const float* Kb = k + kv_off[b] + (int64_t)g * L * D;
    const float* Vb = v + kv_off[b] + (int64_t)g * L * D;
    int32_t n = t1 - t0;
    int32_t t, d;

    for (d = 0; d < D; ++d) o[d] = 0.0f;
    *m_out = -INFINITY;
    *l_out = 0.0f;
    if (n <= 0) return 0;

    float* s = (float*)malloc(sizeof(float) * (size_t)n);
    if (!s) return -1;

    /* pass 1: scores and their max */
    float m = -INFINITY;
    for (t = 0; t < n; ++t) {
        const float* kt = Kb + (int64_t)(t0 + t) * D;
        float dot = 0.0f;
        for (d = 0; d < D; ++d) dot += qv[d] * kt[d];
        s[t] = scale * dot;
        if (s[t] > m) m = s[t];
    }
    /* pass 2: exponentials, their sum, and the weighted sum of V rows */
    float l = 0.0f;
    for (t = 0; t < n; ++t) {
        float e = expf(s[t] - m);
        const float* vt = Vb + (int64_t)(t0 + t) * D;
        l += e;
        for (d = 0; d < D; ++d) o[d] += e * vt[d];
    }
    for (d = 0; d < D; ++d) o[d] = o[d] / l;
    *m_out = m;
    *l_out = l;
    free(s);
    return 0;
}

/* Full-context output for a list of (b, h) rows.  out is [nrows][D].
 * Returns 0 on success, -1 on a bad argument or allocation failure. */
int oracle_decode_rows(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                       const int32_t* seq_lens, const int64_t* kv_off,
                       const float* q, const float* k, const float* v, float scale,
                       int32_t nrows, const int32_t* row_b, const int32_t* row_h,
                       float* out, int32_t nthreads)
{
    int32_t i;
    int err = 0;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0 || nrows < 0)
        return -1;
    for (i = 0; i < nrows; ++i)
        if (row_b[i] < 0 || row_b[i] >= B || row_h[i] < 0 || row_h[i] >= Hq) return -1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    #pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(|:err)
#else
    (void)nthreads;
#endif
    for (i = 0; i < nrows; ++i) {
        float m, l;
        int32_t b = row_b[i];
        err |= row_range(Hq, Hkv, D, seq_lens, kv_off, q, k, v, scale, b, row_h[i],
                         0, seq_lens[b], out + (int64_t)i * D, &m, &l);
    }
    return err ? -1 : 0;
}

/* Every row of the batch: out is [B][Hq][D]. */
int oracle_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                  const int32_t* seq_lens, const int64_t* kv_off,
                  const float* q, const float* k, const float* v, float scale,
                  float* out, int32_t nthreads)
{
    int32_t nrows = B * Hq, i;
    int rc;
    if (B <= 0 || Hq <= 0) return -1;
    int32_t* rb = (int32_t*)malloc(sizeof(int32_t) * (size_t)nrows);
    int32_t* rh = (int32_t*)malloc(sizeof(int32_t) * (size_t)nrows);
    if (!rb || !rh) { free(rb); free(rh); return -1; }
    for (i = 0; i < nrows; ++i) { rb[i] = i / Hq; rh[i] = i % Hq; }
    rc = oracle_decode_rows(B, Hq, Hkv, D, seq_lens, kv_off, q, k, v, scale,
                            nrows, rb, rh, out, nthreads);
    free(rb);
    free(rh);
    return rc;
}

/* The same two-pass softmax restricted to tokens [t0, t1) of one row: the
 * normalised partial output o[D], its max score m and denominator l.  Used by
 * the tests of the log-sum-exp merge algebra, never by the product. */
int oracle_partial(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                   const int32_t* seq_lens, const int64_t* kv_off,
                   const float* q, const float* k, const float* v, float scale,
                   int32_t b, int32_t h, int32_t t0, int32_t t1,
                   float* o, float* m, float* l)
{
    if (b < 0 || b >= B || h < 0 || h >= Hq || Hq % Hkv != 0) return -1;
    if (t0 < 0) t0 = 0;
    if (t1 > seq_lens[b]) t1 = seq_lens[b];
    return row_range(Hq, Hkv, D, seq_lens, kv_off, q, k, v, scale, b, h, t0, t1, o, m, l);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

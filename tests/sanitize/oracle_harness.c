/*
 * CPU harness for the oracle's C code (oracle/oracle.c), built with gcc
 * under AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py.  Test infrastructure for the oracle only: it
 * includes nothing of the GPU library.
 *
 * Every buffer is malloc'd at exactly the size the oracle's contract states
 * (q [B][Hq][D]; K and V the concatenation over b of [Hkv][L_b][D]; out
 * [B][Hq][D] or [nrows][D]; a partial o[D]), so a read or write outside it is
 * reported.  Shapes are random and small, with empty contexts, single
 * tokens and empty or reversed partial ranges among them; every call is
 * also checked against properties the definition fixes: a zero row for an
 * empty context, the V row itself for a single token, and outputs inside
 * the per-element range of the V rows (a convex combination).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_decode_rows(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, const int32_t* seq_lens,
                       const int64_t* kv_off, const float* q, const float* k, const float* v,
                       float scale, int32_t nrows, const int32_t* row_b, const int32_t* row_h,
                       float* out, int32_t nthreads);
int oracle_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, const int32_t* seq_lens,
                  const int64_t* kv_off, const float* q, const float* k, const float* v,
                  float scale, float* out, int32_t nthreads);
int oracle_partial(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, const int32_t* seq_lens,
                   const int64_t* kv_off, const float* q, const float* k, const float* v,
                   float scale, int32_t b, int32_t h, int32_t t0, int32_t t1, float* o,
                   float* m, float* l);

static uint64_t rng_state = 0x243F6A8885A308D3ull;
static uint64_t next_u64(void) { /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int rnd(int lo, int hi) { return lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)); }
static float rnd_f(void) { return (float)((double)(next_u64() >> 11) / 9007199254740992.0 * 4.0 - 2.0); }

static int failures = 0;
#define EXPECT(c)                                                             \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "FAILED %s at line %d (iteration %d)\n", #c, __LINE__, it); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

/* min and max over t < L of V_b[g][t][d] */
static void v_range(const float* v, int64_t off, int32_t L, int32_t g, int32_t D, int32_t d,
                    float* lo, float* hi) {
    *lo = INFINITY;
    *hi = -INFINITY;
    for (int32_t t = 0; t < L; ++t) {
        const float x = v[off + ((int64_t)g * L + t) * D + d];
        if (x < *lo) *lo = x;
        if (x > *hi) *hi = x;
    }
}

int main(int argc, char** argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 300;
    int it;
    for (it = 0; it < iters; ++it) {
        const int32_t B = rnd(1, 4), Hkv = rnd(1, 3), G = rnd(1, 4), Hq = Hkv * G;
        const int32_t D = rnd(0, 2) == 0 ? rnd(1, 9) : (int32_t[]){64, 128, 256}[rnd(0, 2)];
        int32_t* lens = malloc(sizeof(int32_t) * B);
        int64_t* off = malloc(sizeof(int64_t) * B);
        int64_t total = 0;
        for (int32_t b = 0; b < B; ++b) {
            lens[b] = rnd(0, 3) == 0 ? rnd(0, 1) : rnd(0, 90);
            off[b] = total;
            total += (int64_t)Hkv * lens[b] * D;
        }
        const int64_t nq = (int64_t)B * Hq * D;
        float* q = malloc(sizeof(float) * nq);
        float* k = malloc(sizeof(float) * (total > 0 ? total : 1));
        float* v = malloc(sizeof(float) * (total > 0 ? total : 1));
#ifdef ORACLE_HARNESS_PLANT_SHORT_OUT
        /* a planted mistake, for the test that the instrument sees it: the
           output one element short of [B][Hq][D] */
        float* out = malloc(sizeof(float) * (nq - 1));
#else
        float* out = malloc(sizeof(float) * nq);
#endif
        for (int64_t i = 0; i < nq; ++i) q[i] = rnd_f();
        for (int64_t i = 0; i < total; ++i) { k[i] = rnd_f(); v[i] = rnd_f(); }
        const float scale = rnd(0, 4) == 0 ? 0.f : 1.f / sqrtf((float)D);

        EXPECT(oracle_decode(B, Hq, Hkv, D, lens, off, q, k, v, scale, out, rnd(1, 3)) == 0);
        for (int32_t b = 0; b < B; ++b)
            for (int32_t h = 0; h < Hq; ++h) {
                const int32_t g = h / G;
                const float* o = out + ((int64_t)b * Hq + h) * D;
                for (int32_t d = 0; d < D; ++d) {
                    EXPECT(isfinite(o[d]));
                    if (lens[b] == 0) {
                        EXPECT(o[d] == 0.f);
                    } else if (lens[b] == 1) {
                        EXPECT(o[d] == v[off[b] + (int64_t)g * D + d]);
                    } else {
                        float lo, hi;
                        v_range(v, off[b], lens[b], g, D, d, &lo, &hi);
                        const float eps = 1e-5f * (fabsf(lo) + fabsf(hi) + 1.f);
                        EXPECT(o[d] >= lo - eps && o[d] <= hi + eps);
                    }
                }
            }

        /* a subset of rows, in a shuffled order, must equal the full call */
        const int32_t nrows = rnd(0, B * Hq);
        int32_t* rb = malloc(sizeof(int32_t) * (nrows > 0 ? nrows : 1));
        int32_t* rh = malloc(sizeof(int32_t) * (nrows > 0 ? nrows : 1));
        float* ro = malloc(sizeof(float) * (nrows > 0 ? nrows : 1) * D);
        for (int32_t i = 0; i < nrows; ++i) { rb[i] = rnd(0, B - 1); rh[i] = rnd(0, Hq - 1); }
        EXPECT(oracle_decode_rows(B, Hq, Hkv, D, lens, off, q, k, v, scale, nrows, rb, rh, ro,
                                  rnd(1, 3)) == 0);
        for (int32_t i = 0; i < nrows; ++i)
            EXPECT(memcmp(ro + (int64_t)i * D, out + ((int64_t)rb[i] * Hq + rh[i]) * D,
                          sizeof(float) * D) == 0);
        /* out-of-range rows are refused, nothing is written */
        if (nrows > 0) {
            const int32_t keep = rb[0];
            rb[0] = B;
            EXPECT(oracle_decode_rows(B, Hq, Hkv, D, lens, off, q, k, v, scale, nrows, rb, rh, ro,
                                      1) == -1);
            rb[0] = keep;
        }

        /* partial ranges, including empty, reversed and clipped ones */
        float* po = malloc(sizeof(float) * D);
        for (int rep = 0; rep < 4; ++rep) {
            const int32_t b = rnd(0, B - 1), h = rnd(0, Hq - 1);
            const int32_t t0 = rnd(-3, lens[b] + 3), t1 = rnd(-3, lens[b] + 3);
            float m, l;
            EXPECT(oracle_partial(B, Hq, Hkv, D, lens, off, q, k, v, scale, b, h, t0, t1, po, &m,
                                  &l) == 0);
            const int32_t a = t0 < 0 ? 0 : t0, e = t1 > lens[b] ? lens[b] : t1;
            if (e <= a) {
                EXPECT(l == 0.f && isinf(m) && m < 0);
                for (int32_t d = 0; d < D; ++d) EXPECT(po[d] == 0.f);
            } else {
                EXPECT(l >= 1.f && isfinite(m));
                if (a == 0 && e == lens[b])
                    EXPECT(memcmp(po, out + ((int64_t)b * Hq + h) * D, sizeof(float) * D) == 0);
            }
        }
        EXPECT(oracle_partial(B, Hq, Hkv, D, lens, off, q, k, v, scale, B, 0, 0, 1, po, &(float){0},
                              &(float){0}) == -1);
        /* bad shapes are refused before anything is read */
        EXPECT(oracle_decode(0, Hq, Hkv, D, lens, off, q, k, v, scale, out, 1) == -1);
        EXPECT(oracle_decode_rows(B, Hq, Hq + 1, D, lens, off, q, k, v, scale, 0, rb, rh, ro,
                                  1) == -1);  /* Hq not a multiple of Hkv */

        free(po); free(rb); free(rh); free(ro);
        free(q); free(k); free(v); free(out); free(lens); free(off);
    }
    printf("iterations %d failures %d\n", iters, failures);
    return failures == 0 ? 0 : 1;
}

/*
 * cpu_fused.c -- a multi-threaded, vectorised CPU decode GEMV whose epilogue
 * is applied straight out of each accumulator tile: the CPU comparison point
 * for the HIP library (the benchmark's stronger CPU baseline).  It is never a
 * fallback: the HIP binding does not load or call it.
 *
 * What it follows: "ggml-cpu: fuse element-wise epilogues (ADD, MUL, SILU)
 * into ggml_compute_forward_mul_mat", "What": each thread computes a tile of
 * rows into an accumulator tile and applies the element-wise op to that tile
 * before writing dst, instead of a separate pass (and a thread barrier) over
 * the whole output; "Correctness": the tails use a vectorised exp on full
 * vector groups and the scalar libm exp on the remainder, so a fused SILU or
 * SIGMOID can differ from the unfused pass by a couple of ulp where tile
 * boundaries move the vector/remainder split, while ADD, MUL and NONE are
 * bit-identical.  Both paths (fused, and unfused: every accumulator first,
 * then the epilogue over the whole output after the threads join) are here.
 *
 * Layout and formats are those of include/gemv_fused.h.  Products are summed
 * in f32 over 8 vector lanes (row order fixed, so results do not depend on
 * the thread count), then reduced in a fixed order.
 *
 * The vector exp is this file's own: Cody and Waite's range reduction
 * x = n ln2 + r with ln2 split into a short head (exact n * head) and a tail,
 * |r| <= ln2 / 2, then the degree-7 Taylor polynomial of e^r (truncation
 * below 2^-26 relative) and a scale by 2^n built in the exponent field.
 */
#include <immintrin.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#include "gemv_fused.h"

typedef float f8 __attribute__((vector_size(32)));
typedef int32_t i8v __attribute__((vector_size(32)));
typedef uint32_t u8v __attribute__((vector_size(32)));

#define VEC 8
#define TILE_ROWS 16

static inline int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

static inline float half_to_float(uint16_t h) { return _cvtsh_ss(h); }

/* ------------------------------------------------------------ exp and tails */

static inline f8 splat(float v) { return (f8){v, v, v, v, v, v, v, v}; }

static inline f8 select8(i8v mask, f8 a, f8 b) { return (f8)(((i8v)a & mask) | ((i8v)b & ~mask)); }

/* e^x for x <= 0 (the epilogues only need e^-|a|); inputs below -87 clamp
 * to e^-87 whose tail is immaterial next to 1 in 1 + t. */
static inline f8 vexp_nonpos(f8 x)
{
    const f8 lo = splat(-87.0f);
    x = select8(x < lo, lo, x);
    const f8 log2e = splat(1.4426950408889634f);
    const f8 ln2_hi = splat(0.693145751953125f); /* 12 significant bits: n * ln2_hi exact */
    const f8 ln2_lo = splat(1.4286068203094172e-06f);
    f8 t = x * log2e;
    /* round to nearest integer */
    f8 n = (f8)_mm256_round_ps((__m256)t, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
    f8 r = (x - n * ln2_hi) - n * ln2_lo;
    f8 p = splat(1.0f / 5040.0f);
    p = p * r + splat(1.0f / 720.0f);
    p = p * r + splat(1.0f / 120.0f);
    p = p * r + splat(1.0f / 24.0f);
    p = p * r + splat(1.0f / 6.0f);
    p = p * r + splat(0.5f);
    p = p * r + splat(1.0f);
    p = p * r + splat(1.0f);
    i8v ni = __builtin_convertvector(n, i8v);
    f8 scale = (f8)((ni + 127) << 23);
    return p * scale;
}

static inline float sigmoid_s(float a)
{
    float t = expf(-fabsf(a));
    return (a >= 0.0f ? 1.0f : t) / (1.0f + t);
}

static inline float silu_s(float a)
{
    float t = expf(-fabsf(a));
    return (a >= 0.0f ? a : a * t) / (1.0f + t);
}

static inline float epi_s(int act, float a, float v)
{
    switch (act) {
    case GEMV_ACT_SIGMOID:
        return sigmoid_s(a);
    case GEMV_ACT_SILU:
        return silu_s(a);
    case GEMV_ACT_SILU_MUL:
        return silu_s(a) * v;
    case GEMV_ACT_MUL:
        return a * v;
    case GEMV_ACT_ADD:
        return a + v;
    default:
        return a;
    }
}

static inline f8 load8(const float *p)
{
    f8 v;
    memcpy(&v, p, sizeof v);
    return v;
}

static inline void store8(float *p, f8 v) { memcpy(p, &v, sizeof v); }

/* y[i] = epilogue(acc[i]) for i < n: full groups of 8 with the vector exp,
 * the remainder with libm; acc may be y. */
static void epilogue_span(int act, int64_t n, const float *acc, const float *m, const float *r, float *y)
{
    int64_t i = 0;
    for (; i + VEC <= n; i += VEC) {
        f8 a = load8(acc + i), out;
        if (act == GEMV_ACT_SIGMOID || act == GEMV_ACT_SILU || act == GEMV_ACT_SILU_MUL) {
            const f8 zero = splat(0.0f);
            f8 absa = select8(a < zero, -a, a);
            f8 t = vexp_nonpos(-absa);
            i8v pos = a >= zero;
            f8 num = act == GEMV_ACT_SIGMOID ? select8(pos, splat(1.0f), t) : select8(pos, a, a * t);
            out = num / (splat(1.0f) + t);
            if (act == GEMV_ACT_SILU_MUL)
                out = out * load8(m + i);
        } else if (act == GEMV_ACT_MUL) {
            out = a * load8(m + i);
        } else if (act == GEMV_ACT_ADD) {
            out = a + load8(r + i);
        } else {
            out = a;
        }
        store8(y + i, out);
    }
    for (; i < n; ++i) {
        float v = (act == GEMV_ACT_SILU_MUL || act == GEMV_ACT_MUL) ? m[i] : (act == GEMV_ACT_ADD ? r[i] : 0.0f);
        y[i] = epi_s(act, acc[i], v);
    }
}

/* ------------------------------------------------------------ rows */

typedef struct {
    int wfmt;
    int64_t N, K;
    const uint8_t *W;
    const float *x;
    int act;
    const float *m, *r;
    float *dst;
    float *acc; /* where the unfused product goes (dst itself when no scratch is given) */
    int fused;
    int64_t lo, hi; /* rows of this thread */
} Job;

/* Weights k .. k+7 of row n as floats (K is a multiple of 8 for the block
 * formats' 32-blocks; float formats take a scalar tail). */
static inline f8 weights8(const Job *j, int64_t n, int64_t k)
{
    const int64_t K = j->K;
    f8 w;
    switch (j->wfmt) {
    case GEMV_W_F32:
        memcpy(&w, (const float *)j->W + n * K + k, sizeof w);
        return w;
    case GEMV_W_F16: {
        __m128i h;
        memcpy(&h, (const uint16_t *)j->W + n * K + k, sizeof h);
        return (f8)_mm256_cvtph_ps(h);
    }
    case GEMV_W_BF16: {
        const uint16_t *p = (const uint16_t *)j->W + n * K + k;
        u8v b = {p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]};
        return (f8)(b << 16);
    }
    case GEMV_W_Q8B32: {
        const int8_t *c = (const int8_t *)j->W + n * K + k;
        const uint8_t *sc = j->W + align256(j->N * K) + (n * (K / 32) + k / 32) * 2;
        uint16_t sh;
        memcpy(&sh, sc, 2);
        i8v ci = {c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7]};
        return __builtin_convertvector(ci, f8) * splat(half_to_float(sh));
    }
    default: { /* GEMV_W_Q4B32 */
        const uint8_t *c = j->W + n * (K / 2) + k / 2;
        const uint8_t *sc = j->W + align256(j->N * K / 2) + (n * (K / 32) + k / 32) * 2;
        uint16_t sh;
        memcpy(&sh, sc, 2);
        i8v ci = {c[0] & 15, c[0] >> 4, c[1] & 15, c[1] >> 4, c[2] & 15, c[2] >> 4, c[3] & 15, c[3] >> 4};
        return __builtin_convertvector(ci - 8, f8) * splat(half_to_float(sh));
    }
    }
}

static float weight1(const Job *j, int64_t n, int64_t k)
{
    if (j->wfmt == GEMV_W_F32)
        return ((const float *)j->W)[n * j->K + k];
    if (j->wfmt == GEMV_W_F16)
        return half_to_float(((const uint16_t *)j->W)[n * j->K + k]);
    uint32_t b = (uint32_t)((const uint16_t *)j->W)[n * j->K + k] << 16; /* bf16; block formats have K % 32 == 0 */
    float f;
    memcpy(&f, &b, 4);
    return f;
}

static float row_dot(const Job *j, int64_t n)
{
    f8 acc = splat(0.0f);
    int64_t k = 0;
    for (; k + VEC <= j->K; k += VEC)
        acc += weights8(j, n, k) * load8(j->x + k);
    float s = ((acc[0] + acc[4]) + (acc[2] + acc[6])) + ((acc[1] + acc[5]) + (acc[3] + acc[7]));
    for (; k < j->K; ++k)
        s += weight1(j, n, k) * j->x[k];
    return s;
}

static void *run_rows(void *arg)
{
    const Job *j = (const Job *)arg;
    float tile[TILE_ROWS];
    for (int64_t r0 = j->lo; r0 < j->hi; r0 += TILE_ROWS) {
        const int64_t nt = j->hi - r0 < TILE_ROWS ? j->hi - r0 : TILE_ROWS;
        for (int64_t t = 0; t < nt; ++t)
            tile[t] = row_dot(j, r0 + t);
        if (j->fused)
            epilogue_span(j->act, nt, tile, j->m ? j->m + r0 : NULL, j->r ? j->r + r0 : NULL, j->dst + r0);
        else
            memcpy(j->acc + r0, tile, (size_t)nt * sizeof(float));
    }
    return NULL;
}

static void *run_epilogue(void *arg)
{
    const Job *j = (const Job *)arg;
    epilogue_span(j->act, j->hi - j->lo, j->acc + j->lo, j->m ? j->m + j->lo : NULL, j->r ? j->r + j->lo : NULL,
                  j->dst + j->lo);
    return NULL;
}

#define MAX_THREADS 256

static int overlaps(const float *a, const float *b, int64_t n) { return a && b && a < b + n && b < a + n; }

/* dst = epilogue(W x) on the host, with nthreads threads over contiguous row
 * ranges.  fused != 0: the epilogue is applied to each 16-row accumulator
 * tile; fused == 0: every product is first written to acc (N floats of
 * caller scratch), the threads join, and the epilogue runs as its own pass
 * from acc and the operand into dst (split over the same threads), as a
 * separate element-wise op would.  Without acc the unfused products go to
 * dst, which then must not overlap the operand.  All pointers are host
 * pointers; dst may be the identical array as m or r.  Returns 0, or -1 for
 * bad arguments. */
int cpu_fused_gemv(int wfmt, int64_t N, int64_t K, const void *W, const float *x, int act, const float *m,
                   const float *r, float *dst, int nthreads, int fused, float *acc)
{
    if (wfmt < GEMV_W_F32 || wfmt > GEMV_W_Q4B32 || act < GEMV_ACT_NONE || act > GEMV_ACT_ADD || N < 1 || K < 1 ||
        !W || !x || !dst || nthreads < 1)
        return -1;
    if ((wfmt == GEMV_W_Q8B32 || wfmt == GEMV_W_Q4B32) && K % 32)
        return -1;
    if (((act == GEMV_ACT_SILU_MUL || act == GEMV_ACT_MUL) && !m) || (act == GEMV_ACT_ADD && !r))
        return -1;
    const float *op = act == GEMV_ACT_ADD ? r : ((act == GEMV_ACT_SILU_MUL || act == GEMV_ACT_MUL) ? m : NULL);
    if (!fused && act != GEMV_ACT_NONE) {
        if (!acc && overlaps(dst, op, N))
            return -1;
        if (acc && (overlaps(acc, dst, N) || overlaps(acc, op, N)))
            return -1;
    }
    float *prod = (!fused && act != GEMV_ACT_NONE && acc) ? acc : dst;
    if (nthreads > MAX_THREADS)
        nthreads = MAX_THREADS;
    if (nthreads > N)
        nthreads = (int)N;
    Job jobs[MAX_THREADS];
    pthread_t th[MAX_THREADS];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (Job){wfmt, N, K, (const uint8_t *)W, x, act, m, r, dst, prod, fused, N * t / nthreads,
                        N * (t + 1) / nthreads};
    }
    for (int t = 1; t < nthreads; ++t)
        pthread_create(&th[t], NULL, run_rows, &jobs[t]);
    run_rows(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        pthread_join(th[t], NULL);
    if (!fused && act != GEMV_ACT_NONE) {
        /* the element-wise pass splits the output into its own spans of
         * whole vector groups, not along the row ranges of the product */
        const int64_t span = (N + (int64_t)nthreads * VEC - 1) / ((int64_t)nthreads * VEC) * VEC;
        for (int t = 0; t < nthreads; ++t) {
            jobs[t].lo = span * t < N ? span * t : N;
            jobs[t].hi = span * (t + 1) < N ? span * (t + 1) : N;
        }
        for (int t = 1; t < nthreads; ++t)
            pthread_create(&th[t], NULL, run_epilogue, &jobs[t]);
        run_epilogue(&jobs[0]);
        for (int t = 1; t < nthreads; ++t)
            pthread_join(th[t], NULL);
    }
    return 0;
}

/* The vector exp for n values of x <= 0 (n a multiple of 8), for its tests. */
void cpu_vexp_nonpos(int64_t n, const float *x, float *y)
{
    for (int64_t i = 0; i + VEC <= n; i += VEC)
        store8(y + i, vexp_nonpos(load8(x + i)));
}

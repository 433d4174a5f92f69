/*
 * Memory-safety run of the CPU comparison GEMV (cpu/cpu_fused.c), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_host_sanitize.py.  Every buffer is a heap block of exactly the
 * documented size, so a read or write past a row, a tile or a vector group
 * at a ragged edge is reported.  Random shapes (any K for the float formats,
 * K % 32 == 0 for the block formats), every epilogue, fused and unfused, 1..5
 * threads, dst in place over the operand or separate.  As a sanity check of
 * the indexing (parity with the oracle is tested elsewhere) every output is
 * compared with a double-precision dot product and epilogue computed here;
 * an unfused in-place call without a product buffer must be refused.  Exits
 * 1 on a mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gemv_fused.h"

int cpu_fused_gemv(int wfmt, int64_t N, int64_t K, const void *W, const float *x, int act, const float *m,
                   const float *r, float *dst, int nthreads, int fused, float *acc);

static uint64_t state = 0xC0FFEEull;
static uint64_t next(void)
{
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int64_t range(int64_t lo, int64_t hi) { return lo + (int64_t)(next() % (uint64_t)(hi - lo + 1)); }
static double unif(void) { return (double)(next() >> 11) / 9007199254740992.0 * 2.0 - 1.0; }

/* binary16 -> double, by the definition of the format */
static double half_value(uint16_t h)
{
    const int e = (h >> 10) & 31, f = h & 1023;
    const double s = (h & 0x8000) ? -1.0 : 1.0;
    if (e == 0)
        return s * ldexp(f, -24);
    return s * ldexp(1024 + f, e - 25);
}
/* a normal binary16 value in [2^-10, 2^-5) with a random mantissa */
static uint16_t random_scale(void) { return (uint16_t)((range(5, 9) << 10) | range(0, 1023)); }

static int64_t a256(int64_t v) { return (v + 255) / 256 * 256; }

static int64_t wbytes(int fmt, int64_t N, int64_t K)
{
    switch (fmt) {
    case GEMV_W_F32: return N * K * 4;
    case GEMV_W_F16:
    case GEMV_W_BF16: return N * K * 2;
    case GEMV_W_Q8B32: return a256(N * K) + N * (K / 32) * 2;
    default: return a256(N * K / 2) + N * (K / 32) * 2;
    }
}

static void fill_weights(int fmt, int64_t N, int64_t K, uint8_t *W)
{
    const int64_t nb = wbytes(fmt, N, K);
    for (int64_t i = 0; i < nb; ++i)
        W[i] = (uint8_t)next();
    if (fmt == GEMV_W_F32) {
        for (int64_t i = 0; i < N * K; ++i) {
            float v = (float)unif();
            memcpy(W + 4 * i, &v, 4);
        }
    } else if (fmt == GEMV_W_F16) {
        for (int64_t i = 0; i < N * K; ++i) {
            uint16_t h = random_scale() ^ (uint16_t)(range(0, 1) << 15);
            memcpy(W + 2 * i, &h, 2);
        }
    } else if (fmt == GEMV_W_BF16) {
        for (int64_t i = 0; i < N * K; ++i) {
            float v = (float)unif();
            uint32_t b;
            memcpy(&b, &v, 4);
            uint16_t h = (uint16_t)(b >> 16);
            memcpy(W + 2 * i, &h, 2);
        }
    } else {
        const int64_t soff = fmt == GEMV_W_Q8B32 ? a256(N * K) : a256(N * K / 2);
        for (int64_t i = 0; i < N * (K / 32); ++i) {
            uint16_t h = random_scale();
            memcpy(W + soff + 2 * i, &h, 2);
        }
    }
}

static double weight(int fmt, int64_t N, int64_t K, const uint8_t *W, int64_t n, int64_t k)
{
    switch (fmt) {
    case GEMV_W_F32: {
        float v;
        memcpy(&v, W + 4 * (n * K + k), 4);
        return v;
    }
    case GEMV_W_F16: {
        uint16_t h;
        memcpy(&h, W + 2 * (n * K + k), 2);
        return half_value(h);
    }
    case GEMV_W_BF16: {
        uint16_t h;
        memcpy(&h, W + 2 * (n * K + k), 2);
        uint32_t b = (uint32_t)h << 16;
        float v;
        memcpy(&v, &b, 4);
        return v;
    }
    case GEMV_W_Q8B32: {
        uint16_t s;
        memcpy(&s, W + a256(N * K) + 2 * (n * (K / 32) + k / 32), 2);
        return (double)(int8_t)W[n * K + k] * half_value(s);
    }
    default: {
        uint16_t s;
        memcpy(&s, W + a256(N * K / 2) + 2 * (n * (K / 32) + k / 32), 2);
        const uint8_t b = W[(n * K + k) / 2];
        const int c = (k & 1) ? b >> 4 : b & 15;
        return (double)(c - 8) * half_value(s);
    }
    }
}

static double epi(int act, double a, double v)
{
    const double sg = 1.0 / (1.0 + exp(-a));
    switch (act) {
    case GEMV_ACT_SIGMOID: return sg;
    case GEMV_ACT_SILU: return a * sg;
    case GEMV_ACT_SILU_MUL: return a * sg * v;
    case GEMV_ACT_MUL: return a * v;
    case GEMV_ACT_ADD: return a + v;
    default: return a;
    }
}

static void *exact(size_t bytes) { return malloc(bytes ? bytes : 1); }

int main(int argc, char **argv)
{
    const int iters = argc > 1 ? atoi(argv[1]) : 300;
    int bad = 0;
    for (int it = 0; it < iters && bad < 10; ++it) {
        const int fmt = (int)range(GEMV_W_F32, GEMV_W_Q4B32);
        const int block = fmt == GEMV_W_Q8B32 || fmt == GEMV_W_Q4B32;
        const int64_t N = range(1, 70);
        const int64_t K = block ? 32 * range(1, 12) : range(1, 300);
        const int act = (int)range(GEMV_ACT_NONE, GEMV_ACT_ADD);
        const int threads = (int)range(1, 5), fused = (int)range(0, 1);
        const int in_place = (act == GEMV_ACT_ADD || act == GEMV_ACT_MUL || act == GEMV_ACT_SILU_MUL) && range(0, 1);

        uint8_t *W = exact((size_t)wbytes(fmt, N, K));
        float *x = exact(4 * (size_t)K), *op = exact(4 * (size_t)N), *keep = exact(4 * (size_t)N);
        float *dst = in_place ? op : exact(4 * (size_t)N);
        fill_weights(fmt, N, K, W);
        for (int64_t k = 0; k < K; ++k)
            x[k] = (float)unif();
        for (int64_t n = 0; n < N; ++n)
            keep[n] = op[n] = (float)unif();
        const int uses_m = act == GEMV_ACT_SILU_MUL || act == GEMV_ACT_MUL;
        const float *m = uses_m ? op : NULL, *r = act == GEMV_ACT_ADD ? op : NULL;

        /* unfused with an operand: a separate product buffer, or none (then
         * an in-place call must be refused and leave dst alone) */
        float *acc = !fused && act != GEMV_ACT_NONE && range(0, 3) ? exact(4 * (size_t)N) : NULL;
        const int rc = cpu_fused_gemv(fmt, N, K, W, x, act, m, r, dst, threads, fused, acc);
        const int refuse = !fused && act != GEMV_ACT_NONE && !acc && in_place;
        if (rc != (refuse ? -1 : 0)) {
            fprintf(stderr, "iteration %d: status %d, expected %d\n", it, rc, refuse ? -1 : 0);
            ++bad;
        }
        free(acc);
        if (refuse) {
            for (int64_t n = 0; n < N; ++n)
                if (dst[n] != keep[n]) {
                    fprintf(stderr, "iteration %d: a refused call wrote dst\n", it);
                    ++bad;
                    break;
                }
            free(W);
            free(x);
            free(op);
            free(keep);
            continue;
        }
        for (int64_t n = 0; n < N; ++n) {
            double a = 0.0, amag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = weight(fmt, N, K, W, n, k) * x[k];
                a += p;
                amag += fabs(p);
            }
            const double v = keep[n], y = epi(act, a, v);
            const double tol = 1e-5 * (1.0 + fabs(y)) + 1e-5 * amag * (1.0 + fabs(v));
            if (!(fabs((double)dst[n] - y) <= tol)) {
                fprintf(stderr, "iteration %d: fmt %d N %lld K %lld act %d threads %d fused %d row %lld: %.9g vs %.9g\n",
                        it, fmt, (long long)N, (long long)K, act, threads, fused, (long long)n, dst[n], y);
                ++bad;
                break;
            }
        }
        free(W);
        free(x);
        free(op);
        free(keep);
        if (!in_place)
            free(dst);
    }
    if (bad)
        return 1;
    printf("ok %d iterations\n", iters);
    return 0;
}

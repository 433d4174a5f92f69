/*
 * Memory-safety run of the oracle's C code (oracle/gemv_oracle.c), built
 * with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_host_sanitize.py.  Random formats and shapes over heap buffers
 * of exactly the sizes the oracle documents (W of oracle_weight_bytes, x of
 * K floats, outputs of N doubles, scratch of K doubles), every epilogue, the
 * gated-pair epilogue and the signed transform; sub-ranges of rows too.
 * Checks only that every call succeeds and every output is finite: the
 * oracle's values are pinned by tests/test_oracle.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int64_t oracle_weight_bytes(int fmt, int64_t N, int64_t K);
int oracle_gemv_rows(int fmt, int64_t N, int64_t K, const void *W, const float *x, int64_t row_begin,
                     int64_t row_end, double *acc, double *absacc, double *rowbuf);
int oracle_epilogue(int act, int64_t n, const double *acc, const float *m, const float *r, double *y);
int oracle_glu_epilogue(int act, int64_t n, const double *g, const double *u, double *y);
int oracle_fwht_signed(int64_t n, int64_t K, int64_t ns, const float *x, const float *s, double *y, double *d);

static uint64_t state = 0x0AC1Eull;
static uint64_t next(void)
{
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int64_t range(int64_t lo, int64_t hi) { return lo + (int64_t)(next() % (uint64_t)(hi - lo + 1)); }
static float unif(void) { return (float)((double)(next() >> 11) / 9007199254740992.0 * 2.0 - 1.0); }

static int finite_all(const double *v, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(v[i]))
            return 0;
    return 1;
}

int main(int argc, char **argv)
{
    const int iters = argc > 1 ? atoi(argv[1]) : 300;
    int bad = 0;
    for (int it = 0; it < iters && !bad; ++it) {
        const int fmt = (int)range(0, 4);
        const int block = fmt >= 3;
        const int64_t N = range(1, 40), K = block ? 32 * range(1, 8) : range(1, 200);
        const int64_t nb = oracle_weight_bytes(fmt, N, K);
        if (nb <= 0) {
            fprintf(stderr, "iteration %d: weight bytes %lld\n", it, (long long)nb);
            return 1;
        }
        uint8_t *W = malloc((size_t)nb);
        for (int64_t i = 0; i < nb; ++i)
            W[i] = (uint8_t)next();
        if (fmt == 1 || fmt == 3 || fmt == 4) {
            /* keep f16 weights and scales finite: clear the top exponent bit */
            const int64_t off = fmt == 1 ? 0 : (fmt == 3 ? (N * K + 255) / 256 * 256 : (N * K / 2 + 255) / 256 * 256);
            for (int64_t i = off + 1; i < nb; i += 2)
                W[i] &= 0xBF;
        } else if (fmt == 0) {
            for (int64_t i = 0; i < N * K; ++i) {
                float v = unif();
                ((float *)W)[i] = v;
            }
        } else {
            for (int64_t i = 1; i < nb; i += 2)
                W[i] &= 0xBF; /* bf16 high byte: exponent below 2^64 */
        }
        float *x = malloc(4 * (size_t)K), *m = malloc(4 * (size_t)N), *r = malloc(4 * (size_t)N);
        for (int64_t k = 0; k < K; ++k)
            x[k] = unif();
        for (int64_t n = 0; n < N; ++n) {
            m[n] = unif();
            r[n] = unif();
        }
        const int64_t lo = range(0, N - 1), hi = range(lo, N);
        double *acc = malloc(8 * (size_t)N), *mag = malloc(8 * (size_t)N), *row = malloc(8 * (size_t)K);
        double *y = malloc(8 * (size_t)N), *g = malloc(8 * (size_t)N);
        if (oracle_gemv_rows(fmt, N, K, W, x, 0, N, acc, mag, row) != 0 || !finite_all(acc, N) || !finite_all(mag, N))
            bad = 1;
        if (!bad && oracle_gemv_rows(fmt, N, K, W, x, lo, hi, g, mag, row) != 0)
            bad = 1;
        for (int act = 0; act <= 5 && !bad; ++act)
            if (oracle_epilogue(act, N, acc, m, r, y) != 0 || !finite_all(y, N))
                bad = 1;
        if (!bad && (oracle_glu_epilogue(2, N, acc, acc, y) != 0 || oracle_glu_epilogue(1, N, acc, acc, y) != 0))
            bad = 1;
        if (!bad) {
            const int64_t n = (int64_t)1 << range(0, 7);
            const int64_t KK = n * range(1, 4), ns = range(0, 1) ? KK : n;
            float *xs = malloc(4 * (size_t)KK), *s = malloc(4 * (size_t)ns);
            double *fy = malloc(8 * (size_t)KK), *fd = malloc(8 * (size_t)KK);
            for (int64_t k = 0; k < KK; ++k)
                xs[k] = unif();
            for (int64_t k = 0; k < ns; ++k)
                s[k] = range(0, 1) ? 1.0f : -1.0f;
            if (oracle_fwht_signed(n, KK, ns, xs, s, fy, fd) != 0 || !finite_all(fy, KK))
                bad = 1;
            free(xs);
            free(s);
            free(fy);
            free(fd);
        }
        if (bad)
            fprintf(stderr, "iteration %d: fmt %d N %lld K %lld failed\n", it, fmt, (long long)N, (long long)K);
        free(W);
        free(x);
        free(m);
        free(r);
        free(acc);
        free(mag);
        free(row);
        free(y);
        free(g);
    }
    if (bad)
        return 1;
    printf("ok %d iterations\n", iters);
    return 0;
}

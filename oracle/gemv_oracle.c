/*
 * gemv_oracle.c -- plain, slow CPU oracle for the fused decode GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * HIP library: its format and epilogue numbering below belongs to this file.
 *
 * What it computes (the plain definition of the method, no blocking/fusion):
 *   1. decode every weight of a row to its exact value (double);
 *   2. acc_i = sum_j w_ij * x_j in double, j ascending, and alongside it
 *      A_i = sum_j |w_ij * x_j| (the magnitude that bounds the rounding error);
 *   3. the epilogue as a SEPARATE pass over the rows, in double with libm exp;
 *   4. (prologue, at the end of the file) the signed Hadamard transform of x,
 *      each output as its own O(n) sum over Sylvester's matrix.
 *
 * Sources:
 *  - "feat(cuda): fuse activations and residual add into mmv f/q epilogues",
 *    sections "Summary" and "What changed": the product is the decode-path
 *    matrix-vector product with one output column; the post-matmul tails are
 *    sigmoid, silu, silu followed by an element-wise multiply with a per-row
 *    operand, and a residual add (also through a reshape of the output).
 *  - "ggml-cpu: fuse element-wise epilogues (ADD, MUL, SILU) into
 *    ggml_compute_forward_mul_mat", section "What": the MUL_MAT + MUL pair
 *    (gate x up) gives the plain multiply epilogue; section "Correctness":
 *    the fused path must produce the same values as running the element-wise
 *    op as its own pass, which is exactly what this file does.
 *  - Weight encodings: the 32-code block formats are the synthetic decode
 *    workloads' own definitions (8-bit: value = code * fp16 scale; 4-bit:
 *    value = (code - 8) * fp16 scale, two codes per byte).  Their byte layout
 *    (planar: codes, then fp16 scales at the next 256-byte boundary; low
 *    nibble = even element) is this project's choice, decoded here from the
 *    written specification, independently of the GPU loaders.
 *  - "vulkan: fuse the sign multiply into the Hadamard FWHT", Overview: the
 *    sign multiply and the block Hadamard transform of the activation.
 *
 * Parity pins live in the CPU test-suite: exhaustive fp16/bf16 decode against
 * library conversions, hand-built quantised blocks, exact rational brute force
 * on tiny GEMVs, exact-integer cases, closed forms (zero, identity,
 * permutation, rank-1 W) and epilogue identities.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* Weight formats as numbered by this file. */
#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2
#define ORC_Q8B32 3
#define ORC_Q4B32 4

/* Epilogues as numbered by this file. */
#define ORC_NONE 0
#define ORC_SIGMOID 1
#define ORC_SILU 2
#define ORC_SILU_MUL 3
#define ORC_MUL 4
#define ORC_ADD 5

#define ORC_OK 0
#define ORC_EBAD (-1)

/* ---- scalar decoders, written from the IEEE 754 interchange formats ---- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24); /* subnormal: frac * 2^-14 / 2^10 */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), expo - 25); /* 1.frac * 2^(e-15) */
    return sign ? -mag : mag;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_double(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int expo = (b >> 7) & 0xff;
    int frac = b & 0x7f;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -133); /* subnormal: frac * 2^-126 / 2^7 */
    else if (expo == 255)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(128 + frac), expo - 134); /* 1.frac * 2^(e-127) */
    return sign ? -mag : mag;
}

static int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

static uint16_t load_u16(const uint8_t *p)
{
    return (uint16_t)(p[0] | (p[1] << 8)); /* little-endian storage */
}

/* Total bytes of a weight matrix of N rows by K columns in format fmt,
 * or -1 when the arguments do not describe a valid matrix. */
int64_t oracle_weight_bytes(int fmt, int64_t N, int64_t K)
{
    if (N <= 0 || K <= 0)
        return -1;
    switch (fmt) {
    case ORC_F32:
        return N * K * 4;
    case ORC_F16:
    case ORC_BF16:
        return N * K * 2;
    case ORC_Q8B32:
        if (K % 32)
            return -1;
        return align256(N * K) + N * (K / 32) * 2;
    case ORC_Q4B32:
        if (K % 32)
            return -1;
        return align256(N * K / 2) + N * (K / 32) * 2;
    default:
        return -1;
    }
}

/* Decode row n of W into out[0..K-1] (exact values). */
int oracle_decode_row(int fmt, int64_t N, int64_t K, const void *W, int64_t n, double *out)
{
    const uint8_t *w = (const uint8_t *)W;
    if (oracle_weight_bytes(fmt, N, K) < 0 || n < 0 || n >= N)
        return ORC_EBAD;
    for (int64_t k = 0; k < K; ++k) {
        switch (fmt) {
        case ORC_F32: {
            float f;
            memcpy(&f, w + (n * K + k) * 4, 4);
            out[k] = (double)f;
            break;
        }
        case ORC_F16:
            out[k] = oracle_f16_to_double(load_u16(w + (n * K + k) * 2));
            break;
        case ORC_BF16:
            out[k] = oracle_bf16_to_double(load_u16(w + (n * K + k) * 2));
            break;
        case ORC_Q8B32: {
            int8_t code = (int8_t)w[n * K + k];
            const uint8_t *scales = w + align256(N * K);
            double scale = oracle_f16_to_double(load_u16(scales + (n * (K / 32) + k / 32) * 2));
            out[k] = (double)code * scale;
            break;
        }
        case ORC_Q4B32: {
            uint8_t byte = w[n * (K / 2) + k / 2];
            int code = (k % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
            const uint8_t *scales = w + align256(N * K / 2);
            double scale = oracle_f16_to_double(load_u16(scales + (n * (K / 32) + k / 32) * 2));
            out[k] = (double)(code - 8) * scale;
            break;
        }
        }
    }
    return ORC_OK;
}

/* acc[i] = sum_j w_ij x_j and absacc[i] = sum_j |w_ij x_j| for rows
 * row_begin <= i < row_end, written at acc[i - row_begin].  Accumulation is
 * in double with j ascending.  rowbuf is caller scratch of K doubles. */
int oracle_gemv_rows(int fmt, int64_t N, int64_t K, const void *W, const float *x,
                     int64_t row_begin, int64_t row_end, double *acc, double *absacc, double *rowbuf)
{
    if (row_begin < 0 || row_end > N || row_begin > row_end)
        return ORC_EBAD;
    for (int64_t i = row_begin; i < row_end; ++i) {
        if (oracle_decode_row(fmt, N, K, W, i, rowbuf) != ORC_OK)
            return ORC_EBAD;
        double s = 0.0, a = 0.0;
        for (int64_t j = 0; j < K; ++j) {
            double p = rowbuf[j] * (double)x[j];
            s += p;
            a += fabs(p);
        }
        acc[i - row_begin] = s;
        absacc[i - row_begin] = a;
    }
    return ORC_OK;
}

/* Logistic sigmoid and SiLU, written from their definitions. */
double oracle_sigmoid(double a) { return 1.0 / (1.0 + exp(-a)); }
double oracle_silu(double a) { return a / (1.0 + exp(-a)); }

/* The epilogue as its own pass over n values: y = act(acc) with the per-row
 * multiplier m or residual r where the epilogue uses one. */
int oracle_epilogue(int act, int64_t n, const double *acc, const float *m, const float *r, double *y)
{
    if (n < 0)
        return ORC_EBAD;
    if ((act == ORC_SILU_MUL || act == ORC_MUL) && !m)
        return ORC_EBAD;
    if (act == ORC_ADD && !r)
        return ORC_EBAD;
    for (int64_t i = 0; i < n; ++i) {
        double a = acc[i];
        switch (act) {
        case ORC_NONE:
            y[i] = a;
            break;
        case ORC_SIGMOID:
            y[i] = oracle_sigmoid(a);
            break;
        case ORC_SILU:
            y[i] = oracle_silu(a);
            break;
        case ORC_SILU_MUL:
            y[i] = oracle_silu(a) * (double)m[i];
            break;
        case ORC_MUL:
            y[i] = a * (double)m[i];
            break;
        case ORC_ADD:
            y[i] = a + (double)r[i];
            break;
        default:
            return ORC_EBAD;
        }
    }
    return ORC_OK;
}

/* Gated pair of products over the same x (the gate/GLU fusion that the mmv
 * kernels already had, per "feat(cuda): fuse activations and residual add
 * into mmv f/q epilogues", Summary): y_i = act(g_i) * u_i, where g and u are
 * the two row sums (each from oracle_gemv_rows, in double) and act is SILU
 * or SIGMOID.  A separate pass, in double. */
int oracle_glu_epilogue(int act, int64_t n, const double *g, const double *u, double *y)
{
    if (n < 0 || (act != ORC_SILU && act != ORC_SIGMOID))
        return ORC_EBAD;
    for (int64_t i = 0; i < n; ++i)
        y[i] = (act == ORC_SILU ? oracle_silu(g[i]) : oracle_sigmoid(g[i])) * u[i];
    return ORC_OK;
}

/* ---- signed Hadamard transform, a prologue to the product ----
 * "vulkan: fuse the sign multiply into the Hadamard FWHT", Overview: the
 * activation is multiplied element-wise by a sign vector (broadcast over the
 * sign vector's length), reshaped into blocks, and every block is multiplied
 * by a Hadamard matrix; the fused dispatch applies the signs while loading
 * the row, before the transform.  The page fixes neither the matrix's order
 * nor its scale; the readings taken here: Sylvester's matrix
 * H[i][j] = (-1)^popcount(i & j) of order n (a power of two), scaled by
 * 1/sqrt(n) so that the transform is orthonormal, and the sign of element k
 * of a row is s[k mod ns].
 *
 * Plain definition, one O(n) sum per output (no butterflies):
 *   y[b n + i] = n^-1/2 sum_j H[i][j] x[b n + j] s[(b n + j) mod ns]
 * in double, j ascending, and alongside it
 *   d[b n + i] = n^-1/2 sum_j |x[b n + j] s[(b n + j) mod ns]|,
 * the magnitude that bounds the rounding of any evaluation order.  x, s and
 * y hold one row of K values. */
static int popcount_parity(uint64_t v)
{
    int p = 0;
    while (v) {
        p ^= 1;
        v &= v - 1;
    }
    return p;
}

int oracle_fwht_signed(int64_t n, int64_t K, int64_t ns, const float *x, const float *s, double *y, double *d)
{
    if (n < 1 || (n & (n - 1)) != 0 || K < 1 || K % n != 0 || ns < 1 || K % ns != 0)
        return ORC_EBAD;
    const double scale = 1.0 / sqrt((double)n);
    for (int64_t b = 0; b < K; b += n) {
        for (int64_t i = 0; i < n; ++i) {
            double acc = 0.0, mag = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                const double v = (double)x[b + j] * (double)s[(b + j) % ns];
                acc += popcount_parity((uint64_t)(i & j)) ? -v : v;
                mag += fabs(v);
            }
            y[b + i] = acc * scale;
            d[b + i] = mag * scale;
        }
    }
    return ORC_OK;
}

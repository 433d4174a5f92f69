/*
 * gemv_fused.h -- C ABI of the fused-epilogue decode GEMV for MI355X (gfx950).
 *
 * The library computes, for a weight matrix W of N rows by K columns and an
 * f32 vector x of K values, the single-column product a_i = sum_j W_ij x_j
 * (the decode case with one output column) and applies one element-wise
 * epilogue to each a_i straight out of the accumulator, before the single
 * store of the result.  One kernel launch per call; W is streamed once from
 * HBM.
 *
 * Sources (web pages; the sections named are where each fact is stated):
 *  - "feat(cuda): fuse activations and residual add into mmv f/q epilogues",
 *    "Summary": the fusion applies to the matrix-vector kernels for float and
 *    quantised weights on the decode path, one destination column.
 *    "What changed": the tails sigmoid and silu, silu followed by a multiply
 *    with a per-row operand, and a residual add that may reach the product
 *    through a reshape; implementation notes: the activation is selected at
 *    run time (one value meaning "none"); the output keeps the product's
 *    element order even when the caller's buffer is a reshaped view; output i
 *    may overwrite operand element i, nothing else may overlap the weights or
 *    x; operands are contiguous and shaped like the output.
 *    "Why": every folded tail saves a launch, and the residual add also saves
 *    a write and a read of the output.
 *  - "ggml-cpu: fuse element-wise epilogues (ADD, MUL, SILU) into
 *    ggml_compute_forward_mul_mat", "What": the MUL_MAT + MUL pair (gate x up)
 *    is the plain multiply tail.  "Guards": epilogue operands are f32,
 *    identically shaped with no broadcast, row-contiguous and not transposed.
 *    "Correctness": the fused result equals the unfused one (ADD and MUL bit
 *    for bit).
 *  - "vulkan: fuse the sign multiply into the Hadamard FWHT", closing comment:
 *    an overlap guard must be reset between uses; here the checker keeps no
 *    state at all between calls.
 *
 * Ownership and threading: the caller owns every buffer; all data pointers
 * are device pointers (except where stated).  The library never allocates,
 * frees, copies or synchronises, and keeps no pointer after a call returns.
 * Calls are asynchronous on the given HIP stream (NULL = the null stream).
 * The library is stateless apart from a thread-local last-HIP-error, so it may
 * be called from several host threads.
 */
#ifndef GEMV_FUSED_H
#define GEMV_FUSED_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats.  W is row-major: row n produces output n.
 *  GEMV_W_F32   K f32 values per row (4 bytes each).
 *  GEMV_W_F16   K IEEE binary16 values per row.
 *  GEMV_W_BF16  K bfloat16 values per row.
 *  GEMV_W_Q8B32 blocks of 32 int8 codes, one fp16 scale per block,
 *               value = code * scale.  Byte image: the int8 code plane
 *               [N][K] row-major, then at offset align256(N*K) the fp16 scale
 *               plane [N][K/32] row-major.  K must be a multiple of 32.
 *  GEMV_W_Q4B32 blocks of 32 unsigned 4-bit codes, one fp16 scale per block,
 *               value = (code - 8) * scale.  Byte image: the nibble plane
 *               [N][K/2] (byte k/2 of a row holds element k in its low nibble
 *               when k is even, in its high nibble when k is odd), then at
 *               offset align256(N*K/2) the fp16 scale plane [N][K/32].
 *               K must be a multiple of 32.
 * align256(v) rounds v up to a multiple of 256.  All multi-byte values are
 * little-endian.  gemv_weight_bytes() gives the total byte count. */
typedef enum {
    GEMV_W_F32 = 0,
    GEMV_W_F16 = 1,
    GEMV_W_BF16 = 2,
    GEMV_W_Q8B32 = 3,
    GEMV_W_Q4B32 = 4
} gemv_wfmt;

/* Epilogues, applied to a = (W x)_i in f32:
 *  NONE      y = a
 *  SIGMOID   y = 1 / (1 + exp(-a))
 *  SILU      y = a / (1 + exp(-a))
 *  SILU_MUL  y = silu(a) * m_i      (needs mul_operand)
 *  MUL       y = a * m_i            (needs mul_operand)
 *  ADD       y = a + r_i            (needs add_operand)
 * Exactly one epilogue per call. */
typedef enum {
    GEMV_ACT_NONE = 0,
    GEMV_ACT_SIGMOID = 1,
    GEMV_ACT_SILU = 2,
    GEMV_ACT_SILU_MUL = 3,
    GEMV_ACT_MUL = 4,
    GEMV_ACT_ADD = 5
} gemv_act;

/* Status codes.  Every check runs before any launch; a rejected call
 * launches nothing and writes nothing. */
enum {
    GEMV_OK = 0,
    GEMV_E_NULL = -1,    /* a required pointer (W, x, acc, dst, a view's data) is NULL */
    GEMV_E_DIM = -2,     /* N or K < 1 or too large (also when W's byte
                            count would not fit in int64_t), K % 32 != 0 for
                            a block format, ncols outside 1..GEMV_MAX_NCOLS,
                            or the dst view does not hold ncols * N elements */
    GEMV_E_FMT = -3,     /* unknown weight format */
    GEMV_E_ACT = -4,     /* unknown epilogue */
    GEMV_E_OPERAND = -5, /* the epilogue's operand is missing, or an operand it
                            does not use is given */
    GEMV_E_LAYOUT = -6,  /* ndim outside 1..4, a negative extent, a view that
                            is not C-contiguous, or an operand whose shape
                            differs from dst's */
    GEMV_E_ALIAS = -7,   /* dst overlaps W, x or acc/operands other than by
                            being the identical view; a buffer whose bytes
                            would run past the top of the address space
                            counts as overlapping every other buffer */
    GEMV_E_ALIGN = -8,   /* W not 16-byte aligned, or an f32 pointer not
                            4-byte aligned */
    GEMV_E_HIP = -9      /* the HIP launch failed; see gemv_last_hip_error() */
};

#define GEMV_MAX_DIMS 4
#define GEMV_MAX_DIM_EXTENT (1LL << 31) /* N, K and ncols * N must be below this */
#define GEMV_MAX_NCOLS 8

/* A view of f32 device memory: element (i0, .., i_{ndim-1}) lives at
 * data + sum_d i_d * stride[d] (strides in elements).  The library accepts
 * only C-contiguous views (the stride of an extent-1 dimension is ignored),
 * so element i of the flattened view, in C order, is data[i].  A reshape of
 * the output (for example N = 4096 viewed as [32, 128]) is expressed by
 * giving dst and the operand that shape; the kernel writes in matmul order,
 * output row i to data[i]. */
typedef struct {
    float *data;
    int32_t ndim;
    int64_t shape[GEMV_MAX_DIMS];
    int64_t stride[GEMV_MAX_DIMS];
} gemv_view;

/* dst = epilogue(W x), one launch on hip_stream.
 *  W           device pointer to gemv_weight_bytes(wfmt, N, K) bytes in
 *              format wfmt; 16-byte aligned.
 *  N, K        rows (outputs) and columns (inputs) of W.
 *  x           device pointer to K f32 values.
 *  act         a gemv_act value.
 *  mul_operand f32 view, same shape as dst; required by SILU_MUL and MUL,
 *              must be NULL otherwise.
 *  add_operand f32 view, same shape as dst; required by ADD, must be NULL
 *              otherwise.
 *  dst         f32 view holding N elements.  It may be the identical view of
 *              the epilogue's operand (an in-place update: element i is read,
 *              then written, by the same thread); it may not otherwise
 *              overlap the operand, and it may never overlap W or x, which
 *              every row reads across the whole reduction.
 *  hip_stream  a hipStream_t, or NULL.
 * Returns GEMV_OK or a negative status.  Asynchronous: returns after the
 * launch is enqueued. */
int gemv_fused(const void *W, int wfmt, int64_t N, int64_t K, const float *x, int act,
               const gemv_view *mul_operand, const gemv_view *add_operand,
               const gemv_view *dst, void *hip_stream);

/* The gated pair of products over one x (the gate fusion of the
 * matrix-vector kernels that "feat(cuda): fuse activations and residual add
 * into mmv f/q epilogues", Summary, leaves in place, and the gate x up product
 * of "ggml-cpu: fuse element-wise epilogues (ADD, MUL, SILU) into
 * ggml_compute_forward_mul_mat", What): one launch computes
 *     dst_i = act((W_gate x)_i) * (W_up x)_i
 * with act GEMV_ACT_SILU (SwiGLU) or GEMV_ACT_SIGMOID.  Both matrices have
 * format wfmt and shape N x K (16-byte aligned; they may be the same memory);
 * x is K f32 values; dst is an f32 view holding N elements that overlaps
 * neither matrix nor x.  Each row sum is formed exactly as gemv_fused forms it,
 * so the result equals gemv_fused(W_up, NONE) followed by
 * gemv_fused(W_gate, SILU_MUL, m = that output) bit for bit.  Returns GEMV_OK
 * or a negative status (GEMV_E_ACT for any other act); asynchronous on
 * hip_stream; allocates nothing. */
int gemv_glu(const void *W_gate, const void *W_up, int wfmt, int64_t N, int64_t K, const float *x, int act,
             const gemv_view *dst, void *hip_stream);

/* The gated pair over 1..8 destination columns (small-batch or speculative
 * decode): column b of x ([ncols][K] f32) gives
 *     dst[b * N + i] = act((W_gate x_b)_i) * (W_up x_b)_i
 * with the matrices, act and alignment rules of gemv_glu; dst is an f32
 * view holding ncols * N elements that overlaps neither matrix nor x.
 * Normally one launch: both matrices are read once for all columns, each
 * chunk of a row is decoded once and multiplied into every column, and each
 * row sum is formed exactly as gemv_fused_ncols forms it on its vector-ALU
 * column kernels, so column b equals gemv_glu on x_b bit for bit (ncols == 1
 * is gemv_glu).  Where gemv_ncols_kernel reports GEMV_KERNEL_COLUMNS_MATRIX
 * for (wfmt, N, K, ncols) and act is SILU, two matrix-core launches are
 * faster and are taken instead: the up product into dst, then the gate's
 * with silu(g) * u in place; the results then carry the matrix-core
 * kernel's precision (within the formats' tolerances, not bit for bit).
 * Returns GEMV_OK or a negative status (GEMV_E_DIM for ncols outside 1..8);
 * asynchronous on hip_stream; allocates nothing. */
int gemv_glu_ncols(const void *W_gate, const void *W_up, int wfmt, int64_t N, int64_t K, int64_t ncols,
                   const float *x, int act, const gemv_view *dst, void *hip_stream);

/* The host-side checks of gemv_glu_ncols; no HIP call. */
int gemv_glu_ncols_validate(const void *W_gate, const void *W_up, int wfmt, int64_t N, int64_t K, int64_t ncols,
                            const float *x, int act, const gemv_view *dst);

/* The host-side checks of gemv_glu; no HIP call. */
int gemv_glu_validate(const void *W_gate, const void *W_up, int wfmt, int64_t N, int64_t K, const float *x,
                      int act, const gemv_view *dst);

/* Several destination columns over one W (small-batch or speculative decode).
 * "feat(cuda): fuse activations and residual add into mmv f/q epilogues",
 * Summary, states the fused matrix-vector path for one destination column;
 * this entry widens it to ncols columns, each exactly one gemv_fused column:
 *     dst[b*N + i] = epilogue((W x_b)_i, operand[b*N + i]),  x_b = x + b*K,
 * for b < ncols, i < N.  W is streamed from HBM once for all columns.
 *  x           device pointer to ncols * K f32 values, column b at x + b*K.
 *  ncols       1..GEMV_MAX_NCOLS (else GEMV_E_DIM).
 *  mul_operand, add_operand, dst: f32 views of ncols * N elements each, read
 *              in C order as [ncols][N] (any shape with that flattening, such
 *              as [ncols, N] or [ncols, 32, 128]); operand rules, the in-place
 *              case and the overlap rule are those of gemv_fused, with x
 *              spanning ncols * K floats.
 * Kernels (gemv_ncols_kernel names the one a call takes): f32, and the
 * other formats at few columns, run a vector-ALU column kernel whose column
 * b is bit for bit the gemv_fused result for x_b and operand row b whenever
 * K meets the fast-path conditions (K a multiple of the 16-byte chunk: 4
 * f32, 8 f16/bf16 values; always for block formats).  The 16-bit and block
 * formats at more columns run on the matrix cores: there x is carried as
 * two 16-bit pieces per value (f16 pieces of the column scaled by a power
 * of two: 2^-20 relative, and below 2^-48 of the column's largest |x|
 * absolutely; bf16 pieces for bf16 weights: 2^-15 relative), the result
 * agrees with gemv_fused within the format's tolerance, and each column is
 * independent of the others bit for bit.  ncols == 1 is gemv_fused itself.
 * Returns GEMV_OK or a negative status; asynchronous on hip_stream;
 * allocates nothing. */
int gemv_fused_ncols(const void *W, int wfmt, int64_t N, int64_t K, int64_t ncols, const float *x, int act,
                     const gemv_view *mul_operand, const gemv_view *add_operand, const gemv_view *dst,
                     void *hip_stream);

/* The kernel gemv_fused_ncols launches for a format and shape on the current
 * device (the choice depends on the device's compute-unit count, which is
 * queried once per device).  Not part of any computation: for tests,
 * benchmarks and tuning.  Returns a gemv_kernel value, or GEMV_E_FMT /
 * GEMV_E_DIM for arguments gemv_fused_ncols would reject on those grounds
 * (ncols == 1 needs no HIP call). */
typedef enum {
    GEMV_KERNEL_ONE_COLUMN = 1,      /* gemv_fused's kernels (ncols == 1) */
    GEMV_KERNEL_COLUMNS = 2,         /* vector-ALU column kernel, 16-byte chunks */
    GEMV_KERNEL_COLUMNS_GENERIC = 3, /* vector-ALU column kernel, element loads */
    GEMV_KERNEL_COLUMNS_MATRIX = 4   /* matrix-core column kernel */
} gemv_kernel;
int gemv_ncols_kernel(int wfmt, int64_t N, int64_t K, int64_t ncols);

/* The host-side checks of gemv_fused_ncols; no HIP call. */
int gemv_fused_ncols_validate(const void *W, int wfmt, int64_t N, int64_t K, int64_t ncols, const float *x,
                              int act, const gemv_view *mul_operand, const gemv_view *add_operand,
                              const gemv_view *dst);

/* The signed Hadamard transform ("vulkan: fuse the sign multiply into the
 * Hadamard FWHT", Overview: the sign multiply applied while the row is
 * loaded, then the block Hadamard transform, one dispatch):
 *     dst[r][b n + i] = n^-1/2 sum_j H[i][j] x[r][b n + j] s[(b n + j) mod nsigns]
 * for every row r < nrows and block b, with H Sylvester's Hadamard matrix
 * (H[i][j] = (-1)^popcount(i & j)).  The page fixes neither the order nor
 * the scale of H; this library takes the natural (Sylvester) order and the
 * orthonormal scale 1/sqrt(n).
 *  x, dst      device pointers to nrows * K f32 values (rows contiguous); dst
 *              may be x itself (in place) but may not otherwise overlap x,
 *              and may not overlap the signs.
 *  signs       device pointer to nsigns f32 values (typically +-1), applied
 *              with period nsigns along each row.
 *  n           block length: a power of two, 1..1024, dividing K.
 *  nsigns      >= 1, dividing K.
 * Errors: GEMV_E_NULL, GEMV_E_DIM (shapes; nrows * K must be below
 * GEMV_MAX_DIM_EXTENT), GEMV_E_ALIGN (4-byte alignment), GEMV_E_ALIAS,
 * GEMV_E_HIP.  One launch on hip_stream; allocates nothing. */
int gemv_fwht_signed(const float *x, const float *signs, int64_t nrows, int64_t K, int64_t n, int64_t nsigns,
                     float *dst, void *hip_stream);

/* The host-side checks of gemv_fwht_signed; no HIP call. */
int gemv_fwht_signed_validate(const float *x, const float *signs, int64_t nrows, int64_t K, int64_t n,
                              int64_t nsigns, const float *dst);

/* The product after the signed Hadamard transform, in one launch: each
 * workgroup transforms x while staging it (the signs applied as x is loaded)
 * and then streams W as gemv_fused does:
 *     dst = epilogue(W . FWHT_n(x * s))
 * Arguments as for gemv_fused, plus signs, n and nsigns as for
 * gemv_fwht_signed (one row of K values).  The transform uses the same code
 * as gemv_fwht_signed, so the result is bit for bit gemv_fwht_signed into a
 * buffer followed by gemv_fused on it.  Carried by the chunked kernel only:
 * rows must be whole 16-byte chunks (K a multiple of 4 for f32, 8 for
 * f16/bf16, 32 for the block formats) and x must fit its LDS staging (K up
 * to 40960 for f32, 27306 for f16/bf16); otherwise GEMV_E_DIM.  dst may not
 * overlap the signs. */
int gemv_fused_fwht(const void *W, int wfmt, int64_t N, int64_t K, const float *x, const float *signs, int64_t n,
                    int64_t nsigns, int act, const gemv_view *mul_operand, const gemv_view *add_operand,
                    const gemv_view *dst, void *hip_stream);

/* The host-side checks of gemv_fused_fwht; no HIP call. */
int gemv_fused_fwht_validate(const void *W, int wfmt, int64_t N, int64_t K, const float *x, const float *signs,
                             int64_t n, int64_t nsigns, int act, const gemv_view *mul_operand,
                             const gemv_view *add_operand, const gemv_view *dst);

/* The host-side checks of gemv_fused, with no HIP call and no dereference of
 * any device pointer: returns the status gemv_fused would return before
 * launching.  Safe on a machine with no GPU. */
int gemv_validate(const void *W, int wfmt, int64_t N, int64_t K, const float *x, int act,
                  const gemv_view *mul_operand, const gemv_view *add_operand,
                  const gemv_view *dst);

/* The epilogue alone, as a separate element-wise pass (the unfused path):
 * dst_i = epilogue(acc_i) for i < N, one launch on hip_stream.
 *  acc         device pointer to N contiguous f32 values (a gemv_fused
 *              result with act = NONE).
 *  mul_operand, add_operand, dst: as for gemv_fused.  dst may be the same
 *              memory as acc or as the operand (element for element); a
 *              partial overlap is rejected.
 * It uses the same device epilogue code as gemv_fused, so for the same a_i
 * the fused and unfused results are identical. */
int gemv_epilogue(int act, int64_t N, const float *acc, const gemv_view *mul_operand,
                  const gemv_view *add_operand, const gemv_view *dst, void *hip_stream);

/* The host-side checks of gemv_epilogue; no HIP call. */
int gemv_epilogue_validate(int act, int64_t N, const float *acc, const gemv_view *mul_operand,
                           const gemv_view *add_operand, const gemv_view *dst);

/* Size in bytes of an N x K weight matrix in format wfmt, or a negative
 * status (GEMV_E_FMT, GEMV_E_DIM) when the arguments are invalid. */
int64_t gemv_weight_bytes(int wfmt, int64_t N, int64_t K);

/* A static, human-readable description of a status code. */
const char *gemv_strerror(int status);

/* The hipError_t of the last failed launch on the calling thread (0 if
 * none); reset to 0 by every successful launching call (gemv_fused,
 * gemv_fused_ncols, gemv_glu, gemv_glu_ncols, gemv_epilogue, gemv_fwht_signed,
 * gemv_fused_fwht). */
int gemv_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMV_FUSED_H */

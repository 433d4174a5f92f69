// Host-side argument checks for the fused decode GEMV: shapes, formats,
// operand presence, contiguity, alignment and the overlap rule.  No HIP call
// and no dereference of a device pointer, so it runs on a machine without a
// GPU.  Stateless: nothing is remembered between calls (a guard that keeps
// state across uses must be reset, as the closing comment of "vulkan: fuse
// the sign multiply into the Hadamard FWHT" found; this one keeps none).
//
// The overlap rule is the one of "feat(cuda): fuse activations and residual
// add into mmv f/q epilogues", "What changed" (implementation notes): writing
// output i over operand element i is safe, since each output reads only its
// own operand element before its one store; any other overlap of dst with the
// weights or with x is refused, because every output reads all of them.
// Operands are contiguous and of dst's shape.  "ggml-cpu: fuse element-wise
// epilogues (ADD, MUL, SILU) into ggml_compute_forward_mul_mat", "Guards",
// adds the operand conditions: f32, no broadcast, rows contiguous.
#include "gemv_internal.h"

#include <climits>
#include <cstdint>

namespace gemv {

int64_t weight_bytes(int wfmt, int64_t N, int64_t K)
{
    if (wfmt < GEMV_W_F32 || wfmt > GEMV_W_Q4B32)
        return GEMV_E_FMT;
    if (N < 1 || K < 1 || N >= GEMV_MAX_DIM_EXTENT || K >= GEMV_MAX_DIM_EXTENT)
        return GEMV_E_DIM;
    switch (wfmt) {
    case GEMV_W_F32:
        // N * K < 2^62 cannot overflow; four bytes per weight can
        if (N * K > INT64_MAX / 4)
            return GEMV_E_DIM;
        return N * K * 4;
    case GEMV_W_F16:
    case GEMV_W_BF16:
        return N * K * 2;
    case GEMV_W_Q8B32:
        if (K % 32)
            return GEMV_E_DIM;
        return align256(N * K) + N * (K / 32) * 2;
    default: /* GEMV_W_Q4B32 */
        if (K % 32)
            return GEMV_E_DIM;
        return align256(N * K / 2) + N * (K / 32) * 2;
    }
}

namespace {

struct Span {
    uintptr_t lo, hi; // [lo, hi)
};

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Checks one view: ndim, extents, C-contiguity (extent-1 strides ignored).
// On success stores the element count.
int check_view(const gemv_view *v, int64_t *numel)
{
    if (v->ndim < 1 || v->ndim > GEMV_MAX_DIMS)
        return GEMV_E_LAYOUT;
    int64_t n = 1;
    for (int d = 0; d < v->ndim; ++d) {
        if (v->shape[d] < 0)
            return GEMV_E_LAYOUT;
        if (v->shape[d] >= GEMV_MAX_DIM_EXTENT)
            return GEMV_E_DIM;
        n *= v->shape[d];
        if (n >= GEMV_MAX_DIM_EXTENT)
            return GEMV_E_DIM;
    }
    int64_t expect = 1;
    for (int d = v->ndim - 1; d >= 0; --d) {
        if (v->shape[d] != 1 && v->stride[d] != expect)
            return GEMV_E_LAYOUT;
        expect *= v->shape[d];
    }
    *numel = n;
    return GEMV_OK;
}

bool same_shape(const gemv_view *a, const gemv_view *b)
{
    if (a->ndim != b->ndim)
        return false;
    for (int d = 0; d < a->ndim; ++d)
        if (a->shape[d] != b->shape[d])
            return false;
    return true;
}

// [p, p + bytes) as addresses.  A span that would run past the top of the
// address space is no real buffer: it is widened to the whole space, so that
// it overlaps every other buffer and the call is rejected.
Span span_of(const void *p, int64_t bytes)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    const uintptr_t b = static_cast<uintptr_t>(bytes);
    if (b > UINTPTR_MAX - lo)
        return Span{0, UINTPTR_MAX};
    return Span{lo, lo + b};
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_act(int act) { return (act < GEMV_ACT_NONE || act > GEMV_ACT_ADD) ? GEMV_E_ACT : GEMV_OK; }

bool uses_mul(int act) { return act == GEMV_ACT_SILU_MUL || act == GEMV_ACT_MUL; }
bool uses_add(int act) { return act == GEMV_ACT_ADD; }

// Operand presence, null data, layout of dst and the active operand, numel of
// dst == N, 4-byte alignment.  Writes the active operand (or NULL).
int check_epilogue_views(int act, int64_t N, const gemv_view *mul_operand, const gemv_view *add_operand,
                         const gemv_view *dst, const gemv_view **operand)
{
    if (!dst || !dst->data)
        return GEMV_E_NULL;
    if ((mul_operand && !mul_operand->data) || (add_operand && !add_operand->data))
        return GEMV_E_NULL;
    if (uses_mul(act) != (mul_operand != nullptr) || uses_add(act) != (add_operand != nullptr))
        return GEMV_E_OPERAND;
    *operand = uses_mul(act) ? mul_operand : (uses_add(act) ? add_operand : nullptr);

    int64_t nd = 0;
    int st = check_view(dst, &nd);
    if (st != GEMV_OK)
        return st;
    if (nd != N)
        return GEMV_E_DIM;
    if (*operand) {
        int64_t no = 0;
        st = check_view(*operand, &no);
        if (st != GEMV_OK)
            return st;
        if (!same_shape(*operand, dst))
            return GEMV_E_LAYOUT;
    }
    if (!aligned(dst->data, 4) || (*operand && !aligned((*operand)->data, 4)))
        return GEMV_E_ALIGN;
    return GEMV_OK;
}

} // namespace

int validate_ncols(const void *W, int wfmt, int64_t N, int64_t K, int64_t ncols, const float *x, int act,
                   const gemv_view *mul_operand, const gemv_view *add_operand, const gemv_view *dst)
{
    if (!W || !x)
        return GEMV_E_NULL;
    if (wfmt < GEMV_W_F32 || wfmt > GEMV_W_Q4B32)
        return GEMV_E_FMT;
    int st = check_act(act);
    if (st != GEMV_OK)
        return st;
    if (ncols < 1 || ncols > GEMV_MAX_NCOLS)
        return GEMV_E_DIM;
    int64_t wbytes = weight_bytes(wfmt, N, K);
    if (wbytes < 0)
        return static_cast<int>(wbytes);
    const int64_t nout = N * ncols; // N < 2^31 and ncols <= 8: no overflow
    if (nout >= GEMV_MAX_DIM_EXTENT)
        return GEMV_E_DIM;

    const gemv_view *operand = nullptr;
    st = check_epilogue_views(act, nout, mul_operand, add_operand, dst, &operand);
    if (st != GEMV_OK)
        return st;
    if (!aligned(W, 16) || !aligned(x, 4))
        return GEMV_E_ALIGN;

    // dst never overlaps the matmul inputs; it overlaps the operand only as
    // the identical view (same pointer; shapes are equal and both contiguous).
    Span sd = span_of(dst->data, nout * 4);
    if (overlap(sd, span_of(W, wbytes)) || overlap(sd, span_of(x, ncols * K * 4)))
        return GEMV_E_ALIAS;
    if (operand && overlap(sd, span_of(operand->data, nout * 4)) && operand->data != dst->data)
        return GEMV_E_ALIAS;
    return GEMV_OK;
}

int validate(const void *W, int wfmt, int64_t N, int64_t K, const float *x, int act,
             const gemv_view *mul_operand, const gemv_view *add_operand, const gemv_view *dst)
{
    return validate_ncols(W, wfmt, N, K, 1, x, act, mul_operand, add_operand, dst);
}

// The gated pair: both matrices of one format and shape, the gate act SILU
// or SIGMOID, dst (N f32, C-contiguous) overlapping neither matrix nor x.
int validate_glu(const void *W_gate, const void *W_up, int wfmt, int64_t N, int64_t K, const float *x, int act,
                 const gemv_view *dst)
{
    return validate_glu_ncols(W_gate, W_up, wfmt, N, K, 1, x, act, dst);
}

// The gated pair over ncols destination columns: x is [ncols][K], dst holds
// ncols * N values; otherwise the rules of the one-column pair.
int validate_glu_ncols(const void *W_gate, const void *W_up, int wfmt, int64_t N, int64_t K, int64_t ncols,
                       const float *x, int act, const gemv_view *dst)
{
    if (!W_gate || !W_up || !x)
        return GEMV_E_NULL;
    if (wfmt < GEMV_W_F32 || wfmt > GEMV_W_Q4B32)
        return GEMV_E_FMT;
    if (act != GEMV_ACT_SILU && act != GEMV_ACT_SIGMOID)
        return GEMV_E_ACT;
    if (ncols < 1 || ncols > GEMV_MAX_NCOLS)
        return GEMV_E_DIM;
    int64_t wbytes = weight_bytes(wfmt, N, K);
    if (wbytes < 0)
        return static_cast<int>(wbytes);
    const int64_t nout = N * ncols; // N < 2^31 and ncols <= 8: no overflow
    if (nout >= GEMV_MAX_DIM_EXTENT)
        return GEMV_E_DIM;
    const gemv_view *operand = nullptr;
    int st = check_epilogue_views(GEMV_ACT_NONE, nout, nullptr, nullptr, dst, &operand);
    if (st != GEMV_OK)
        return st;
    if (!aligned(W_gate, 16) || !aligned(W_up, 16) || !aligned(x, 4))
        return GEMV_E_ALIGN;
    Span sd = span_of(dst->data, nout * 4);
    if (overlap(sd, span_of(W_gate, wbytes)) || overlap(sd, span_of(W_up, wbytes)) ||
        overlap(sd, span_of(x, ncols * K * 4)))
        return GEMV_E_ALIAS;
    return GEMV_OK;
}

// The signed Hadamard transform's shape rules: n a power of two up to 1024
// (one wave's tile), dividing K; the sign period dividing K.
namespace {
int check_fwht_shape(int64_t K, int64_t n, int64_t nsigns)
{
    if (n < 1 || n > 1024 || (n & (n - 1)) != 0 || K % n != 0)
        return GEMV_E_DIM;
    if (nsigns < 1 || K % nsigns != 0)
        return GEMV_E_DIM;
    return GEMV_OK;
}
} // namespace

int validate_fwht(const float *x, const float *signs, int64_t nrows, int64_t K, int64_t n, int64_t nsigns,
                  const float *dst)
{
    if (!x || !signs || !dst)
        return GEMV_E_NULL;
    if (nrows < 1 || K < 1 || nrows >= GEMV_MAX_DIM_EXTENT || K >= GEMV_MAX_DIM_EXTENT ||
        nrows * K >= GEMV_MAX_DIM_EXTENT)
        return GEMV_E_DIM;
    int st = check_fwht_shape(K, n, nsigns);
    if (st != GEMV_OK)
        return st;
    if (!aligned(x, 4) || !aligned(signs, 4) || !aligned(dst, 4))
        return GEMV_E_ALIGN;
    // in place (dst == x) or disjoint; never over the signs
    Span sd = span_of(dst, nrows * K * 4);
    if (overlap(sd, span_of(x, nrows * K * 4)) && dst != x)
        return GEMV_E_ALIAS;
    if (overlap(sd, span_of(signs, nsigns * 4)))
        return GEMV_E_ALIAS;
    return GEMV_OK;
}

// The product after the transform: the checks of gemv_fused, the transform's
// shape rules, and the chunked kernel (rows of whole 16-byte chunks, x within
// the LDS limit), the only one that carries the transform; dst never
// overlaps the signs.
int validate_fused_fwht(const void *W, int wfmt, int64_t N, int64_t K, const float *x, const float *signs, int64_t n,
                        int64_t nsigns, int act, const gemv_view *mul_operand, const gemv_view *add_operand,
                        const gemv_view *dst)
{
    int st = validate(W, wfmt, N, K, x, act, mul_operand, add_operand, dst);
    if (st != GEMV_OK)
        return st;
    if (!signs)
        return GEMV_E_NULL;
    st = check_fwht_shape(K, n, nsigns);
    if (st != GEMV_OK)
        return st;
    // weights per 16-byte chunk and LDS floats per chunk of the chunked kernel
    static const int kE[] = {4, 8, 8, 16, 32}, kXS[] = {4, 12, 12, 20, 36};
    const int64_t row_bytes = wfmt == GEMV_W_F32 ? K * 4 : (wfmt == GEMV_W_Q8B32 ? K : (wfmt == GEMV_W_Q4B32 ? K / 2 : K * 2));
    if (row_bytes % 16 != 0 || (K / kE[wfmt]) * kXS[wfmt] * 4 > 160 * 1024)
        return GEMV_E_DIM;
    if (!aligned(signs, 4))
        return GEMV_E_ALIGN;
    if (overlap(span_of(dst->data, N * 4), span_of(signs, nsigns * 4)))
        return GEMV_E_ALIAS;
    return GEMV_OK;
}

int validate_epilogue(int act, int64_t N, const float *acc, const gemv_view *mul_operand,
                      const gemv_view *add_operand, const gemv_view *dst)
{
    if (!acc)
        return GEMV_E_NULL;
    int st = check_act(act);
    if (st != GEMV_OK)
        return st;
    if (N < 1 || N >= GEMV_MAX_DIM_EXTENT)
        return GEMV_E_DIM;
    const gemv_view *operand = nullptr;
    st = check_epilogue_views(act, N, mul_operand, add_operand, dst, &operand);
    if (st != GEMV_OK)
        return st;
    if (!aligned(acc, 4))
        return GEMV_E_ALIGN;
    // Element-wise pass: dst may be the same memory as acc or the operand,
    // never a shifted overlap of either.
    Span sd = span_of(dst->data, N * 4);
    if (overlap(sd, span_of(acc, N * 4)) && acc != dst->data)
        return GEMV_E_ALIAS;
    if (operand && overlap(sd, span_of(operand->data, N * 4)) && operand->data != dst->data)
        return GEMV_E_ALIAS;
    return GEMV_OK;
}

const char *strerror_of(int status)
{
    switch (status) {
    case GEMV_OK:
        return "ok";
    case GEMV_E_NULL:
        return "a required pointer is NULL";
    case GEMV_E_DIM:
        return "invalid dimensions (N, K < 1 or too large, K not a multiple of 32 for a block "
               "format, ncols outside 1..8, or dst does not hold ncols * N elements)";
    case GEMV_E_FMT:
        return "unknown weight format";
    case GEMV_E_ACT:
        return "unknown epilogue";
    case GEMV_E_OPERAND:
        return "epilogue operand missing, or an unused operand was given";
    case GEMV_E_LAYOUT:
        return "view is not C-contiguous, has a bad rank or extent, or its shape differs from dst";
    case GEMV_E_ALIAS:
        return "dst overlaps W, x, or an operand other than as the identical view";
    case GEMV_E_ALIGN:
        return "misaligned pointer (W needs 16 bytes, f32 data 4 bytes)";
    case GEMV_E_HIP:
        return "HIP launch failed (see gemv_last_hip_error)";
    default:
        return "unknown status";
    }
}

} // namespace gemv

extern "C" {

int gemv_validate(const void *W, int wfmt, int64_t N, int64_t K, const float *x, int act,
                  const gemv_view *mul_operand, const gemv_view *add_operand, const gemv_view *dst)
{
    return gemv::validate(W, wfmt, N, K, x, act, mul_operand, add_operand, dst);
}

int gemv_fused_ncols_validate(const void *W, int wfmt, int64_t N, int64_t K, int64_t ncols, const float *x, int act,
                              const gemv_view *mul_operand, const gemv_view *add_operand, const gemv_view *dst)
{
    return gemv::validate_ncols(W, wfmt, N, K, ncols, x, act, mul_operand, add_operand, dst);
}

int gemv_fwht_signed_validate(const float *x, const float *signs, int64_t nrows, int64_t K, int64_t n, int64_t nsigns,
                              const float *dst)
{
    return gemv::validate_fwht(x, signs, nrows, K, n, nsigns, dst);
}

int gemv_fused_fwht_validate(const void *W, int wfmt, int64_t N, int64_t K, const float *x, const float *signs,
                             int64_t n, int64_t nsigns, int act, const gemv_view *mul_operand,
                             const gemv_view *add_operand, const gemv_view *dst)
{
    return gemv::validate_fused_fwht(W, wfmt, N, K, x, signs, n, nsigns, act, mul_operand, add_operand, dst);
}

int gemv_epilogue_validate(int act, int64_t N, const float *acc, const gemv_view *mul_operand,
                           const gemv_view *add_operand, const gemv_view *dst)
{
    return gemv::validate_epilogue(act, N, acc, mul_operand, add_operand, dst);
}

int gemv_glu_ncols_validate(const void *W_gate, const void *W_up, int wfmt, int64_t N, int64_t K, int64_t ncols,
                            const float *x, int act, const gemv_view *dst)
{
    return gemv::validate_glu_ncols(W_gate, W_up, wfmt, N, K, ncols, x, act, dst);
}

int gemv_glu_validate(const void *W_gate, const void *W_up, int wfmt, int64_t N, int64_t K, const float *x, int act,
                      const gemv_view *dst)
{
    return gemv::validate_glu(W_gate, W_up, wfmt, N, K, x, act, dst);
}

int64_t gemv_weight_bytes(int wfmt, int64_t N, int64_t K) { return gemv::weight_bytes(wfmt, N, K); }

const char *gemv_strerror(int status) { return gemv::strerror_of(status); }

} // extern "C"

// Internal declarations shared by the host checks (gemv_validate.cpp) and the
// HIP translation unit (gemv_kernels.hip).  Host code only.
#pragma once

#include <cstdint>

#include "gemv_fused.h"

namespace gemv {

inline int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

int64_t weight_bytes(int wfmt, int64_t N, int64_t K);
int validate(const void *W, int wfmt, int64_t N, int64_t K, const float *x, int act,
             const gemv_view *mul_operand, const gemv_view *add_operand, const gemv_view *dst);
int validate_epilogue(int act, int64_t N, const float *acc, const gemv_view *mul_operand,
                      const gemv_view *add_operand, const gemv_view *dst);
int validate_glu(const void *W_gate, const void *W_up, int wfmt, int64_t N, int64_t K, const float *x, int act,
                 const gemv_view *dst);
int validate_glu_ncols(const void *W_gate, const void *W_up, int wfmt, int64_t N, int64_t K, int64_t ncols,
                       const float *x, int act, const gemv_view *dst);
const char *strerror_of(int status);
int validate_ncols(const void *W, int wfmt, int64_t N, int64_t K, int64_t ncols, const float *x, int act,
                   const gemv_view *mul_operand, const gemv_view *add_operand, const gemv_view *dst);

int validate_fwht(const float *x, const float *signs, int64_t nrows, int64_t K, int64_t n, int64_t nsigns,
                  const float *dst);
int validate_fused_fwht(const void *W, int wfmt, int64_t N, int64_t K, const float *x, const float *signs, int64_t n,
                        int64_t nsigns, int act, const gemv_view *mul_operand, const gemv_view *add_operand,
                        const gemv_view *dst);

// Arguments of one several-column product, checked by validate_ncols.
struct ColsArgs {
    const unsigned char *W;
    const float *x;
    int N, K, act;
    const float *m, *r;
    float *dst;
    const unsigned char *W2 = nullptr; // up matrix of a gated pair (act is the gate's)
};

// The matrix-core column kernels (16-bit and block formats).  The plan: tiles
// of 16 rows per workgroup (rt, 0 where the kernels are not taken), W steps
// per wave (sw; per wave and segment when kseg > 0), x octets per builder
// lane (vo), and the segment length in values (kseg, 0 for a single
// segment), for a device of `cus` compute units.  launch_cols_mfma launches
// on the stream and returns the hipError_t of the launch, or -1 without
// launching where the plan is empty.
struct MfmaPlan {
    int rt, sw, vo, kseg;
};
MfmaPlan cols_mfma_plan(int wfmt, int ncols, int64_t N, int64_t K, int64_t cus);
int launch_cols_mfma(int wfmt, int ncols, const ColsArgs &c, void *stream);

// Records a launch's hipError_t as the calling thread's last HIP error and
// maps it to GEMV_OK or GEMV_E_HIP.
int finish_launch(int hip_error);
int last_hip_error();

} // namespace gemv

// Entry points of the fused-epilogue decode GEMV for one output column
// (gemv_fused, the gated pair gemv_glu, the separate epilogue pass
// gemv_epilogue) and the library's per-thread last-HIP-error state.  The
// kernels themselves are in gemv_fast.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "gemv_fast.h"

namespace gemv {

namespace {
thread_local int t_last_hip_error = 0;
}

int finish_launch(int hip_error)
{
    t_last_hip_error = hip_error;
    return hip_error == (int)hipSuccess ? GEMV_OK : GEMV_E_HIP;
}

int last_hip_error() { return t_last_hip_error; }

} // namespace gemv

extern "C" {

int gemv_fused(const void *W, int wfmt, int64_t N, int64_t K, const float *x, int act,
               const gemv_view *mul_operand, const gemv_view *add_operand, const gemv_view *dst, void *hip_stream)
{
    int st = gemv::validate(W, wfmt, N, K, x, act, mul_operand, add_operand, dst);
    if (st != GEMV_OK)
        return st;
    gemv::Call c{static_cast<const unsigned char *>(W), nullptr, x, (int)N, (int)K, act,
                 mul_operand ? mul_operand->data : nullptr, add_operand ? add_operand->data : nullptr, dst->data,
                 gemv::FwhtArgs{}};
    return gemv::finish(gemv::dispatch_any<false>(wfmt, c, static_cast<hipStream_t>(hip_stream)));
}

int gemv_glu(const void *W_gate, const void *W_up, int wfmt, int64_t N, int64_t K, const float *x, int act,
             const gemv_view *dst, void *hip_stream)
{
    int st = gemv::validate_glu(W_gate, W_up, wfmt, N, K, x, act, dst);
    if (st != GEMV_OK)
        return st;
    gemv::Call c{static_cast<const unsigned char *>(W_gate), static_cast<const unsigned char *>(W_up), x, (int)N,
                 (int)K, act, nullptr, nullptr, dst->data, gemv::FwhtArgs{}};
    return gemv::finish(gemv::dispatch_any<true>(wfmt, c, static_cast<hipStream_t>(hip_stream)));
}

int gemv_epilogue(int act, int64_t N, const float *acc, const gemv_view *mul_operand, const gemv_view *add_operand,
                  const gemv_view *dst, void *hip_stream)
{
    int st = gemv::validate_epilogue(act, N, acc, mul_operand, add_operand, dst);
    if (st != GEMV_OK)
        return st;
    int n = (int)N;
    const float *m = mul_operand ? mul_operand->data : nullptr;
    const float *r = add_operand ? add_operand->data : nullptr;
    float *d = dst->data;
    void *args[] = {&n, &acc, &act, &m, &r, &d};
    int grid = (n + 255) / 256;
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&gemv::gemv_epilogue_kernel), dim3(grid), dim3(256),
                                   args, 0, static_cast<hipStream_t>(hip_stream));
    return gemv::finish(e);
}

int gemv_last_hip_error(void) { return gemv::last_hip_error(); }

} // extern "C"

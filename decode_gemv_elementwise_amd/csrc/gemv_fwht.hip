// The signed Hadamard transform of "vulkan: fuse the sign multiply into the
// Hadamard FWHT" (Overview): the sign multiply folded into the transform's
// load, one dispatch (gemv_fwht_signed); and the same transform as a prologue
// inside the GEMV's staging of x, so that epilogue(W . FWHT(x * s)) is one
// launch (gemv_fused_fwht).  The transform is done a 1024-value tile per wave
// (FwhtTile in gemv_fast.h); both entry points use that same code, so the
// fused result is bit for bit gemv_fwht_signed followed by gemv_fused.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "gemv_fast.h"

namespace gemv {
namespace {

constexpr int kFwhtWaves = 4;

// One wave per (row, tile); the output of each lane's 16 values goes back to
// the same places, so dst may be x itself.
__global__ __launch_bounds__(kFwhtWaves *kWave) void gemv_fwht_kernel(const float *x, FwhtArgs f, int nrows, int K,
                                                                      float *dst)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int ntiles = (K + kFwhtTile - 1) / kFwhtTile;
    const int job = blockIdx.x * kFwhtWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (job >= nrows * ntiles)
        return;
    const int row = job / ntiles, t = job % ntiles;
    const float *xr = x + (int64_t)row * K;
    float *dr = dst + (int64_t)row * K;
    const bool vec = (K % 4 == 0) && ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
    FwhtTile ft;
    ft.load(xr, f, K, t, lane, vec);
    ft.transform(f, lane);
    const int k0 = t * kFwhtTile + 16 * lane;
    if (vec) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (k0 + 4 * q < K)
                *reinterpret_cast<f32x4 *>(dr + k0 + 4 * q) =
                    f32x4{ft.v[4 * q], ft.v[4 * q + 1], ft.v[4 * q + 2], ft.v[4 * q + 3]};
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (k0 + j < K)
                dr[k0 + j] = ft.v[j];
    }
}

FwhtArgs fwht_args(const float *signs, int64_t n, int64_t nsigns)
{
    return FwhtArgs{signs, (int)n, (int)nsigns, (float)(1.0 / std::sqrt((double)n))};
}

} // namespace
} // namespace gemv

extern "C" {

int gemv_fwht_signed(const float *x, const float *signs, int64_t nrows, int64_t K, int64_t n, int64_t nsigns,
                     float *dst, void *hip_stream)
{
    int st = gemv::validate_fwht(x, signs, nrows, K, n, nsigns, dst);
    if (st != GEMV_OK)
        return st;
    const int64_t jobs = nrows * ((K + gemv::kFwhtTile - 1) / gemv::kFwhtTile);
    const int grid = (int)((jobs + gemv::kFwhtWaves - 1) / gemv::kFwhtWaves);
    gemv::FwhtArgs f = gemv::fwht_args(signs, n, nsigns);
    int nr = (int)nrows, k = (int)K;
    void *args[] = {&x, &f, &nr, &k, &dst};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&gemv::gemv_fwht_kernel), dim3(grid),
                                   dim3(gemv::kFwhtWaves * gemv::kWave), args, 0, static_cast<hipStream_t>(hip_stream));
    return gemv::finish_launch((int)e);
}

int gemv_fused_fwht(const void *W, int wfmt, int64_t N, int64_t K, const float *x, const float *signs, int64_t n,
                    int64_t nsigns, int act, const gemv_view *mul_operand, const gemv_view *add_operand,
                    const gemv_view *dst, void *hip_stream)
{
    int st = gemv::validate_fused_fwht(W, wfmt, N, K, x, signs, n, nsigns, act, mul_operand, add_operand, dst);
    if (st != GEMV_OK)
        return st;
    gemv::Call c{static_cast<const unsigned char *>(W), nullptr, x, (int)N, (int)K, act,
                 mul_operand ? mul_operand->data : nullptr, add_operand ? add_operand->data : nullptr, dst->data,
                 gemv::fwht_args(signs, n, nsigns)};
    return gemv::finish_launch(
        (int)gemv::dispatch_any<false, true>(wfmt, c, static_cast<hipStream_t>(hip_stream)));
}

} // extern "C"

// The one-column kernels of the fused-epilogue decode GEMV for CDNA4 (gfx950):
// dst = epilogue(W x), one output column, one launch per call, optionally
// after a signed Hadamard transform of x.  Included by the translation units
// that instantiate them.
//
// What is computed follows "feat(cuda): fuse activations and residual add
// into mmv f/q epilogues" ("Summary", "What changed"): the matrix-vector
// product of the decode path with a run-time epilogue (none, sigmoid, silu,
// silu times a per-row operand, a residual add, possibly through a reshape of
// the output) applied to the accumulator before the one store; and "ggml-cpu:
// fuse element-wise epilogues (ADD, MUL, SILU) into
// ggml_compute_forward_mul_mat" ("What") for the plain multiply tail.  The
// kernel design is this library's own, for gfx950:
//
//  * x is staged once per workgroup into LDS, as f32, laid out in 16-byte
//    W-chunk order with 4 floats of padding after every chunk of 8+ floats,
//    so that the 16-byte LDS reads of consecutive lanes (consecutive chunks)
//    fall in distinct banks.
//  * Each wave streams R rows at a time: lane l loads 16-byte chunks
//    l, l + 64, ... of each row with nontemporal 128-bit loads (a wave's load
//    instruction covers 1 KiB of one row), reads the matching x values from
//    LDS once and uses them for all R rows.
//  * Register-level dequantisation: f16 and 4-bit codes become packed f16
//    pairs consumed by mixed-precision FMAs (f16 x f32 + f32); bf16 is a
//    shift; 8-bit codes a sign-extending convert.  All products are formed
//    exactly inside the FMA; only the f32 sums round.
//  * The 64 lane partials of a row are reduced with DPP row operations and
//    four lane reads, in a fixed order: results are deterministic.
//  * The epilogue is a run-time switch on a uniform value, applied by one lane
//    per row; the same __device__ function serves the unfused pass, so fused
//    and unfused results are identical for the same accumulator.
//
// No MFMA: one column is not a dense contraction, and the kernel is bound by
// HBM bandwidth (<= 4 flops per weight byte).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "gemv_device.h"
#include "gemv_internal.h"

namespace gemv {
namespace {

// ------------------------------------------------------------------ fast kernel
// Requires: W 16-byte aligned, row_bytes(K) % 16 == 0, (K / E) * XS * 4 bytes
// of LDS.  One tile of WAVES * R rows per workgroup; wave w owns rows
// tile*WAVES*R + w*R + [0, R).
//
// Lane l owns the 16-byte chunks l, l + 64, ... of each of its rows
// (cpl = ceil(nchunks / 64) of them), fetched in batches of U chunks per row,
// all loads of a batch issued before any is used; with more than one batch
// the next is issued before the current one is consumed.
//
// No load sits behind a branch.  Chunks past the end of a row (a ragged last
// batch) and rows past N are clamped to valid addresses and their
// contributions discarded by a select; a branch around a load would make the
// compiler wait for every outstanding load at the join.  Loads are issued in
// the order they are needed (epilogue operand, x, then W), because the
// hardware's load counter retires in order: waiting for x then does not wait
// for W, and the barrier after staging waits only for LDS.


template <int FMT, int R, int U>
__device__ __forceinline__ void consume_batch(const Batch<FMT, R, U> &b, const float *xs, float *acc, int lane,
                                              int jb, int nchunks)
{
    using F = Fmt<FMT>;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int craw = lane + kWave * (jb + u);
        const bool valid = craw < nchunks;
        const unsigned c = (unsigned)min(craw, nchunks - 1);
        float xv[F::E];
        const f32x4 *xl = reinterpret_cast<const f32x4 *>(xs + c * F::XS);
#pragma unroll
        for (int i = 0; i < F::E / 4; ++i) {
            f32x4 t = xl[i];
            xv[4 * i] = t.x;
            xv[4 * i + 1] = t.y;
            xv[4 * i + 2] = t.z;
            xv[4 * i + 3] = t.w;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float t;
            if constexpr (F::kBlock)
                t = F::dot(b.q[r][u], xv, b.sc[r][u], acc[r]);
            else
                t = F::dot(b.q[r][u], xv, acc[r]);
            acc[r] = valid ? t : acc[r];
        }
    }
}

// x staging into LDS, in padded chunk order: a pass loads S float4 per thread
// (indices clamped to the last float4; the duplicate writes that clamping
// causes store the same value) and then writes them.  When a row is one batch
// (U chunks per lane), K <= 64 * U * E, so S = ceil(E * U / (4 * WAVES)) loads
// per thread cover x in one pass; longer rows take passes of 8.
template <int FMT, int WAVES, int U, bool MULTI> constexpr int stage_loads()
{
    return MULTI ? 8 : (Fmt<FMT>::E * U + 4 * WAVES - 1) / (4 * WAVES);
}

template <int FMT, int kStage> struct XStage {
    f32x4 v[kStage];
    __device__ __forceinline__ void load(const float *x, int K, int base, bool aligned16)
    {
        const int nt = blockDim.x;
        if (aligned16) {
            const int n4 = K / 4;
            const f32x4 *x4 = reinterpret_cast<const f32x4 *>(x);
#pragma unroll
            for (int j = 0; j < kStage; ++j)
                v[j] = x4[min(base + j * nt + (int)threadIdx.x, n4 - 1)];
        } else {
#pragma unroll
            for (int j = 0; j < kStage; ++j) {
                const int k = 4 * min(base + j * nt + (int)threadIdx.x, K / 4 - 1);
                v[j] = f32x4{x[k], x[k + 1], x[k + 2], x[k + 3]};
            }
        }
    }
    __device__ __forceinline__ void store(float *xs, int K, int base) const
    {
        using F = Fmt<FMT>;
        const int nt = blockDim.x;
#pragma unroll
        for (int j = 0; j < kStage; ++j) {
            // non-negative: unsigned division by the power-of-two E is a shift
            const unsigned k = 4u * (unsigned)min(base + j * nt + (int)threadIdx.x, K / 4 - 1);
            *reinterpret_cast<f32x4 *>(xs + (k / F::E) * F::XS + (k % F::E)) = v[j];
        }
    }
};



// ------------------------------------------------------------------ signed Hadamard prologue
// "vulkan: fuse the sign multiply into the Hadamard FWHT", Overview: x is
// multiplied by a sign vector (element k by s[k mod nsigns]) and every block
// of n values is transformed by the Hadamard matrix (Sylvester order, scaled
// by 1/sqrt(n)); the signs are applied as the row is loaded.  A wave takes a
// tile of 1024 values, lane l holding elements 16 l .. 16 l + 15: butterflies
// of span 1..8 stay in a lane, spans 16..512 pair lane l with lane l ^ (span
// / 16) through a lane shuffle.  Blocks never straddle tiles (n <= 1024
// divides K, and tiles start at multiples of 1024).

struct FwhtArgs {
    const float *signs;
    int n;       // block length: a power of two, 1..1024
    int nsigns;  // sign period: divides K
    float scale; // 1/sqrt(n), rounded to f32
};

constexpr int kFwhtTile = 1024;

struct FwhtTile {
    float v[16];

    template <int M> __device__ static __forceinline__ float partner(float x, int lane)
    {
        const int xi = __builtin_bit_cast(int, x);
        int p;
        if constexpr (M == 1) {
            p = __builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xF, 0xF, false); // quad_perm [1,0,3,2]
        } else if constexpr (M == 2) {
            p = __builtin_amdgcn_update_dpp(0, xi, 0x4E, 0xF, 0xF, false); // quad_perm [2,3,0,1]
        } else if constexpr (M == 4) {
            p = __builtin_amdgcn_update_dpp(0, xi, 0x12C, 0xF, 0x5, false); // row_ror:12 -> lane + 4
            p = __builtin_amdgcn_update_dpp(p, xi, 0x124, 0xF, 0xA, false); // row_ror:4 -> lane - 4
        } else if constexpr (M == 8) {
            p = __builtin_amdgcn_update_dpp(0, xi, 0x128, 0xF, 0xF, false); // row_ror:8
        } else if constexpr (M == 16) {
            const auto r = __builtin_amdgcn_permlane16_swap((unsigned)xi, (unsigned)xi, false, false);
            p = (int)((lane & 16) ? r[0] : r[1]);
        } else {
            const auto r = __builtin_amdgcn_permlane32_swap((unsigned)xi, (unsigned)xi, false, false);
            p = (int)((lane & 32) ? r[0] : r[1]);
        }
        return __builtin_bit_cast(float, p);
    }

    template <int M> __device__ __forceinline__ void lane_stage(int lane)
    {
        const float sgn = (lane & M) ? -1.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            v[j] = fmaf(sgn, v[j], partner<M>(v[j], lane));
    }

    // Loads tile t of a K-row (x + row offset) times its signs; elements past
    // K read a clamped, valid address and become 0.  Branch-free.  vec: K is a
    // multiple of 4 and x is 16-byte aligned.
    __device__ __forceinline__ void load(const float *x, const FwhtArgs &f, int K, int t, int lane, bool vec)
    {
        const int k0 = t * kFwhtTile + 16 * lane;
        if (vec) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = k0 + 4 * q;
                const f32x4 a = *reinterpret_cast<const f32x4 *>(x + min(k, K - 4));
                const bool ok = k < K;
                v[4 * q] = ok ? a.x : 0.0f;
                v[4 * q + 1] = ok ? a.y : 0.0f;
                v[4 * q + 2] = ok ? a.z : 0.0f;
                v[4 * q + 3] = ok ? a.w : 0.0f;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int k = k0 + j;
                const float a = x[min(k, K - 1)];
                v[j] = k < K ? a : 0.0f;
            }
        }
        if (f.nsigns % 16 == 0 && (reinterpret_cast<uintptr_t>(f.signs) & 15) == 0) {
            // The lane's 16 signs are contiguous and 16-byte aligned.  nsigns
            // divides K here, so K is a multiple of 16 and so is every tile
            // start k0: a lane inside the row starts at k0 <= K - 16, and a
            // lane past the end (whose values are zero) is clamped to K - 16,
            // so that s0 + 15 < nsigns for every lane.
            const int s0 = min(k0, K - 16) % f.nsigns;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 sg = *reinterpret_cast<const f32x4 *>(f.signs + s0 + 4 * q);
                v[4 * q] *= sg.x;
                v[4 * q + 1] *= sg.y;
                v[4 * q + 2] *= sg.z;
                v[4 * q + 3] *= sg.w;
            }
        } else {
            int si = min(k0, K - 1) % f.nsigns;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                v[j] *= f.signs[si];
                si = si + 1 == f.nsigns ? 0 : si + 1;
            }
        }
    }

    // Butterflies of every span below n, then the scale.  A lane-crossing
    // butterfly takes its partner's value p and forms p + v (lower lane) or
    // p - v (upper lane) as one fma(+-1, v, p), rounded once like the plain
    // sum or difference.  Partners: lane ^ 1 and ^ 2 by DPP quad
    // permutations, ^ 4 by DPP row rotations by 12 (lower lanes, banks 0 and
    // 2 of each row) and by 4 (upper lanes, banks 1 and 3), ^ 8 by a row
    // rotation by 8, ^ 16 and ^ 32 by the permlane swaps.
    __device__ __forceinline__ void transform(const FwhtArgs &f, int lane)
    {
#pragma unroll
        for (int h = 1; h < 16; h <<= 1) {
            if (h < f.n) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    if (!(j & h)) {
                        const float a = v[j], b = v[j + h];
                        v[j] = a + b;
                        v[j + h] = a - b;
                    }
                }
            }
        }
        if (16 < f.n)
            lane_stage<1>(lane);
        if (32 < f.n)
            lane_stage<2>(lane);
        if (64 < f.n)
            lane_stage<4>(lane);
        if (128 < f.n)
            lane_stage<8>(lane);
        if (256 < f.n)
            lane_stage<16>(lane);
        if (512 < f.n)
            lane_stage<32>(lane);
#pragma unroll
        for (int j = 0; j < 16; ++j)
            v[j] *= f.scale;
    }
};

template <int FMT, int WAVES, int R, int U, bool MULTI, bool GLU, bool FWHT = false>
__global__ __launch_bounds__(WAVES *kWave, 1) void gemv_fast_kernel(const unsigned char *__restrict__ W,
                                                                 const unsigned char *__restrict__ W2,
                                                                 const float *__restrict__ x, int N, int K,
                                                                 int act, const float *mop, const float *rop,
                                                                 float *dst, FwhtArgs pro)
{
    constexpr int RR = GLU ? 2 * R : R; // rows loaded per wave
    using F = Fmt<FMT>;
    extern __shared__ f32x4 lds4[];
    float *xs = reinterpret_cast<float *>(lds4);

    const int lane = threadIdx.x & (kWave - 1);
    // uniform across the wave: row addresses are then computed on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nchunks = K / F::E;
    const int cpl = (nchunks + kWave - 1) / kWave;
    const int nb = (cpl + U - 1) / U;
    const int row0 = (blockIdx.x * WAVES + wave) * R;
    const int64_t rbytes = row_bytes<FMT>(K);
    const unsigned char *scales = F::kBlock ? W + align256_dev((int64_t)N * rbytes) : nullptr;
    const unsigned char *scales2 = (F::kBlock && GLU) ? W2 + align256_dev((int64_t)N * rbytes) : nullptr;
    const int64_t sbytes = (int64_t)(K / 32) * 2;

    // 1. epilogue operand of the row this lane stores (lane r stores row0 + r;
    //    other lanes and rows past N read a clamped, valid element)
    const bool has_op = act == GEMV_ACT_SILU_MUL || act == GEMV_ACT_MUL || act == GEMV_ACT_ADD;
    const float *opp = act == GEMV_ACT_ADD ? rop : (has_op ? mop : x);
    const int oplim = has_op ? N - 1 : K - 1;
    const float opv = opp[min(row0 + min(lane, R - 1), oplim)];

    // 2. x (first staging pass; with the prologue, this wave's first tile)
    const bool x16 = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
    constexpr int S = FWHT ? 1 : stage_loads<FMT, WAVES, U, MULTI>();
    XStage<FMT, S> st;
    FwhtTile ft;
    const int ntiles = (K + kFwhtTile - 1) / kFwhtTile;
    if constexpr (FWHT)
        ft.load(x, pro, K, min(wave, ntiles - 1), lane, x16);
    else
        st.load(x, K, 0, x16);

    // 3. W, first batch
    const unsigned char *wrow[RR];
    const unsigned char *srow[RR];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, N - 1);
        wrow[r] = W + (int64_t)row * rbytes;
        srow[r] = F::kBlock ? scales + (int64_t)row * sbytes : nullptr;
        if constexpr (GLU) {
            wrow[R + r] = W2 + (int64_t)row * rbytes;
            srow[R + r] = F::kBlock ? scales2 + (int64_t)row * sbytes : nullptr;
        }
    }
    Batch<FMT, RR, U> b0;
    issue_batch<FMT, RR, U>(b0, wrow, srow, lane, 0, nchunks);
    // keep the W loads ahead of the staging stores (the scheduler may otherwise
    // sink them below the wait for x, serialising the two round trips)
    __builtin_amdgcn_sched_barrier(0);

    // 4. finish staging
    if constexpr (FWHT) {
        // transformed tiles go to LDS in the padded chunk layout (K is a
        // multiple of 4, so each float4 lies inside one chunk)
        for (int t = wave; t < ntiles; t += WAVES) {
            if (t != wave)
                ft.load(x, pro, K, t, lane, x16);
            ft.transform(pro, lane);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = t * kFwhtTile + 16 * lane + 4 * q;
                if (k < K)
                    *reinterpret_cast<f32x4 *>(xs + (k / F::E) * F::XS + (k % F::E)) =
                        f32x4{ft.v[4 * q], ft.v[4 * q + 1], ft.v[4 * q + 2], ft.v[4 * q + 3]};
            }
        }
    } else {
        st.store(xs, K, 0);
        for (int base = S * (int)blockDim.x; base < K / 4; base += S * (int)blockDim.x) {
            st.load(x, K, base, x16);
            st.store(xs, K, base);
        }
    }
    lds_barrier();

    // 5. stream the rows
    float acc[RR];
#pragma unroll
    for (int r = 0; r < RR; ++r)
        acc[r] = 0.0f;
    if constexpr (!MULTI) {
        consume_batch<FMT, RR, U>(b0, xs, acc, lane, 0, nchunks);
    } else {
        // several batches per row: double-buffered
        Batch<FMT, RR, U> b1;
        int i = 0;
        for (; i + 2 < nb; i += 2) {
            issue_batch<FMT, RR, U>(b1, wrow, srow, lane, (i + 1) * U, nchunks);
            consume_batch<FMT, RR, U>(b0, xs, acc, lane, i * U, nchunks);
            issue_batch<FMT, RR, U>(b0, wrow, srow, lane, (i + 2) * U, nchunks);
            consume_batch<FMT, RR, U>(b1, xs, acc, lane, (i + 1) * U, nchunks);
        }
        if (nb - i == 2) {
            issue_batch<FMT, RR, U>(b1, wrow, srow, lane, (i + 1) * U, nchunks);
            consume_batch<FMT, RR, U>(b0, xs, acc, lane, i * U, nchunks);
            consume_batch<FMT, RR, U>(b1, xs, acc, lane, (i + 1) * U, nchunks);
        } else {
            consume_batch<FMT, RR, U>(b0, xs, acc, lane, i * U, nchunks);
        }
    }

    // 6. reduce each row; lane r takes row r's sum, one epilogue for all rows
    float mine = 0.0f, mine2 = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float s = wave_sum(acc[r]);
        mine = lane == r ? s : mine;
        if constexpr (GLU) {
            const float s2 = wave_sum(acc[R + r]);
            mine2 = lane == r ? s2 : mine2;
        }
    }
    float y;
    if constexpr (GLU)
        y = apply_glu(act, mine, mine2);
    else
        y = apply_epilogue(act, mine, opv);
    if (lane < R && row0 + lane < N)
        dst[row0 + lane] = y;
}

// ------------------------------------------------------------------ generic kernel
// Any K and alignment (float formats with K not a multiple of the 16-byte
// chunk, or x too long for LDS): one wave per row, element loads, x read
// through the caches.

template <int FMT> __device__ __forceinline__ float weight_at(const unsigned char *W, int N, int K, int row, int k)
{
    if constexpr (FMT == GEMV_W_F32) {
        return reinterpret_cast<const float *>(W)[(int64_t)row * K + k];
    } else if constexpr (FMT == GEMV_W_F16) {
        return (float)reinterpret_cast<const _Float16 *>(W)[(int64_t)row * K + k];
    } else if constexpr (FMT == GEMV_W_BF16) {
        unsigned short b = reinterpret_cast<const unsigned short *>(W)[(int64_t)row * K + k];
        return __builtin_bit_cast(float, (unsigned)b << 16);
    } else if constexpr (FMT == GEMV_W_Q8B32) {
        const unsigned char *scales = W + align256_dev((int64_t)N * K);
        float s = load_scale(scales + ((int64_t)row * (K / 32) + k / 32) * 2);
        return (float)(int)(signed char)W[(int64_t)row * K + k] * s;
    } else {
        const unsigned char *scales = W + align256_dev((int64_t)N * K / 2);
        float s = load_scale(scales + ((int64_t)row * (K / 32) + k / 32) * 2);
        unsigned char b = W[(int64_t)row * (K / 2) + k / 2];
        int c = (k & 1) ? (b >> 4) : (b & 0xF);
        return (float)(c - 8) * s;
    }
}

template <int FMT, bool GLU>
__global__ __launch_bounds__(256) void gemv_generic_kernel(const unsigned char *__restrict__ W,
                                                           const unsigned char *__restrict__ W2,
                                                           const float *__restrict__ x, int N, int K, int act,
                                                           const float *mop, const float *rop, float *dst)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int nwaves = gridDim.x * (blockDim.x / kWave);
    for (int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; row < N; row += nwaves) {
        float acc = 0.0f, acc2 = 0.0f;
        for (int k = lane; k < K; k += kWave) {
            acc = fmaf(weight_at<FMT>(W, N, K, row, k), x[k], acc);
            if constexpr (GLU)
                acc2 = fmaf(weight_at<FMT>(W2, N, K, row, k), x[k], acc2);
        }
        const float s = wave_sum(acc);
        float y;
        if constexpr (GLU)
            y = apply_glu(act, s, wave_sum(acc2));
        else
            y = apply_epilogue(act, s, operand_of(act, mop, rop, row));
        if (lane == 0)
            dst[row] = y;
    }
}

// ------------------------------------------------------------------ unfused epilogue

__global__ __launch_bounds__(256) void gemv_epilogue_kernel(int N, const float *acc, int act, const float *mop,
                                                            const float *rop, float *dst)
{
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < N)
        dst[i] = apply_epilogue(act, acc[i], operand_of(act, mop, rop, i));
}

// ------------------------------------------------------------------ host dispatch

struct Call {
    const unsigned char *W;
    const unsigned char *W2; // up matrix of a gated pair, else nullptr
    const float *x;
    int N, K, act;
    const float *m, *r;
    float *dst;
    FwhtArgs pro; // the signed Hadamard prologue (FWHT kernels only)
};

template <int FMT> constexpr int lds_bytes_fast(int K) { return (K / Fmt<FMT>::E) * Fmt<FMT>::XS * 4; }

template <int FMT, int WAVES, int R, int U, bool MULTI, bool GLU, bool FWHT = false>
hipError_t launch_fast(const Call &c, hipStream_t s)
{
    const void *fn = reinterpret_cast<const void *>(&gemv_fast_kernel<FMT, WAVES, R, U, MULTI, GLU, FWHT>);
    size_t lds = (size_t)lds_bytes_fast<FMT>(c.K);
    if (lds > 64 * 1024) {
        static std::once_flag once;
        static hipError_t attr_err = hipSuccess;
        std::call_once(once, [&] { attr_err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds); });
        if (attr_err != hipSuccess)
            return attr_err;
    }
    const int rows_per_tile = WAVES * R;
    const int grid = (c.N + rows_per_tile - 1) / rows_per_tile;
    const unsigned char *W = c.W, *W2 = c.W2;
    const float *x = c.x;
    int N = c.N, K = c.K, act = c.act;
    const float *m = c.m, *r = c.r;
    float *dst = c.dst;
    FwhtArgs pro = c.pro;
    void *args[] = {&W, &W2, &x, &N, &K, &act, &m, &r, &dst, &pro};
    return hipLaunchKernel(fn, dim3(grid), dim3(WAVES * kWave), args, lds, s);
}

template <int FMT, bool GLU> hipError_t launch_generic(const Call &c, hipStream_t s)
{
    const void *fn = reinterpret_cast<const void *>(&gemv_generic_kernel<FMT, GLU>);
    int grid = (c.N + 3) / 4;
    if (grid > 65536)
        grid = 65536;
    const unsigned char *W = c.W, *W2 = c.W2;
    const float *x = c.x;
    int N = c.N, K = c.K, act = c.act;
    const float *m = c.m, *r = c.r;
    float *dst = c.dst;
    void *args[] = {&W, &W2, &x, &N, &K, &act, &m, &r, &dst};
    return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, s);
}

// Waves per workgroup: float formats favour smaller workgroups (more of them
// resident per CU), block formats larger ones (fewer copies of x staged).
template <int FMT> constexpr int waves_of() { return Fmt<FMT>::kBlock ? 8 : 4; }
constexpr int kLoadsPerLane = 8; // R * U target
// Below this many row tiles a launch takes one row per wave, so that more
// CUs take part.
constexpr int kMinTiles = 512;

// Rows per wave for a batch of U chunk loads per row: about kLoadsPerLane
// loads of 16 bytes per lane in flight.  A row longer than one batch (more
// than 8 chunks per lane) is streamed one row per wave, double-buffered.
// A gated pair loads two rows (gate and up) per output row, so it takes half
// as many output rows per wave.
template <int FMT, int kWaves, int U, bool GLU, bool FWHT> hipError_t launch_uw(const Call &c, hipStream_t s, bool multi)
{
    constexpr int R1 = U >= kLoadsPerLane ? 1 : (2 * U > kLoadsPerLane ? 1 : (4 * U > kLoadsPerLane ? 2 : (8 * U > kLoadsPerLane ? 4 : 8)));
    constexpr int R0 = GLU ? (R1 > 1 ? R1 / 2 : 1) : R1;
    // Every workgroup transforms all of x itself, so with the Hadamard
    // prologue a workgroup takes at least 16 rows to spread that work thin.
    constexpr int kFwhtRows = (16 + kWaves - 1) / kWaves;
    constexpr int R = FWHT && R0 < kFwhtRows ? kFwhtRows : R0;
    if constexpr (U >= 5) {
        if (multi)
            return launch_fast<FMT, kWaves, FWHT ? 2 : 1, U, true, GLU, FWHT>(c, s);
    }
    // Few tiles: one row per wave so that more CUs take part.
    const int64_t tiles = ((int64_t)c.N + kWaves * R - 1) / (kWaves * R);
    if (!FWHT && R > 1 && tiles < kMinTiles)
        return launch_fast<FMT, kWaves, 1, U, false, GLU, FWHT>(c, s);
    return launch_fast<FMT, kWaves, R, U, false, GLU, FWHT>(c, s);
}

// Waves per workgroup for the float formats' one-column calls, from the
// shape (measured on MI355X across N = 32..28672, K = 4096..14336): long rows
// stream best with 16 waves from three batches per row up (one workgroup per
// CU by LDS) and with 8 at two batches, as long as every CU still gets a
// workgroup; one batch per row
// and rows that fill exactly one 16-wave workgroup per CU take 16 waves (one
// copy of x staged per CU); everything else keeps the 4-wave tiles, whose
// finer grain balances the many-workgroup shapes.  The choice depends only on
// (format, N, K), so the reduction order of a row (one wave, lanes over its
// chunks) is the same whatever it picks.
template <int FMT, int U, bool GLU, bool FWHT = false> hipError_t launch_u(const Call &c, hipStream_t s, bool multi)
{
    if constexpr (!Fmt<FMT>::kBlock && !GLU) {
        const int64_t cus = device_cus();
        if (multi && U >= 5) {
            const int cpl = (c.K / Fmt<FMT>::E + kWave - 1) / kWave;
            const int nbatch = (cpl + 7) / 8;
            // with the prologue a long-row wave takes 2 rows: 8 waves keep the
            // 16-row workgroups that spread the transform
            if (!FWHT && nbatch >= 3 && (c.N + 15) / 16 >= cus)
                return launch_uw<FMT, 16, U, GLU, FWHT>(c, s, multi);
            if ((c.N + (FWHT ? 15 : 7)) / (FWHT ? 16 : 8) >= cus)
                return launch_uw<FMT, 8, U, GLU, FWHT>(c, s, multi);
        } else if (!multi && U >= kLoadsPerLane && (c.N + 15) / 16 == cus) {
            return launch_uw<FMT, 16, U, GLU, FWHT>(c, s, multi);
        }
    }
    return launch_uw<FMT, waves_of<FMT>(), U, GLU, FWHT>(c, s, multi);
}

// The path depends only on (format, N, K), never on the epilogue, so a fused
// call and its unfused composition reduce in the same order.  The Hadamard
// prologue exists only on the chunked path (its callers check for it).
template <int FMT, bool GLU, bool FWHT = false> hipError_t dispatch(const Call &c, hipStream_t s)
{
    const bool fast = (row_bytes<FMT>(c.K) % 16 == 0) && lds_bytes_fast<FMT>(c.K) <= kMaxLds;
    if (!fast) {
        if constexpr (FWHT)
            return hipErrorInvalidValue;
        else
            return launch_generic<FMT, GLU>(c, s);
    }
    const int nchunks = c.K / Fmt<FMT>::E;
    const int cpl = (nchunks + kWave - 1) / kWave;
    const int nbatch = (cpl + 7) / 8;
    const int u = (cpl + nbatch - 1) / nbatch; // 1..8, batches of equal size
    switch (u) {
    case 1:
        return launch_u<FMT, 1, GLU, FWHT>(c, s, nbatch > 1);
    case 2:
        return launch_u<FMT, 2, GLU, FWHT>(c, s, nbatch > 1);
    case 3:
        return launch_u<FMT, 3, GLU, FWHT>(c, s, nbatch > 1);
    case 4:
        return launch_u<FMT, 4, GLU, FWHT>(c, s, nbatch > 1);
    case 5:
        return launch_u<FMT, 5, GLU, FWHT>(c, s, nbatch > 1);
    case 6:
        return launch_u<FMT, 6, GLU, FWHT>(c, s, nbatch > 1);
    case 7:
        return launch_u<FMT, 7, GLU, FWHT>(c, s, nbatch > 1);
    default:
        return launch_u<FMT, 8, GLU, FWHT>(c, s, nbatch > 1);
    }
}

template <bool GLU, bool FWHT = false> hipError_t dispatch_any(int wfmt, const Call &c, hipStream_t s)
{
    switch (wfmt) {
    case GEMV_W_F32:
        return dispatch<GEMV_W_F32, GLU, FWHT>(c, s);
    case GEMV_W_F16:
        return dispatch<GEMV_W_F16, GLU, FWHT>(c, s);
    case GEMV_W_BF16:
        return dispatch<GEMV_W_BF16, GLU, FWHT>(c, s);
    case GEMV_W_Q8B32:
        return dispatch<GEMV_W_Q8B32, GLU, FWHT>(c, s);
    default:
        return dispatch<GEMV_W_Q4B32, GLU, FWHT>(c, s);
    }
}

int finish(hipError_t e) { return finish_launch((int)e); }

} // namespace
} // namespace gemv

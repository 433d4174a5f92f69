// Several destination columns over one weight matrix (ncols = 2..8):
// dst[b*N + i] = epilogue((W x_b)_i, operand[b*N + i]).
//
// "feat(cuda): fuse activations and residual add into mmv f/q epilogues",
// Summary, states the fused matrix-vector path for one destination column;
// with a handful of columns (small-batch or speculative decode) W is still
// the only large operand, so the kernel streams it from HBM once and applies
// every chunk to all columns.  Each 16-byte chunk is decoded once into
// registers and then multiplied into the ncols running sums of its row; as
// ncols grows the work per weight byte grows with it, and the kernel moves
// from the HBM roof towards the VALU roof.
//
// Layout of the work, per workgroup of kWaves waves and a tile of kWaves * R
// rows (wave w owns rows tile*kWaves*R + w*R + [0, R)); where a row fits one
// segment and x of every column fits LDS, a "one-shot" variant stages x once
// and issues every chunk of the wave's rows up front (see dispatch_cols):
//  * K is walked in segments of 64 * U chunks.  A segment of x, for all
//    columns, is copied global -> LDS with direct-to-LDS loads into one of
//    two buffers (ncols planes of 64 * U * E floats each): the next
//    segment's copy and W batch (R rows x U chunks per lane) are in flight
//    while the current segment is consumed.
//  * Lane l owns chunks l, l + 64, ... of each row, in the same order as the
//    one-column kernel, and the row sums are reduced with the same wave
//    reduction: column b of the result is bit for bit the one-column result.
//  * LDS holds each plane without padding; the 16-byte pieces of a chunk are
//    permuted by an XOR of the chunk index so that the 16-byte reads of 8 (or
//    16) consecutive lanes fall in distinct bank groups.
//  * Lane j < R * ncols finishes output (row R-block j % R, column j / R):
//    consecutive lanes store consecutive rows of one column.
//  * The one-shot form runs on a resident grid (gemv_cols_tiles_kernel): a
//    workgroup stages x once and walks row tiles, so no tile waits for a
//    fresh copy of x before issuing its W.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "gemv_device.h"
#include "gemv_internal.h"

namespace gemv {
namespace {

// Launch shape (measured on MI355X, see the ColsCfg comments): 4-wave
// workgroups for the segmented form; an x-staging budget of 64 values per
// lane per segment and about 8 chunk loads per lane per batch; 8-wave
// workgroups for the one-shot form, 2 output rows per wave for plain columns
// and 1 for the gated pair (which loads a gate and an up row per output row).
constexpr int kColsWaves = 4;
constexpr int kColsXBudget = 64;
constexpr int kColsLoads = 8;
constexpr int kColsOneShotWaves = 8;
constexpr int kColsOneShotRows = 2;
constexpr int kColsOneShotGluWaves = 8;
constexpr int kColsOneShotGluRows = 1;

// UO == 0: segments of kColsXBudget / (NC * E) chunks per lane.
// UO > 0: a whole row in one segment of UO chunks per lane ("one-shot": x of
// every column staged once, every W chunk of the wave's rows issued at once),
// used when that fits LDS; 8 waves of 2 rows (16 rows per workgroup) keep
// 2 * UO loads per lane in flight.
template <int FMT, int NC, int UO = 0, bool GLU = false> struct ColsCfg {
    static constexpr int E = Fmt<FMT>::E;
    static constexpr int kWaves = UO > 0 ? (GLU ? kColsOneShotGluWaves : kColsOneShotWaves) : kColsWaves;
    // chunks per lane per segment: kColsXBudget / (NC * E), 1..8 (a
    // short segment keeps the LDS per workgroup small and occupancy up)
    static constexpr int kU0 = kColsXBudget / (NC * E);
    static constexpr int U = UO > 0 ? UO : (kU0 < 1 ? 1 : (kU0 > 8 ? 8 : kU0));
    // rows per wave: about kColsLoads chunk loads per lane per batch, 1..4
    // (a gated pair loads a gate and an up row per output row: half as many)
    static constexpr int kR0 = kColsLoads / U;
    static constexpr int kR1 = UO > 0 ? kColsOneShotRows : (kR0 > 4 ? 4 : (kR0 < 1 ? 1 : kR0));
    static constexpr int R = GLU ? (UO > 0 ? kColsOneShotGluRows : (kR1 > 1 ? kR1 / 2 : 1)) : kR1;
    static constexpr int SEG = 64 * U * E;     // x floats per column per segment
    static constexpr int kPlane4 = SEG / 4;    // float4 slots per plane (a multiple of 64)
    static constexpr int kBuf4 = NC * kPlane4; // float4 slots per segment buffer
    static constexpr int kCopies = kBuf4 / kWave;                // 64-slot wave copies per segment
    static constexpr int kDma = (kCopies + kWaves - 1) / kWaves; // copies per wave (the last may be idle)
    static_assert(R * NC <= kWave, "a wave's outputs are finished one per lane");
    static_assert(kWaves * kWave <= 1024, "at most 1024 threads per workgroup");
};

// Copies segment seg of x (all columns) from global memory straight into an
// LDS buffer (global_load_lds): a wave's 16-byte copy fills 64 consecutive
// float4 slots, lane i slot p0 + i, so lane i fetches the float4 whose
// swizzled slot is p0 + i (the swizzle is its own inverse).  When x is not
// 16-byte aligned the same slots are filled by 4-byte copies, 16 slots per
// instruction.  Elements past K fetch a clamped, valid address; those slots
// belong to chunks past the end of the row and are never used.
template <int FMT, int NC, int UO, bool GLU>
__device__ __forceinline__ void dma_x_segment(f32x4 *buf, const float *x, int K, int seg, int wave, int lane,
                                              bool aligned16)
{
    using C = ColsCfg<FMT, NC, UO, GLU>; // the kernel's own wave count splits the copies
    const int k4 = K / 4; // K is a multiple of 4 on this path
    if (aligned16) {
#pragma unroll
        for (int j = 0; j < C::kDma; ++j) {
            const int copy = wave + C::kWaves * j; // wave-uniform
            if (C::kCopies % C::kWaves != 0 && copy >= C::kCopies)
                break;
            const int p0 = kWave * copy;           // first slot of this copy
            const int b = p0 / C::kPlane4;         // a copy never straddles planes
            const int f = swz<FMT>(p0 % C::kPlane4 + lane);
            const int g = min(seg * C::kPlane4 + f, k4 - 1);
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(x + (int64_t)b * K + 4 * g),
                                             (__attribute__((address_space(3))) void *)(buf + p0), 16, 0, 0);
        }
    } else {
        float *bufd = reinterpret_cast<float *>(buf);
#pragma unroll
        for (int j = 0; j < 4 * C::kDma; ++j) {
            const int copy = wave + C::kWaves * j; // 64-dword copies, wave-uniform
            if (copy >= 4 * C::kCopies)
                break;
            const int d = kWave * copy + lane;     // dword slot of this lane
            const int p = d / 4;
            const int b = p / C::kPlane4;
            const int f = swz<FMT>(p % C::kPlane4);
            const int g = min(seg * C::kPlane4 + f, k4 - 1);
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(x + (int64_t)b * K + 4 * g + d % 4),
                                             (__attribute__((address_space(3))) void *)(bufd + kWave * copy), 4,
                                             0, 0);
        }
    }
}

template <int FMT, int NC, int UO, int R, int U>
__device__ __forceinline__ void consume_cols(const Batch<FMT, R, U> &b, const f32x4 *xs, float (&acc)[R][NC],
                                             int lane, int chunk0, int nchunks)
{
    using F = Fmt<FMT>;
    constexpr int P = F::E / 4;
    constexpr int kPlane4 = ColsCfg<FMT, NC, UO>::kPlane4;
    const f32x4 *xs4 = xs;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int cl = lane + kWave * u; // chunk within the segment
        const bool valid = chunk0 + cl < nchunks;
        typename F::Dq dq[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            dq[r] = F::decode(b.q[r][u]);
#pragma unroll
        for (int col = 0; col < NC; ++col) {
            float xv[F::E];
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const f32x4 t = xs4[col * kPlane4 + swz<FMT>(cl * P + i)];
                xv[4 * i] = t.x;
                xv[4 * i + 1] = t.y;
                xv[4 * i + 2] = t.z;
                xv[4 * i + 3] = t.w;
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float t;
                if constexpr (F::kBlock)
                    t = F::dotd(dq[r], xv, b.sc[r][u], acc[r][col]);
                else
                    t = F::dotd(dq[r], xv, acc[r][col]);
                acc[r][col] = valid ? t : acc[r][col];
            }
            // one column at a time: hoisting the x reads of every column ahead
            // of the FMAs would hold U * NC * E floats in registers
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// GLU: the gated pair; W2 is the up matrix, act the gate's (SILU or
// SIGMOID), and each wave loads its R gate rows and the same R up rows.
template <int FMT, int NC, int UO, bool GLU = false>
__global__ __launch_bounds__((ColsCfg<FMT, NC, UO, GLU>::kWaves * kWave)) void gemv_cols_kernel(
    const unsigned char *__restrict__ W, const float *__restrict__ x, int N, int K, int act, const float *mop,
    const float *rop, float *dst, const unsigned char *__restrict__ W2)
{
    using F = Fmt<FMT>;
    using C = ColsCfg<FMT, NC, UO, GLU>;
    constexpr int R = C::R, U = C::U, SEGC = kWave * C::U;
    constexpr int RR = GLU ? 2 * R : R; // rows loaded per wave
    // two segment buffers (x of segment s+1 lands in one while segment s is
    // read from the other); a row of one segment gets only the first
    extern __shared__ f32x4 lds4[];
    f32x4 *const xa = lds4;
    f32x4 *const xb = lds4 + C::kBuf4;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nchunks = K / F::E;
    const int nseg = (nchunks + SEGC - 1) / SEGC;
    const int row0 = (blockIdx.x * C::kWaves + wave) * R;
    const int64_t rbytes = row_bytes<FMT>(K);
    const unsigned char *scales = F::kBlock ? W + align256_dev((int64_t)N * rbytes) : nullptr;
    const unsigned char *scales2 = (F::kBlock && GLU) ? W2 + align256_dev((int64_t)N * rbytes) : nullptr;
    const int64_t sbytes = (int64_t)(K / 32) * 2;

    // 1. epilogue operand of the output this lane finishes (lane j: row
    //    row0 + j % R of column j / R; other lanes read a clamped element)
    const int jo = min(lane, R * NC - 1);
    const int orow = min(row0 + jo % R, N - 1), ocol = jo / R;
    const bool has_op = act == GEMV_ACT_SILU_MUL || act == GEMV_ACT_MUL || act == GEMV_ACT_ADD;
    const float *opp = act == GEMV_ACT_ADD ? rop : (has_op ? mop : x);
    const float opv = opp[has_op ? (int64_t)ocol * N + orow : 0];

    // 2. x of the first segment, straight into LDS
    const bool x16 = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
    dma_x_segment<FMT, NC, UO, GLU>(xa, x, K, 0, wave, lane, x16);

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
    Batch<FMT, RR, U> b0, b1;
    if constexpr (UO == 0) // one-shot: W follows the wait for x (below)
        issue_batch<FMT, RR, U>(b0, wrow, srow, lane, 0, nchunks);

    float acc[RR][NC];
#pragma unroll
    for (int r = 0; r < RR; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c)
            acc[r][c] = 0.0f;

    // 4. segments, two per trip: even segments use buffer xa and batch b0, odd
    //    ones xb and b1.  At the top of a segment this wave's only outstanding
    //    loads are that segment's x copy and W batch, both needed now, so it
    //    waits for all of them; the barrier then makes every wave's copy
    //    visible and guarantees that all waves are done with the other buffer,
    //    which the next segment's copy overwrites.
    if constexpr (UO > 0) {
        // the whole row is one segment: wait for the x copy, barrier, then
        // issue every W chunk, so that the FMAs wait for each chunk as it
        // lands (the copy's wait would otherwise have waited for all of W)
        __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0); expcnt, lgkmcnt not waited for
        __builtin_amdgcn_s_barrier();
        issue_batch<FMT, RR, U>(b0, wrow, srow, lane, 0, nchunks);
        consume_cols<FMT, NC, UO, RR, U>(b0, xa, acc, lane, 0, nchunks);
    } else
    for (int s = 0;;) {
        __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0); expcnt, lgkmcnt not waited for
        __builtin_amdgcn_s_barrier();
        if (s + 1 < nseg) {
            dma_x_segment<FMT, NC, UO, GLU>(xb, x, K, s + 1, wave, lane, x16);
            issue_batch<FMT, RR, U>(b1, wrow, srow, lane, (s + 1) * U, nchunks);
        }
        consume_cols<FMT, NC, UO, RR, U>(b0, xa, acc, lane, s * SEGC, nchunks);
        if (++s == nseg)
            break;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __builtin_amdgcn_s_barrier();
        if (s + 1 < nseg) {
            dma_x_segment<FMT, NC, UO, GLU>(xa, x, K, s + 1, wave, lane, x16);
            issue_batch<FMT, RR, U>(b0, wrow, srow, lane, (s + 1) * U, nchunks);
        }
        consume_cols<FMT, NC, UO, RR, U>(b1, xb, acc, lane, s * SEGC, nchunks);
        if (++s == nseg)
            break;
    }

    // 5. reduce every (row, column) sum; lane j takes output j (and its up
    //    sum for a gated pair), then one epilogue per lane
    float mine = 0.0f, mine2 = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float sum = wave_sum(acc[r][c]);
            mine = lane == c * R + r ? sum : mine;
            if constexpr (GLU) {
                const float sum2 = wave_sum(acc[R + r][c]);
                mine2 = lane == c * R + r ? sum2 : mine2;
            }
        }
    const float y = GLU ? apply_glu(act, mine, mine2) : apply_epilogue(act, mine, opv);
    if (lane < R * NC && row0 + lane % R < N)
        dst[(int64_t)(lane / R) * N + row0 + lane % R] = y;
}

// The one-shot form on a resident grid: each workgroup stages x of every
// column once, then walks the row tiles blockIdx.x, blockIdx.x + gridDim.x,
// ...; a tile's rows are computed exactly as in gemv_cols_kernel (same lanes,
// same chunk order, same reduction), so results are bitwise the same.  Tiles
// after the first need no barrier: x in LDS is only read.
template <int FMT, int NC, int UO, bool GLU>
__global__ __launch_bounds__((ColsCfg<FMT, NC, UO, GLU>::kWaves * kWave)) void gemv_cols_tiles_kernel(
    const unsigned char *__restrict__ W, const float *__restrict__ x, int N, int K, int act, const float *mop,
    const float *rop, float *dst, const unsigned char *__restrict__ W2)
{
    static_assert(UO > 0, "the whole row is one segment");
    using F = Fmt<FMT>;
    using C = ColsCfg<FMT, NC, UO, GLU>;
    constexpr int R = C::R, U = C::U;
    constexpr int RR = GLU ? 2 * R : R;
    extern __shared__ f32x4 lds4[];
    f32x4 *const xa = lds4;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nchunks = K / F::E;
    const int ntiles = (N + C::kWaves * R - 1) / (C::kWaves * R);
    const int64_t rbytes = row_bytes<FMT>(K);
    const unsigned char *scales = F::kBlock ? W + align256_dev((int64_t)N * rbytes) : nullptr;
    const unsigned char *scales2 = (F::kBlock && GLU) ? W2 + align256_dev((int64_t)N * rbytes) : nullptr;
    const int64_t sbytes = (int64_t)(K / 32) * 2;
    const int jo = min(lane, R * NC - 1);
    const bool has_op = act == GEMV_ACT_SILU_MUL || act == GEMV_ACT_MUL || act == GEMV_ACT_ADD;
    const float *opp = act == GEMV_ACT_ADD ? rop : (has_op ? mop : x);

    const bool x16 = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
    dma_x_segment<FMT, NC, UO, GLU>(xa, x, K, 0, wave, lane, x16);
    __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0); expcnt, lgkmcnt not waited for
    __builtin_amdgcn_s_barrier();

    auto tile_rows = [&](int row0, const unsigned char *(&wrow)[RR], const unsigned char *(&srow)[RR]) {
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
    };
    auto operand_of = [&](int row0) {
        const int orow = min(row0 + jo % R, N - 1), ocol = jo / R;
        return opp[has_op ? (int64_t)ocol * N + orow : 0];
    };
    // consume a landed batch, reduce every (row, column) sum and store
    auto finish = [&](const Batch<FMT, RR, U> &b, int row0, float opv) {
        float acc[RR][NC];
#pragma unroll
        for (int r = 0; r < RR; ++r)
#pragma unroll
            for (int c = 0; c < NC; ++c)
                acc[r][c] = 0.0f;
        consume_cols<FMT, NC, UO, RR, U>(b, xa, acc, lane, 0, nchunks);
        float mine = 0.0f, mine2 = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float sum = wave_sum(acc[r][c]);
                mine = lane == c * R + r ? sum : mine;
                if constexpr (GLU) {
                    const float sum2 = wave_sum(acc[R + r][c]);
                    mine2 = lane == c * R + r ? sum2 : mine2;
                }
            }
        const float y = GLU ? apply_glu(act, mine, mine2) : apply_epilogue(act, mine, opv);
        if (lane < R * NC && row0 + lane % R < N)
            dst[(int64_t)(lane / R) * N + row0 + lane % R] = y;
    };
    const unsigned char *wrow[RR];
    const unsigned char *srow[RR];

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int row0 = (tile * C::kWaves + wave) * R;
        // epilogue operand first: the loads retire in order, so the W waits
        // below cover it
        const float opv = operand_of(row0);
        tile_rows(row0, wrow, srow);
        Batch<FMT, RR, U> b0;
        issue_batch<FMT, RR, U>(b0, wrow, srow, lane, 0, nchunks);
        finish(b0, row0, opv);
    }
}

// Any K (float formats whose rows are not whole 16-byte chunks, or x too long
// for the one-column kernel's LDS): one wave per row, element loads, x read
// through the caches, in the order of the one-column generic kernel.
template <int FMT>
__device__ __forceinline__ float weight_at_cols(const unsigned char *W, int N, int K, int row, int k)
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

template <int FMT, int NC, bool GLU = false>
__global__ __launch_bounds__(256) void gemv_cols_generic_kernel(const unsigned char *__restrict__ W,
                                                                const float *__restrict__ x, int N, int K, int act,
                                                                const float *mop, const float *rop, float *dst,
                                                                const unsigned char *__restrict__ W2)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int nwaves = gridDim.x * (blockDim.x / kWave);
    for (int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; row < N; row += nwaves) {
        float acc[NC], acc2[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c)
            acc[c] = acc2[c] = 0.0f;
        for (int k = lane; k < K; k += kWave) {
            const float w = weight_at_cols<FMT>(W, N, K, row, k);
#pragma unroll
            for (int c = 0; c < NC; ++c)
                acc[c] = fmaf(w, x[(int64_t)c * K + k], acc[c]);
            if constexpr (GLU) {
                const float w2 = weight_at_cols<FMT>(W2, N, K, row, k);
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    acc2[c] = fmaf(w2, x[(int64_t)c * K + k], acc2[c]);
            }
        }
        float mine = 0.0f, mine2 = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float sum = wave_sum(acc[c]);
            mine = lane == c ? sum : mine;
            if constexpr (GLU) {
                const float sum2 = wave_sum(acc2[c]);
                mine2 = lane == c ? sum2 : mine2;
            }
        }
        if (lane < NC) {
            const int64_t o = (int64_t)lane * N + row;
            if constexpr (GLU) {
                dst[o] = apply_glu(act, mine, mine2);
            } else {
                const bool has_op = act == GEMV_ACT_SILU_MUL || act == GEMV_ACT_MUL || act == GEMV_ACT_ADD;
                const float v = has_op ? (act == GEMV_ACT_ADD ? rop[o] : mop[o]) : 0.0f;
                dst[o] = apply_epilogue(act, mine, v);
            }
        }
    }
}

// ------------------------------------------------------------------ host dispatch

using ColsCall = ColsArgs;

template <int FMT, int NC, int UO, bool GLU = false> hipError_t launch_cols(const ColsCall &c, hipStream_t s)
{
    using C = ColsCfg<FMT, NC, UO, GLU>;
    const void *fn = reinterpret_cast<const void *>(&gemv_cols_kernel<FMT, NC, UO, GLU>);
    const int nchunks = c.K / C::E;
    const int nseg = (nchunks + kWave * C::U - 1) / (kWave * C::U);
    const size_t lds = (size_t)(nseg > 1 ? 2 : 1) * C::kBuf4 * 16;
    if (2 * C::kBuf4 * 16 > 64 * 1024) {
        static std::once_flag once;
        static hipError_t attr_err = hipSuccess;
        std::call_once(once, [&] { attr_err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds); });
        if (attr_err != hipSuccess)
            return attr_err;
    }
    const int rows_per_tile = C::kWaves * C::R;
    int grid = (c.N + rows_per_tile - 1) / rows_per_tile;
    // the one-shot form runs on a resident grid (occupancy x CUs) whose
    // workgroups stage x once and walk the row tiles: measured 2-9 % faster
    // for the gated pair at 14336x4096 (8-bit at 4 columns 33.6 -> 30.6 us)
    // and 0-3 % for float-format plain columns
    if constexpr (UO > 0) {
        fn = reinterpret_cast<const void *>(&gemv_cols_tiles_kernel<FMT, NC, UO, GLU>);
        static std::once_flag once;
        static hipError_t attr_err = hipSuccess;
        static int per_cu = 0;
        constexpr size_t lds1 = (size_t)C::kBuf4 * 16; // one segment: lds == lds1 here
        std::call_once(once, [&] {
            if (lds1 > 64 * 1024)
                attr_err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
            if (attr_err == hipSuccess)
                attr_err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, C::kWaves * kWave, lds1);
        });
        if (attr_err != hipSuccess)
            return attr_err;
        const int slots = (per_cu > 0 ? per_cu : 1) * device_cus();
        if (grid > slots)
            grid = slots;
    }
    const unsigned char *W = c.W;
    const float *x = c.x;
    int N = c.N, K = c.K, act = c.act;
    const float *m = c.m, *r = c.r;
    float *dst = c.dst;
    const unsigned char *W2 = c.W2;
    void *args[] = {&W, &x, &N, &K, &act, &m, &r, &dst, &W2};
    return hipLaunchKernel(fn, dim3(grid), dim3(C::kWaves * kWave), args, lds, s);
}

template <int FMT, int NC, bool GLU = false> hipError_t launch_cols_generic(const ColsCall &c, hipStream_t s)
{
    const void *fn = reinterpret_cast<const void *>(&gemv_cols_generic_kernel<FMT, NC, GLU>);
    int grid = (c.N + 3) / 4;
    if (grid > 65536)
        grid = 65536;
    const unsigned char *W = c.W;
    const float *x = c.x;
    int N = c.N, K = c.K, act = c.act;
    const float *m = c.m, *r = c.r;
    float *dst = c.dst;
    const unsigned char *W2 = c.W2;
    void *args[] = {&W, &x, &N, &K, &act, &m, &r, &dst, &W2};
    return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, s);
}

// The chunked kernel exactly where the one-column call takes its chunked
// kernel (rows of whole 16-byte chunks, x of one column fits the one-column
// kernel's padded LDS staging), so that every column reduces in the same
// order as the one-column call.
// One segment per row (UO chunks per lane) wherever the row fits it and x
// of every column fits LDS: f16/bf16/f32 up to 8 chunks per lane, the 8-bit
// format up to 4 and the 4-bit format up to 2 (K <= 4096 for the 16-bit and
// block formats, 2048 for f32).
template <int FMT> constexpr int oneshot_u() { return Fmt<FMT>::E <= 8 ? 8 : (Fmt<FMT>::E == 16 ? 4 : 2); }

template <int FMT, int NC, bool GLU = false> hipError_t dispatch_cols(const ColsCall &c, hipStream_t s)
{
    const int64_t lds1 = (int64_t)(c.K / Fmt<FMT>::E) * Fmt<FMT>::XS * 4;
    const bool fast = (row_bytes<FMT>(c.K) % 16 == 0) && lds1 <= kMaxLds;
    if (!fast)
        return launch_cols_generic<FMT, NC, GLU>(c, s);
    constexpr int UO = oneshot_u<FMT>();
    const int cpl = (c.K / Fmt<FMT>::E + kWave - 1) / kWave;
    if constexpr (NC * kWave * UO * Fmt<FMT>::E * 4 <= kMaxLds) {
        // measured on the resident grid: the block formats gain wherever it
        // fits; the float formats wherever x of all columns stays within
        // 64 KiB (two workgroups per CU), at any row count (bf16 1024x4096
        // at 3 columns 7.5 -> 6.2 us, f16 4096^2 at 2 columns 8.6 -> 8.0 us;
        // the gated pair: f32 4096x2048 at 2 columns 14.7 -> 12.2 us), and
        // beyond it only where the 16-row workgroups are exactly one round
        const int64_t lds = (int64_t)NC * kWave * cpl * Fmt<FMT>::E * 4;
        const int64_t wgs = (c.N + 15) / 16, cus = device_cus();
        const bool take = Fmt<FMT>::kBlock || lds <= 64 * 1024 || (NC >= 3 && wgs == cus);
        if (cpl <= UO && take)
            return launch_cols<FMT, NC, UO, GLU>(c, s);
    }
    return launch_cols<FMT, NC, 0, GLU>(c, s);
}

template <int NC, bool GLU = false> hipError_t dispatch_cols_fmt(int wfmt, const ColsCall &c, hipStream_t s)
{
    switch (wfmt) {
    case GEMV_W_F32:
        return dispatch_cols<GEMV_W_F32, NC, GLU>(c, s);
    case GEMV_W_F16:
        return dispatch_cols<GEMV_W_F16, NC, GLU>(c, s);
    case GEMV_W_BF16:
        return dispatch_cols<GEMV_W_BF16, NC, GLU>(c, s);
    case GEMV_W_Q8B32:
        return dispatch_cols<GEMV_W_Q8B32, NC, GLU>(c, s);
    default:
        return dispatch_cols<GEMV_W_Q4B32, NC, GLU>(c, s);
    }
}

template <bool GLU = false> hipError_t dispatch_ncols(int wfmt, int ncols, const ColsCall &c, hipStream_t s)
{
    switch (ncols) {
    case 2:
        return dispatch_cols_fmt<2, GLU>(wfmt, c, s);
    case 3:
        return dispatch_cols_fmt<3, GLU>(wfmt, c, s);
    case 4:
        return dispatch_cols_fmt<4, GLU>(wfmt, c, s);
    case 5:
        return dispatch_cols_fmt<5, GLU>(wfmt, c, s);
    case 6:
        return dispatch_cols_fmt<6, GLU>(wfmt, c, s);
    case 7:
        return dispatch_cols_fmt<7, GLU>(wfmt, c, s);
    default:
        return dispatch_cols_fmt<8, GLU>(wfmt, c, s);
    }
}

} // namespace
} // namespace gemv

namespace gemv {
namespace {

// The chunked column kernel's condition (dispatch_cols) for a run-time format.
bool cols_fast(int wfmt, int64_t K)
{
    static const int kE[5] = {4, 8, 8, 16, 32}, kXS[5] = {4, 12, 12, 20, 36};
    const int64_t rb = wfmt == GEMV_W_F32 ? 4 * K : (wfmt == GEMV_W_Q8B32 ? K : (wfmt == GEMV_W_Q4B32 ? K / 2 : 2 * K));
    return rb % 16 == 0 && (K / kE[wfmt]) * kXS[wfmt] * 4 <= kMaxLds;
}

} // namespace
} // namespace gemv

extern "C" {

int gemv_ncols_kernel(int wfmt, int64_t N, int64_t K, int64_t ncols)
{
    if (wfmt < GEMV_W_F32 || wfmt > GEMV_W_Q4B32)
        return GEMV_E_FMT;
    if (N < 1 || K < 1 || ncols < 1 || ncols > GEMV_MAX_NCOLS || N >= GEMV_MAX_DIM_EXTENT ||
        K >= GEMV_MAX_DIM_EXTENT || ((wfmt == GEMV_W_Q8B32 || wfmt == GEMV_W_Q4B32) && K % 32 != 0))
        return GEMV_E_DIM;
    if (ncols == 1)
        return GEMV_KERNEL_ONE_COLUMN;
    if (gemv::cols_mfma_plan(wfmt, (int)ncols, N, K, gemv::device_cus()).rt)
        return GEMV_KERNEL_COLUMNS_MATRIX;
    return gemv::cols_fast(wfmt, K) ? GEMV_KERNEL_COLUMNS : GEMV_KERNEL_COLUMNS_GENERIC;
}

int gemv_fused_ncols(const void *W, int wfmt, int64_t N, int64_t K, int64_t ncols, const float *x, int act,
                     const gemv_view *mul_operand, const gemv_view *add_operand, const gemv_view *dst,
                     void *hip_stream)
{
    int st = gemv::validate_ncols(W, wfmt, N, K, ncols, x, act, mul_operand, add_operand, dst);
    if (st != GEMV_OK)
        return st;
    if (ncols == 1)
        return gemv_fused(W, wfmt, N, K, x, act, mul_operand, add_operand, dst, hip_stream);
    gemv::ColsCall c{static_cast<const unsigned char *>(W), x, (int)N, (int)K, act,
                     mul_operand ? mul_operand->data : nullptr, add_operand ? add_operand->data : nullptr,
                     dst->data};
    // f16, bf16 and the block formats take the matrix-core kernel
    // (gemv_mfma.hip) where the shape fits it
    const int e = gemv::launch_cols_mfma(wfmt, (int)ncols, c, hip_stream);
    if (e >= 0)
        return gemv::finish_launch(e);
    return gemv::finish_launch(
        (int)gemv::dispatch_ncols(wfmt, (int)ncols, c, static_cast<hipStream_t>(hip_stream)));
}

int gemv_glu_ncols(const void *W_gate, const void *W_up, int wfmt, int64_t N, int64_t K, int64_t ncols,
                   const float *x, int act, const gemv_view *dst, void *hip_stream)
{
    int st = gemv::validate_glu_ncols(W_gate, W_up, wfmt, N, K, ncols, x, act, dst);
    if (st != GEMV_OK)
        return st;
    if (ncols == 1)
        return gemv_glu(W_gate, W_up, wfmt, N, K, x, act, dst, hip_stream);
    // Where one matrix's columns would run on the matrix cores, two
    // matrix-core launches beat the vector-ALU pair (measured): the up
    // product into dst, then the gate's with silu(g) * u in place (dst is
    // the multiplier's identical view).  apply_epilogue's SILU_MUL and
    // apply_glu's SILU are the same arithmetic.
    if (act == GEMV_ACT_SILU && gemv::cols_mfma_plan(wfmt, (int)ncols, N, K, gemv::device_cus()).rt) {
        const gemv::ColsCall up{static_cast<const unsigned char *>(W_up), x, (int)N, (int)K, GEMV_ACT_NONE, nullptr,
                                nullptr, dst->data};
        int e = gemv::launch_cols_mfma(wfmt, (int)ncols, up, hip_stream);
        if (e != 0)
            return gemv::finish_launch(e);
        const gemv::ColsCall gate{static_cast<const unsigned char *>(W_gate), x, (int)N, (int)K, GEMV_ACT_SILU_MUL,
                                  dst->data, nullptr, dst->data};
        return gemv::finish_launch(gemv::launch_cols_mfma(wfmt, (int)ncols, gate, hip_stream));
    }
    gemv::ColsCall c{static_cast<const unsigned char *>(W_gate), x, (int)N, (int)K, act, nullptr, nullptr,
                     dst->data, static_cast<const unsigned char *>(W_up)};
    return gemv::finish_launch(
        (int)gemv::dispatch_ncols<true>(wfmt, (int)ncols, c, static_cast<hipStream_t>(hip_stream)));
}

} // extern "C"

// Device code shared by the HIP translation units of the fused decode GEMV:
// vector types, the epilogue functions, the wave reduction, the weight-format
// decoders and dot products, W batch loads and the LDS barrier.  Everything
// sits in an unnamed namespace, so each translation unit has its own copy.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "gemv_fused.h"

namespace gemv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
__host__ __device__ __forceinline__ int64_t align256_dev(int64_t v) { return (v + 255) / 256 * 256; }
constexpr int kMaxLds = 160 * 1024; // LDS bytes a gfx950 workgroup may allocate

// ------------------------------------------------------------------ epilogue

// sigmoid(a) = 1 / (1 + e^-a) and silu(a) = a * sigmoid(a), evaluated with
// t = e^-|a| <= 1 so that nothing overflows: for a < 0 the same values are
// t / (1 + t) and a t / (1 + t).  (The direct form turns silu(a) into -0 once
// e^-a overflows, near a = -88.7, although the true value is still a normal
// float there.)
//
// Below a = -80, e^a (under 2e-35) is leaving float's normal range: on its
// own it would round to zero or to a few subnormal bits before |a| and a
// multiplier scale it back up (silu(-103) * 40 is about -5e-42, a float,
// while e^-103 alone rounds to 0).  There the product f * e^a is formed
// 2^64 times larger, where e^(a + 64 ln 2) is a normal float, and scaled
// back once, so that it rounds into the subnormal range a single time;
// 1 + e^a is 1 in float there.  -inf still gives silu NaN and sigmoid 0.
constexpr float kTailA = -80.0f;
constexpr float kLn2Times64 = 44.3614195558365f; // 64 ln 2

__device__ __forceinline__ float tail_scaled(float f, float a) { return ldexpf(f * expf(a + kLn2Times64), -64); }

__device__ __forceinline__ float sigmoid_f(float a)
{
    if (a < kTailA)
        return tail_scaled(1.0f, a);
    float t = expf(-fabsf(a));
    return (a >= 0.0f ? 1.0f : t) / (1.0f + t);
}

__device__ __forceinline__ float silu_f(float a)
{
    if (a < kTailA)
        return tail_scaled(a, a);
    float t = expf(-fabsf(a));
    return (a >= 0.0f ? a : a * t) / (1.0f + t);
}

// silu(a) * v and sigmoid(a) * v, with v taken into the product before the
// final scaling in the tail ((a e) v: a e is 0 rather than a v overflowing).
__device__ __forceinline__ float silu_mul_f(float a, float v)
{
    if (a < kTailA)
        return ldexpf(a * expf(a + kLn2Times64) * v, -64);
    return silu_f(a) * v;
}

__device__ __forceinline__ float sigmoid_mul_f(float a, float v)
{
    if (a < kTailA)
        return tail_scaled(v, a);
    return sigmoid_f(a) * v;
}

// The epilogue of one output: v is m_i for SILU_MUL and MUL, r_i for ADD.
__device__ __forceinline__ float apply_epilogue(int act, float a, float v)
{
    switch (act) {
    case GEMV_ACT_SIGMOID:
        return sigmoid_f(a);
    case GEMV_ACT_SILU:
        return silu_f(a);
    case GEMV_ACT_SILU_MUL:
        return silu_mul_f(a, v);
    case GEMV_ACT_MUL:
        return a * v;
    case GEMV_ACT_ADD:
        return a + v;
    default:
        return a;
    }
}

__device__ __forceinline__ float operand_of(int act, const float *m, const float *r, int64_t i)
{
    if (act == GEMV_ACT_SILU_MUL || act == GEMV_ACT_MUL)
        return m[i];
    if (act == GEMV_ACT_ADD)
        return r[i];
    return 0.0f;
}

// ------------------------------------------------------------------ wave reduce

// A DPP lane permutation of v.  Every pattern used below reads a valid lane,
// so bound_ctrl is irrelevant to the result; setting it lets the compiler
// fold the move into the consuming add (v_add_f32_dpp).
template <int CTRL> __device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float lane_read(float v, int l)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Sum of v over the 64 lanes, returned uniformly.  quad_perm swaps, then
// half-row and row mirrors leave each 16-lane row's sum in all its lanes.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp<0xB1>(v);  // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);  // quad_perm [2,3,0,1]
    v += dpp<0x141>(v); // row_half_mirror
    v += dpp<0x140>(v); // row_mirror
    return (lane_read(v, 0) + lane_read(v, 16)) + (lane_read(v, 32) + lane_read(v, 48));
}

// ------------------------------------------------------------------ formats
// E:   weights per 16-byte chunk of W.
// XS:  LDS floats per chunk of x (E plus padding).
// kBlock: the format has an fp16 scale plane; a chunk is 1/kChunksPerBlock
//         of a 32-weight block.

__device__ __forceinline__ float f16lo(unsigned d) { return (float)__builtin_bit_cast(f16x2, d).x; }
__device__ __forceinline__ float f16hi(unsigned d) { return (float)__builtin_bit_cast(f16x2, d).y; }

template <int FMT> struct Fmt;

// Each format decodes a 16-byte chunk once into a register form (Dq) that
// dotd() reads, so that several columns can share one decode; dot() fuses the
// two for the one-column kernels.  Both perform the same FMAs in the same
// order, so a product formed through either path rounds identically.
template <> struct Fmt<GEMV_W_F32> {
    static constexpr int E = 4, XS = 4;
    static constexpr bool kBlock = false;
    static constexpr int kChunksPerBlock = 0;
    struct Dq {
        float w[4];
    };
    __device__ static __forceinline__ Dq decode(u32x4 q)
    {
        // Copy the lanes out before reinterpreting: __builtin_bit_cast applied
        // to an element of an ext_vector_type reads the vector's first element.
        unsigned d[4] = {q.x, q.y, q.z, q.w};
        Dq r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.w[i] = __builtin_bit_cast(float, d[i]);
        return r;
    }
    __device__ static __forceinline__ float dotd(const Dq &w, const float *xv, float acc)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = fmaf(w.w[i], xv[i], acc);
        return acc;
    }
    __device__ static __forceinline__ float dot(u32x4 q, const float *xv, float acc) { return dotd(decode(q), xv, acc); }
};

template <> struct Fmt<GEMV_W_F16> {
    static constexpr int E = 8, XS = 12;
    static constexpr bool kBlock = false;
    static constexpr int kChunksPerBlock = 0;
    struct Dq {
        unsigned d[4]; // the f16 pairs as loaded; the FMAs convert them exactly
    };
    __device__ static __forceinline__ Dq decode(u32x4 q) { return Dq{{q.x, q.y, q.z, q.w}}; }
    __device__ static __forceinline__ float dotd(const Dq &w, const float *xv, float acc)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = fmaf(f16lo(w.d[i]), xv[2 * i], acc);
            acc = fmaf(f16hi(w.d[i]), xv[2 * i + 1], acc);
        }
        return acc;
    }
    __device__ static __forceinline__ float dot(u32x4 q, const float *xv, float acc) { return dotd(decode(q), xv, acc); }
};

template <> struct Fmt<GEMV_W_BF16> {
    static constexpr int E = 8, XS = 12;
    static constexpr bool kBlock = false;
    static constexpr int kChunksPerBlock = 0;
    struct Dq {
        float w[8];
    };
    __device__ static __forceinline__ Dq decode(u32x4 q)
    {
        unsigned d[4] = {q.x, q.y, q.z, q.w};
        Dq r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r.w[2 * i] = __builtin_bit_cast(float, d[i] << 16);
            r.w[2 * i + 1] = __builtin_bit_cast(float, d[i] & 0xFFFF0000u);
        }
        return r;
    }
    __device__ static __forceinline__ float dotd(const Dq &w, const float *xv, float acc)
    {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc = fmaf(w.w[i], xv[i], acc);
        return acc;
    }
    __device__ static __forceinline__ float dot(u32x4 q, const float *xv, float acc)
    {
        unsigned d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = fmaf(__builtin_bit_cast(float, d[i] << 16), xv[2 * i], acc);
            acc = fmaf(__builtin_bit_cast(float, d[i] & 0xFFFF0000u), xv[2 * i + 1], acc);
        }
        return acc;
    }
};

// 8-bit blocks: a chunk is 16 codes (half a block).  Partial sum of code * x,
// then one multiply-add by the block scale.
template <> struct Fmt<GEMV_W_Q8B32> {
    static constexpr int E = 16, XS = 20;
    static constexpr bool kBlock = true;
    static constexpr int kChunksPerBlock = 2;
    struct Dq {
        float w[16];
    };
    __device__ static __forceinline__ Dq decode(u32x4 q)
    {
        unsigned d[4] = {q.x, q.y, q.z, q.w};
        Dq r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                r.w[4 * i + b] = (float)(int)(signed char)((d[i] >> (8 * b)) & 0xFF);
        return r;
    }
    __device__ static __forceinline__ float dotd(const Dq &w, const float *xv, _Float16 scale, float acc)
    {
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            p = fmaf(w.w[i], xv[i], p);
        return fmaf(p, (float)scale, acc);
    }
    __device__ static __forceinline__ float dot(u32x4 q, const float *xv, _Float16 scale, float acc)
    {
        unsigned d[4] = {q.x, q.y, q.z, q.w};
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                float w = (float)(int)(signed char)((d[i] >> (8 * b)) & 0xFF);
                p = fmaf(w, xv[4 * i + b], p);
            }
        }
        return fmaf(p, (float)scale, acc);
    }
};

// (d & mask) | bits in one VALU op.  The compiler emits an AND and an OR with
// literal operands; v_and_or_b32 takes one constant from an SGPR and the other
// from a VGPR (gfx9 VOP3 reads at most one scalar operand).
__device__ __forceinline__ unsigned and_or(unsigned d, unsigned mask, unsigned bits)
{
    unsigned r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(d), "s"(mask), "v"(bits));
    return r;
}

// 4-bit blocks: a chunk is one whole block of 32 codes.  A dword holds
// elements 8i..8i+7, element k in bits 4k..4k+3.  OR-ing a nibble into the
// mantissa of the f16 constant 1024 gives 1024 + c exactly (nibble at bit 0)
// or 1024 + 16c (nibble at bit 4); subtracting 1032 leaves c - 8 exactly, and
// (1024 + 16c) / 16 - 72, one packed f16 FMA, leaves c - 8 exactly too (the
// product is 64 + c, the sum c - 8, each exact in f16).  Each instruction
// turns two nibbles into two exact f16 weights.  The block's sum is then
// scaled by its fp16 scale in one mixed-precision FMA.
template <> struct Fmt<GEMV_W_Q4B32> {
    static constexpr int E = 32, XS = 36;
    static constexpr bool kBlock = true;
    static constexpr int kChunksPerBlock = 1;
    struct Dq {
        f16x2 h[4][4]; // per dword: (c0-8, c4-8), (c1-8, c5-8), (c2-8, c6-8), (c3-8, c7-8)
    };
    // low nibbles of each 16-bit half: 1024 + c -> c - 8
    __device__ static __forceinline__ f16x2 lo_pair(unsigned d)
    {
        const f16x2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
        return __builtin_bit_cast(f16x2, and_or(d, 0x000F000Fu, 0x64006400u)) - off;
    }
    // second nibbles: 1024 + 16 c -> (1024 + 16 c) / 16 - 72 = c - 8
    __device__ static __forceinline__ f16x2 hi_pair(unsigned d)
    {
        const f16x2 k = {(_Float16)0.0625f, (_Float16)0.0625f};
        const f16x2 off = {(_Float16)-72.0f, (_Float16)-72.0f};
        return __builtin_elementwise_fma(__builtin_bit_cast(f16x2, and_or(d, 0x00F000F0u, 0x64006400u)), k, off);
    }
    __device__ static __forceinline__ Dq decode(u32x4 q)
    {
        unsigned d[4] = {q.x, q.y, q.z, q.w};
        Dq r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const unsigned e = d[i] >> 8;
            r.h[i][0] = lo_pair(d[i]);
            r.h[i][1] = hi_pair(d[i]);
            r.h[i][2] = lo_pair(e);
            r.h[i][3] = hi_pair(e);
        }
        return r;
    }
    __device__ static __forceinline__ float dotd(const Dq &w, const float *xv, _Float16 scale, float acc)
    {
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float *xi = xv + 8 * i;
            a0 = fmaf((float)w.h[i][0].x, xi[0], a0);
            a0 = fmaf((float)w.h[i][0].y, xi[4], a0);
            a0 = fmaf((float)w.h[i][2].x, xi[2], a0);
            a0 = fmaf((float)w.h[i][2].y, xi[6], a0);
            a1 = fmaf((float)w.h[i][1].x, xi[1], a1);
            a1 = fmaf((float)w.h[i][1].y, xi[5], a1);
            a1 = fmaf((float)w.h[i][3].x, xi[3], a1);
            a1 = fmaf((float)w.h[i][3].y, xi[7], a1);
        }
        return fmaf(a0 + a1, (float)scale, acc);
    }
    __device__ static __forceinline__ float dot(u32x4 q, const float *xv, _Float16 scale, float acc)
    {
        unsigned d[4] = {q.x, q.y, q.z, q.w};
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float *xi = xv + 8 * i;
            const unsigned e = d[i] >> 8;
            const f16x2 h0 = lo_pair(d[i]); // c0-8, c4-8
            const f16x2 h1 = hi_pair(d[i]); // c1-8, c5-8
            const f16x2 h2 = lo_pair(e);    // c2-8, c6-8
            const f16x2 h3 = hi_pair(e);    // c3-8, c7-8
            a0 = fmaf((float)h0.x, xi[0], a0);
            a0 = fmaf((float)h0.y, xi[4], a0);
            a0 = fmaf((float)h2.x, xi[2], a0);
            a0 = fmaf((float)h2.y, xi[6], a0);
            a1 = fmaf((float)h1.x, xi[1], a1);
            a1 = fmaf((float)h1.y, xi[5], a1);
            a1 = fmaf((float)h3.x, xi[3], a1);
            a1 = fmaf((float)h3.y, xi[7], a1);
        }
        return fmaf(a0 + a1, (float)scale, acc);
    }
};

// Byte layout helpers (see the header for the formats).
template <int FMT> __host__ __device__ __forceinline__ int64_t row_bytes(int64_t K)
{
    return FMT == GEMV_W_F32 ? K * 4 : (FMT == GEMV_W_Q8B32 ? K : (FMT == GEMV_W_Q4B32 ? K / 2 : K * 2));
}

__device__ __forceinline__ float load_scale(const unsigned char *p)
{
    unsigned short h = *reinterpret_cast<const unsigned short *>(p);
    return (float)__builtin_bit_cast(_Float16, h);
}

// A block scale kept as loaded: the dot products take it as the f16 operand
// of their final mixed-precision FMA, which converts it exactly.
__device__ __forceinline__ _Float16 load_scale_h(const unsigned char *p)
{
    return __builtin_bit_cast(_Float16, *reinterpret_cast<const unsigned short *>(p));
}

template <int FMT, int R, int U> struct Batch {
    u32x4 q[R][U];
    _Float16 sc[R][U];
};

template <int FMT, int R, int U>
__device__ __forceinline__ void issue_batch(Batch<FMT, R, U> &b, const unsigned char *const *wrow,
                                            const unsigned char *const *srow, int lane, int jb, int nchunks)
{
    using F = Fmt<FMT>;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // non-negative and below 2^31: as an unsigned offset the load takes the
        // row's (uniform) base address from scalar registers
        const unsigned c = (unsigned)min(lane + kWave * (jb + u), nchunks - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            b.q[r][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wrow[r]) + c);
            if constexpr (F::kBlock)
                b.sc[r][u] = load_scale_h(srow[r] + 2 * (c / F::kChunksPerBlock));
        }
    }
}

// Physical float4 slot of float4 f of an unpadded x plane in LDS: the E/4 pieces of chunk
// c = f / (E/4) are permuted by an XOR with bits of c, so that for any 8 (or
// 16) consecutive chunks read by consecutive lanes the same piece lands in 8
// (or 16) distinct 16-byte bank groups.
template <int FMT> __device__ __forceinline__ int swz(int f)
{
    constexpr int P = Fmt<FMT>::E / 4;        // pieces per chunk: 1, 2, 4 or 8
    constexpr int e = P == 1 ? 0 : (P == 2 ? 1 : (P == 4 ? 2 : 3));
    const int c = f >> e;
    return f ^ (((c >> (3 - e)) ^ (c >> (4 - e))) & (P - 1));
}

// Compute units of the current device (queried once per device).
inline int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Workgroup barrier for LDS only: waits for this wave's LDS writes, not for
// its outstanding global loads.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The gated pair of products (GLU): W is the gate matrix and W2 the up matrix,
// both streamed over the same staged x; the wave's batch holds R gate rows
// followed by the same R up rows, and the epilogue is act(gate) * up.
__device__ __forceinline__ float apply_glu(int act, float g, float u)
{
    // SILU is apply_epilogue's SILU_MUL with v = u, operation for operation
    return act == GEMV_ACT_SIGMOID ? sigmoid_mul_f(g, u) : silu_mul_f(g, u);
}

} // namespace
} // namespace gemv

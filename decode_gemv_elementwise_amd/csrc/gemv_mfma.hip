// Matrix-core form of the several-column product (ncols = 2..8) for the
// 16-bit and the block formats: dst[b*N + i] = epilogue((W x_b)_i, ...).
//
// "feat(cuda): fuse activations and residual add into mmv f/q epilogues",
// Summary, states the fused matrix-vector path for one destination column.
// With several columns every weight meets ncols values of x, and on the
// vector ALUs the multiply-adds, not the bytes, set the time (the 4-bit
// format crosses over at two columns).  Here the products run on the gfx950
// matrix cores instead (v_mfma_f32_16x16x32_f16, _bf16 for bf16 weights),
// and the vector ALUs keep only the unpack of the codes and the block scales.
//
// Operands of one matrix-core step (32 values of k, 16 rows):
//  * B (32 x 16) is W: lane n + 16 g holds row n's values k = 32 s + 8 g + p,
//    p = 0..7, as f16 (bf16).  16-bit weights are the loaded chunk itself;
//    8-bit codes and (code - 8) of the 4-bit format are exact in f16.
//  * A (16 x 32) is x: row m = 2 b + piece of column b.  For the f16 MFMA
//    each column is scaled by a power of two 2^(15 - e_b) (e_b the binary
//    exponent of the largest finite |x_bk|) and split into hi = f16(x') and
//    lo = f16(2^10 (x' - hi)), both rounded toward zero: every product with
//    an f16 weight is exact in f32, hi + 2^-10 lo carries x' to 2^-20
//    relative, and because lo is scaled up the f16 subnormals only limit
//    values below 2^-48 of the column's largest.  For the bf16 MFMA, hi is
//    the upper half of x and lo that of x - hi (2^-15 relative; bf16 has the
//    exponent range of f32, so nothing is scaled).  An infinite x is hi
//    alone (lo = 0) and a NaN x a NaN piece, so special values propagate as
//    in the plain product.  The pieces of every column are built once per
//    workgroup in LDS, in the A operand's lane layout.
//  * D (16 x 16): lane n + 16 g' holds row n of pieces 4 g' .. 4 g' + 3, that
//    is hi and lo of columns 2 g' and 2 g' + 1, so a column is finished
//    without lane exchange: y = (hi + 2^-10 lo) 2^(e_b - 15) (hi + lo for
//    bf16).
// For the block formats every step is one 32-code block: the step's product
// is scaled by the row's fp16 block scale into a running sum (one FMA per
// output); 16-bit weights accumulate in the matrix core across steps.
//
// Work layout: a workgroup of 16 waves owns RT tiles of 16 rows.  Waves 8..15
// build the pieces: each reads a whole column of x (for its maximum) and
// converts its share of it.  Waves 0..7 split K into KS = 8 / RT slices
// (wave w: tile w % RT, slice w / RT): they load the epilogue operands, the
// block scales and W (some of it before the pieces are ready, the rest one
// load unit ahead of its use), and run the matrix-core steps.  A wave blocks
// while the memory pipeline is full, so loading W and building the pieces
// are kept in different waves.  The slices' sums meet in LDS in a fixed
// order, so the result is deterministic; it differs from the one-column
// kernel's by rounding only.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "gemv_device.h"
#include "gemv_internal.h"

namespace gemv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4))); // x may be 4-byte aligned only
typedef unsigned u32x4u __attribute__((ext_vector_type(4), aligned(4))); // scale runs: 4-byte aligned

constexpr int kMW = 8;      // W and matrix-core waves per workgroup
constexpr int kWG = 16;     // waves per workgroup: kMW, then 8 builders of the x pieces
constexpr int kXShift = 15; // a column's largest |x| is scaled into [2^14, 2^15)
constexpr int kLoShift = 10;

// Slot e of a lane's 8 B values <-> position within its 8 consecutive k (the
// 4-bit unpack yields the codes of a dword in the order 0, 4, 1, 5, 2, 6, 3, 7).
template <int FMT> __host__ __device__ constexpr int slot_pos(int e)
{
    return FMT == GEMV_W_Q4B32 ? (e >> 1) + 4 * (e & 1) : e;
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return fmaxf(fmaxf(lane_read(v, 0), lane_read(v, 16)), fmaxf(lane_read(v, 32), lane_read(v, 48)));
}

// A column's largest finite magnitude over the VO octets of x a builder
// lane holds (octets past nocts excluded), reduced over the wave, and
// whether the column holds an infinity.  NaNs drop out of the maximum by
// themselves (fmaxf returns the other operand); an infinity would make the
// scale exponent meaningless, so such a column takes a second pass over its
// finite values.  The result is uniform across the wave.
template <int VO>
__device__ __forceinline__ float column_max(const float (&xv)[VO][8], int lane, int nocts, bool &has_inf)
{
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < VO; ++i) {
        const bool ok = lane + kWave * i < nocts;
#pragma unroll
        for (int p = 0; p < 8; ++p)
            mx = fmaxf(mx, ok ? fabsf(xv[i][p]) : 0.0f);
    }
    mx = wave_max(mx);
    has_inf = !(mx <= 3.40282347e38f);
    if (has_inf) {
        mx = 0.0f;
#pragma unroll
        for (int i = 0; i < VO; ++i) {
            const bool ok = lane + kWave * i < nocts;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const float a = fabsf(xv[i][p]);
                mx = fmaxf(mx, ok && a <= 3.40282347e38f ? a : 0.0f);
            }
        }
        mx = wave_max(mx);
    }
    return mx;
}

__device__ __forceinline__ f16x8 as_f16x8(u32x4 q) { return __builtin_bit_cast(f16x8, q); }

// 8 codes of the 4-bit format (element p in bits 4p..4p+3) -> f16 slots
// (c0-8, c4-8, c1-8, c5-8, c2-8, c6-8, c3-8, c7-8).  A nibble OR-ed into the
// mantissa of 1024 gives 1024 + c (low nibble) or 1024 + 16 c (high nibble);
// subtracting 1032, or the fused (1024 + 16 c) / 16 - 72, leaves c - 8
// exactly, two codes per packed f16 operation.
__device__ __forceinline__ f16x8 unpack_q4(unsigned d)
{
    const f16x2 off1 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const f16x2 k16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const f16x2 off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const unsigned magic = 0x64006400u;
    const unsigned e = d >> 8;
    const f16x2 h0 = __builtin_bit_cast(f16x2, and_or(d, 0x000F000Fu, magic)) - off1;
    const f16x2 h1 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, and_or(d, 0x00F000F0u, magic)), k16, off16);
    const f16x2 h2 = __builtin_bit_cast(f16x2, and_or(e, 0x000F000Fu, magic)) - off1;
    const f16x2 h3 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, and_or(e, 0x00F000F0u, magic)), k16, off16);
    u32x4 r = {__builtin_bit_cast(unsigned, h0), __builtin_bit_cast(unsigned, h1), __builtin_bit_cast(unsigned, h2),
               __builtin_bit_cast(unsigned, h3)};
    return as_f16x8(r);
}

// 4 int8 codes -> two f16 pairs: byte b ^ 0x80 = c + 128 is OR-ed into the
// mantissa of 1024 (v_perm places it and the 0x64 exponent byte), and
// 1152 is subtracted: c exactly.
__device__ __forceinline__ void unpack_q8(unsigned d, unsigned &lo, unsigned &hi)
{
    const f16x2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
    const unsigned u = d ^ 0x80808080u;
    lo = __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - off);
    hi = __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - off);
}

// 4x4 transpose of dwords across the lane groups g = lane / 16: on entry
// v[i] of group g is dword i of block g; on exit v[i] of group g is dword g
// of block i.  permlane32_swap exchanges the upper half of its first operand
// with the lower half of its second; permlane16_swap the odd 16-lane rows of
// the first with the even rows of the second.
__device__ __forceinline__ void transpose4(unsigned (&v)[4])
{
    {
        const auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
        v[0] = a[0];
        v[2] = a[1];
        const auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
        v[1] = b[0];
        v[3] = b[1];
    }
    {
        const auto a = __builtin_amdgcn_permlane16_swap(v[0], v[1], false, false);
        v[0] = a[0];
        v[1] = a[1];
        const auto b = __builtin_amdgcn_permlane16_swap(v[2], v[3], false, false);
        v[2] = b[0];
        v[3] = b[1];
    }
}

// Lane group G holds dwords 4 G .. 4 G + 3 of a row's two blocks (64 bytes);
// afterwards v[0..1] of group g are dwords 2 g, 2 g + 1 (block 0) and v[2..3]
// dwords 8 + 2 g, 9 + 2 g (block 1).  Two 2x2 exchanges: lane-group bit 0
// with the pair index, then lane-group bit 1 with it.
__device__ __forceinline__ void permute_q8(unsigned (&v)[4])
{
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const auto a = __builtin_amdgcn_permlane16_swap(v[i], v[i + 2], false, false);
        v[i] = a[0];
        v[i + 2] = a[1];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const auto a = __builtin_amdgcn_permlane32_swap(v[i], v[i + 2], false, false);
        v[i] = a[0];
        v[i + 2] = a[1];
    }
}

// W of one wave: its 16 rows (lane n + 16 g: row n) over its slice of steps,
// in load units of 16 bytes per lane.  f16: a unit is one step (lane group
// g: the step's 8 weights k = 32 s + 8 g ..).  4-bit: a unit is 4 steps
// (lane group g loads block s + g whole; transpose4 then gives every lane
// its 8 codes of each of the 4 blocks).  8-bit: a unit is 2 steps (lane
// group g loads bytes 16 g .. 16 g + 15 of the two blocks; permute_q8).
// Block scales: units of 8 consecutive fp16 (16 bytes), every lane of a row
// loading the same ones.
template <int FMT> constexpr bool is16() { return FMT == GEMV_W_F16 || FMT == GEMV_W_BF16; }
template <int FMT> constexpr int steps_per_unit() { return is16<FMT>() ? 1 : (FMT == GEMV_W_Q4B32 ? 4 : 2); }
template <int FMT> constexpr int step_bytes() { return is16<FMT>() ? 64 : (FMT == GEMV_W_Q4B32 ? 16 : 32); }

template <int FMT> constexpr int64_t scale_plane_offset(int64_t N, int64_t K)
{
    return align256_dev(N * row_bytes<FMT>(K));
}

// LDS: [pieces or slice sums][per-wave maxima].  Pieces: piece row m, octet
// o = 4 s + g (step s, lane group g) -> 16-byte slot m * (K/8 + 1) + o.  The
// odd row length in slots puts the 16 rows a matrix-core read touches in 16
// distinct bank groups, and the builders' writes (consecutive octets of one
// row) are consecutive slots.
__host__ __device__ constexpr int64_t piece_row_slots(int64_t K) { return K / 8 + 1; }
template <int NC> __host__ __device__ constexpr int64_t pieces_bytes(int64_t K) { return 2 * NC * piece_row_slots(K) * 16; }
__host__ __device__ constexpr int64_t mfma_union_bytes(int64_t pb)
{
    return pb > kMW * kWave * 16 ? pb : kMW * kWave * 16;
}

// Steps per wave slice: a whole number of scale units (8 steps) for the
// block formats.
__host__ __device__ inline int mfma_spw(int nsteps, int KS, bool block)
{
    int spw = (nsteps + KS - 1) / KS;
    return block ? (spw + 7) & ~7 : spw;
}

// The hi and lo pieces of one octet of x (v, in position order) into their
// A-layout slots: slot[0] (hi) and slot[rs] (lo).  sh: the column's scale
// exponent (unused for bf16, whose pieces are not scaled).
//
// Special values keep IEEE semantics: an infinite x is carried whole by hi
// (an infinity of f16 or bf16) with lo = 0, so that the matrix core forms
// w * inf (and 0 * inf = NaN) as the plain product would; a NaN x gives a
// NaN piece (through the plain conversions already).  The column's scale
// exponent comes from its largest finite magnitude (column_max).  For
// the f16 pieces INF selects that care: columns without an infinity (the
// builders know from the column's maximum) skip it.
template <int FMT, bool INF = true>
__device__ __forceinline__ void write_pieces(const float (&v)[8], int sh, u32x4 *slot, int rs)
{
    unsigned hw[4], lw[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        if constexpr (FMT == GEMV_W_BF16) {
            // the upper half of an infinity is the bf16 infinity itself
            const unsigned b0 = __builtin_bit_cast(unsigned, v[e]), b1 = __builtin_bit_cast(unsigned, v[e + 1]);
            const float r0 = __builtin_isinf(v[e]) ? 0.0f : v[e] - __builtin_bit_cast(float, b0 & 0xFFFF0000u);
            const float r1 = __builtin_isinf(v[e + 1]) ? 0.0f : v[e + 1] - __builtin_bit_cast(float, b1 & 0xFFFF0000u);
            hw[e / 2] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
            lw[e / 2] = __builtin_amdgcn_perm(__builtin_bit_cast(unsigned, r1), __builtin_bit_cast(unsigned, r0), 0x07060302u);
        } else {
            const float v0 = v[slot_pos<FMT>(e)], v1 = v[slot_pos<FMT>(e + 1)];
            f16x2 hp = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(ldexpf(v0, sh), ldexpf(v1, sh)));
            // converting an infinity to f16 gives the f16 infinity in any rounding mode
            const bool i0 = INF && __builtin_isinf(v0), i1 = INF && __builtin_isinf(v1);
            hp.x = i0 ? (_Float16)v0 : hp.x;
            hp.y = i1 ? (_Float16)v1 : hp.y;
            const float r0 = i0 ? 0.0f : fmaf((float)hp.x, -1024.0f, ldexpf(v0, sh + kLoShift));
            const float r1 = i1 ? 0.0f : fmaf((float)hp.y, -1024.0f, ldexpf(v1, sh + kLoShift));
            hw[e / 2] = __builtin_bit_cast(unsigned, hp);
            lw[e / 2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(r0, r1));
        }
    }
    slot[0] = u32x4{hw[0], hw[1], hw[2], hw[3]};
    slot[rs] = u32x4{lw[0], lw[1], lw[2], lw[3]};
}

// The matrix-core steps of one W load unit (SPU steps): pa[4 * s] is the A
// operand of step s; j is the unit's first step within the wave's slice,
// whose block scales sq[j / 8] holds.  16-bit weights accumulate in the
// matrix core; block formats scale each step's sums into acc.
template <int FMT>
__device__ __forceinline__ void mfma_unit(f32x4 &acc, const u32x4 &w, const u32x4 *pa, int s, int j, const u32x4 *sq)
{
    if constexpr (FMT == GEMV_W_F16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(pa[4 * s]), as_f16x8(w), acc, 0, 0, 0);
    } else if constexpr (FMT == GEMV_W_BF16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pa[4 * s]), __builtin_bit_cast(bf16x8, w),
                                                       acc, 0, 0, 0);
    } else {
        constexpr int SPU = steps_per_unit<FMT>();
        unsigned d[4] = {w.x, w.y, w.z, w.w};
        if constexpr (FMT == GEMV_W_Q4B32)
            transpose4(d);
        else
            permute_q8(d);
#pragma unroll
        for (int i = 0; i < SPU; ++i) {
            f16x8 b;
            if constexpr (FMT == GEMV_W_Q4B32) {
                b = unpack_q4(d[i]);
            } else {
                unsigned u0, u1, u2, u3;
                unpack_q8(d[2 * i], u0, u1);
                unpack_q8(d[2 * i + 1], u2, u3);
                b = as_f16x8(u32x4{u0, u1, u2, u3});
            }
            const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            const f32x4 dd = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(pa[4 * (s + i)]), b, z, 0, 0, 0);
            const int jj = j + i;
            const u32x4 sv = sq[jj / 8];
            const int k2 = (jj % 8) / 2;
            const unsigned sd = k2 == 0 ? sv.x : (k2 == 1 ? sv.y : (k2 == 2 ? sv.z : sv.w));
            const float scv = (jj & 1) ? f16hi(sd) : f16lo(sd);
            acc[0] = fmaf(scv, dd[0], acc[0]);
            acc[1] = fmaf(scv, dd[1], acc[1]);
            acc[2] = fmaf(scv, dd[2], acc[2]);
            acc[3] = fmaf(scv, dd[3], acc[3]);
        }
    }
}

template <int FMT, int NC, int SW, int VO>
__global__ __launch_bounds__(kWG *kWave) void gemv_cols_mfma_kernel(const unsigned char *W, const float *x, int N,
                                                                     int K, int RT, int act, const float *mop,
                                                                     const float *rop, float *dst)
{
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int PC = 2 * NC;    // piece rows of A
    constexpr int WPC = kMW / NC; // builder waves per column
    constexpr bool kBlock = Fmt<FMT>::kBlock;
    constexpr int SPU = steps_per_unit<FMT>();
    constexpr int NU = SW / SPU;             // W load units per lane
    // units issued before the pieces are ready (measured per format): f16
    // has nothing to do meanwhile and issues all; the 4-bit unpack is the
    // longest, and with 16 units per lane it overlaps the stream best when
    // three quarters are issued one ahead of their use (with 8, half)
    constexpr int PU = is16<FMT>() ? NU : (FMT == GEMV_W_Q4B32 ? (NU >= 16 ? NU / 4 : NU / 2) : NU / 2);
    constexpr int NSU = kBlock ? SW / 8 : 1; // scale units per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const bool wwave = w < kMW; // W and matrix-core wave; else a builder
    const int n = lane & 15, g = lane >> 4;
    const int nsteps = K / 32;
    const int KS = kMW / RT;
    const int t = w % RT, q = (w % kMW) / RT;
    const int spw = mfma_spw(nsteps, KS, kBlock);
    const int s0 = q * spw;
    const int cnt = max(0, min(spw, nsteps - s0));
    const int row0 = (blockIdx.x * RT + t) * 16;
    const int row = min(row0 + n, N - 1);
    const int rs = (int)piece_row_slots(K);

    // builders: the whole of column c (for its maximum), VO octets of 8
    // values per lane, clamped so that every load is valid; the workgroup
    // starts at an octet of its own so that the workgroups do not all read
    // the same lines at once
    const int c = (w - kMW) % NC, h = (w - kMW) / NC;
    const int nocts = K / 8;
    const int rot = (int)(((int64_t)blockIdx.x * kWave) % nocts);
    float xv[VO][8];
    if (!wwave) {
#pragma unroll
        for (int i = 0; i < VO; ++i) {
            const int o = (min(lane + kWave * i, nocts - 1) + rot) % nocts;
            const float *xp = x + (int64_t)c * K + 8 * o;
            const f32x4u a = *reinterpret_cast<const f32x4u *>(xp);
            const f32x4u b = *reinterpret_cast<const f32x4u *>(xp + 4);
            xv[i][0] = a.x, xv[i][1] = a.y, xv[i][2] = a.z, xv[i][3] = a.w;
            xv[i][4] = b.x, xv[i][5] = b.y, xv[i][6] = b.z, xv[i][7] = b.w;
        }
    }
    // the x loads are queued before any W load
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // W waves: the epilogue operands of this lane's two outputs (row, columns
    // 2g and 2g + 1; clamped indices, used only where valid), the block
    // scales and the first PU units of W
    const float *opnd = (act == GEMV_ACT_SILU_MUL || act == GEMV_ACT_MUL) ? mop : (act == GEMV_ACT_ADD ? rop : nullptr);
    float ov[2] = {0.0f, 0.0f};
    const unsigned char *wp = W + (int64_t)row * row_bytes<FMT>(K) + 16 * g;
    u32x4 wq[NU];
    u32x4 sq[NSU];
    float *wmax = reinterpret_cast<float *>(lds + mfma_union_bytes(pieces_bytes<NC>(K)));
    if (wwave) {
        if (opnd != nullptr && q == 0) {
#pragma unroll
            for (int u = 0; u < 2; ++u)
                ov[u] = opnd[(int64_t)min(2 * g + u, NC - 1) * N + row];
        }
        if constexpr (kBlock) {
            const unsigned char *sp = W + scale_plane_offset<FMT>(N, K) + (int64_t)row * (K / 32) * 2;
#pragma unroll
            for (int v = 0; v < NSU; ++v) {
                const int s = min(s0 + 8 * v, nsteps - 8);
                sq[v] = *reinterpret_cast<const u32x4u *>(sp + 2 * s);
            }
        }
#pragma unroll
        for (int u = 0; u < PU; ++u) {
            const int s = min(s0 + SPU * u, nsteps - SPU);
            wq[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wp + (int64_t)step_bytes<FMT>() * s));
        }
    } else if (FMT == GEMV_W_BF16 && h < WPC) {
        // builders (bf16 weights): x = hi + lo with hi the upper 16 bits of x
        // and lo those of x - hi (exact in f32), both bf16; no scaling, since
        // bf16 has the exponent range of f32
        const int opw = (nocts + WPC - 1) / WPC;
        const int oa = h * opw, ob = min(oa + opw, nocts);
#pragma unroll
        for (int i = 0; i < VO; ++i) {
            const int o = (lane + kWave * i + rot) % nocts;
            if (lane + kWave * i < nocts && o >= oa && o < ob)
                write_pieces<FMT>(xv[i], 0, reinterpret_cast<u32x4 *>(lds) + 2 * c * rs + o, rs);
        }
    } else if (h < WPC) {
        // builders: column maximum -> binary exponent, then hi / lo pieces
        // of this builder's share of the column into the A layout (octet
        // o is step o / 4, lane group o % 4)
        bool has_inf;
        const float mx = column_max<VO>(xv, lane, nocts, has_inf);
        int ec;
        (void)frexpf(mx, &ec);
        const int sh = kXShift - ec;
        if (lane == 0 && h == 0)
            wmax[c] = mx;
        const int opw = (nocts + WPC - 1) / WPC;
        const int oa = h * opw, ob = min(oa + opw, nocts);
#pragma unroll
        for (int i = 0; i < VO; ++i) {
            const int o = (lane + kWave * i + rot) % nocts;
            if (lane + kWave * i < nocts && o >= oa && o < ob) {
                u32x4 *slot = reinterpret_cast<u32x4 *>(lds) + 2 * c * rs + o;
                if (has_inf)
                    write_pieces<FMT, true>(xv[i], sh, slot, rs);
                else
                    write_pieces<FMT, false>(xv[i], sh, slot, rs);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();

    // W waves: the slice's steps; unit u + PU is issued before unit u is consumed
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (wwave) {
        const u32x4 *pa = reinterpret_cast<const u32x4 *>(lds) + (n % PC) * rs + g;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            if (u + PU < NU) {
                const int s = min(s0 + SPU * (u + PU), nsteps - SPU);
                wq[u + PU] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wp + (int64_t)step_bytes<FMT>() * s));
            }
            __builtin_amdgcn_sched_barrier(0);
            if (SPU * u < cnt)
                mfma_unit<FMT>(acc, wq[u], pa, s0 + SPU * u, SPU * u, sq);
        }
    }

    // slice sums meet in LDS (over the pieces, once every wave is done)
    lds_barrier();
    f32x4 *red = reinterpret_cast<f32x4 *>(lds);
    if (wwave)
        red[w * kWave + lane] = acc;
    lds_barrier();
    if (wwave && q == 0) {
        f32x4 tot = red[t * kWave + lane];
        for (int qq = 1; qq < KS; ++qq) {
            const f32x4 v = red[(t + qq * RT) * kWave + lane];
            tot[0] += v[0];
            tot[1] += v[1];
            tot[2] += v[2];
            tot[3] += v[3];
        }
        const int ro = row0 + n;
        if (ro < N) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int b = 2 * g + u;
                if (b < NC) {
                    float y;
                    if constexpr (FMT == GEMV_W_BF16) {
                        y = tot[2 * u] + tot[2 * u + 1];
                    } else {
                        int eb;
                        (void)frexpf(wmax[b], &eb);
                        y = ldexpf(fmaf(tot[2 * u + 1], 1.0f / 1024.0f, tot[2 * u]), eb - kXShift);
                    }
                    dst[(int64_t)b * N + ro] = apply_epilogue(act, y, ov[u]);
                }
            }
        }
    }
}

// Rows longer than one LDS load of pieces: K in segments of KSEG values,
// the pieces of two segments double-buffered in LDS, and one workgroup
// barrier per segment.  Each segment carries its own per-column exponent
// (its largest |x|), so a builder needs only the segment's values, which
// it prefetches one segment ahead; W waves fold each segment's sums into
// their running totals with that exponent.  In segment s, W wave q takes
// steps q * SWS .. q * SWS + SWS - 1 of the segment's KSEG / 32, and keeps
// the W of two segments in flight.
template <int NC> __host__ __device__ constexpr int64_t seg_buf_bytes(int64_t kseg)
{
    return 2 * NC * piece_row_slots(kseg) * 16;
}

template <int FMT, int NC, int SWS>
__global__ __launch_bounds__(kWG *kWave) void gemv_cols_mfma_seg_kernel(const unsigned char *W, const float *x,
                                                                         int N, int K, int RT, int KSEG, int act,
                                                                         const float *mop, const float *rop,
                                                                         float *dst)
{
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int PC = 2 * NC;
    constexpr int WPC = kMW / NC;
    constexpr bool kBlock = Fmt<FMT>::kBlock;
    constexpr int SPU = steps_per_unit<FMT>();
    constexpr int SU = SWS / SPU;              // W load units per lane per segment
    constexpr int SSU = kBlock ? SWS / 8 : 1;  // scale units per lane per segment
    constexpr int VO = 4;                      // x octets per builder lane per segment (KSEG <= 2048)
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const bool wwave = w < kMW;
    const int n = lane & 15, g = lane >> 4;
    const int t = w % RT, q = (w % kMW) / RT;
    const int nseg = K / KSEG, ss = KSEG / 32;
    const int row0 = (blockIdx.x * RT + t) * 16;
    const int row = min(row0 + n, N - 1);
    const int rs = (int)piece_row_slots(KSEG);
    const int64_t bufb = seg_buf_bytes<NC>(KSEG);
    float *smax = reinterpret_cast<float *>(lds + 2 * bufb); // [2][NC]

    // builders: segment s of column c in registers (VO octets per lane,
    // clamped), rotated per workgroup
    const int c = (w - kMW) % NC, h = (w - kMW) / NC;
    const bool builder = !wwave && h < WPC;
    const int nocts = KSEG / 8;
    const int rot = (int)(((int64_t)blockIdx.x * kWave) % nocts);
    float xa[VO][8], xb[VO][8];
    auto load_x = [&](float (&xv)[VO][8], int sg) {
#pragma unroll
        for (int i = 0; i < VO; ++i) {
            const int o = (min(lane + kWave * i, nocts - 1) + rot) % nocts;
            const float *xp = x + (int64_t)c * K + (int64_t)sg * KSEG + 8 * o;
            const f32x4u a = *reinterpret_cast<const f32x4u *>(xp);
            const f32x4u b = *reinterpret_cast<const f32x4u *>(xp + 4);
            xv[i][0] = a.x, xv[i][1] = a.y, xv[i][2] = a.z, xv[i][3] = a.w;
            xv[i][4] = b.x, xv[i][5] = b.y, xv[i][6] = b.z, xv[i][7] = b.w;
        }
    };
    auto build = [&](const float (&xv)[VO][8], int pb) {
        int sh = 0;
        bool has_inf = true; // bf16 pieces always take the care (they have no maximum)
        if constexpr (FMT != GEMV_W_BF16) {
            const float mx = column_max<VO>(xv, lane, nocts, has_inf);
            int ec;
            (void)frexpf(mx, &ec);
            sh = kXShift - ec;
            if (lane == 0 && h == 0)
                smax[pb * NC + c] = mx;
        }
        const int opw = (nocts + WPC - 1) / WPC;
        const int oa = h * opw, ob = min(oa + opw, nocts);
#pragma unroll
        for (int i = 0; i < VO; ++i) {
            const int o = (lane + kWave * i + rot) % nocts;
            if (lane + kWave * i < nocts && o >= oa && o < ob) {
                u32x4 *slot = reinterpret_cast<u32x4 *>(lds + pb * bufb) + 2 * c * rs + o;
                if (has_inf)
                    write_pieces<FMT, true>(xv[i], sh, slot, rs);
                else
                    write_pieces<FMT, false>(xv[i], sh, slot, rs);
            }
        }
    };

    // W waves: W of segment s, this wave's SWS steps
    const unsigned char *wp = W + (int64_t)row * row_bytes<FMT>(K) + 16 * g;
    const unsigned char *sp = W + scale_plane_offset<FMT>(N, K) + (int64_t)row * (K / 32) * 2;
    u32x4 wa[SU], wb[SU], sa[SSU], sb[SSU];
    auto issue = [&](u32x4 (&wq)[SU], u32x4 (&sq)[SSU], int sg) {
        const int sbase = sg * ss + q * SWS;
        if constexpr (kBlock) {
#pragma unroll
            for (int v = 0; v < SSU; ++v)
                sq[v] = *reinterpret_cast<const u32x4u *>(sp + 2 * (sbase + 8 * v));
        }
#pragma unroll
        for (int u = 0; u < SU; ++u)
            wq[u] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(wp + (int64_t)step_bytes<FMT>() * (sbase + SPU * u)));
    };
    float tot[2] = {0.0f, 0.0f};
    auto consume = [&](const u32x4 (&wq)[SU], const u32x4 (&sq)[SSU], int pb) {
        const u32x4 *pa = reinterpret_cast<const u32x4 *>(lds + pb * bufb) + (n % PC) * rs + g;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < SU; ++u)
            mfma_unit<FMT>(acc, wq[u], pa, q * SWS + SPU * u, SPU * u, sq);
        // fold the segment into the totals of this lane's two columns
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if constexpr (FMT == GEMV_W_BF16) {
                tot[u] += acc[2 * u] + acc[2 * u + 1];
            } else {
                int eb;
                (void)frexpf(smax[pb * NC + min(2 * g + u, NC - 1)], &eb);
                tot[u] += ldexpf(fmaf(acc[2 * u + 1], 1.0f / 1024.0f, acc[2 * u]), eb - kXShift);
            }
        }
    };

    // The two roles run separate loops with the same sequence of barriers
    // (so that each role's registers are live only in its own loop): x of
    // segments 0 and 1 is queued before any W load; then one barrier per
    // segment: segment s's pieces are ready, and segment s - 1's buffer is free.
    if (wwave) {
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const float *opnd = (act == GEMV_ACT_SILU_MUL || act == GEMV_ACT_MUL) ? mop : (act == GEMV_ACT_ADD ? rop : nullptr);
        float ov[2] = {0.0f, 0.0f};
        if (opnd != nullptr && q == 0) {
#pragma unroll
            for (int u = 0; u < 2; ++u)
                ov[u] = opnd[(int64_t)min(2 * g + u, NC - 1) * N + row];
        }
        issue(wa, sa, 0);
        if (nseg > 1)
            issue(wb, sb, 1);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        // segment s: consume it, then issue segment s + 2 into its registers
        for (int sg = 0; sg < nseg; sg += 2) {
            consume(wa, sa, 0);
            if (sg + 2 < nseg)
                issue(wa, sa, sg + 2);
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
            if (sg + 1 < nseg) {
                consume(wb, sb, 1);
                if (sg + 3 < nseg)
                    issue(wb, sb, sg + 3);
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier();
            }
        }
        // the slices' totals meet in LDS
        float2 *red = reinterpret_cast<float2 *>(lds);
        red[w * kWave + lane] = float2{tot[0], tot[1]};
        lds_barrier();
        if (q == 0) {
            const int KS = kMW / RT;
            float2 sum = red[t * kWave + lane];
            for (int qq = 1; qq < KS; ++qq) {
                const float2 v = red[(t + qq * RT) * kWave + lane];
                sum.x += v.x;
                sum.y += v.y;
            }
            const int ro = row0 + n;
            if (ro < N) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int b = 2 * g + u;
                    if (b < NC)
                        dst[(int64_t)b * N + ro] = apply_epilogue(act, u ? sum.y : sum.x, ov[u]);
                }
            }
        }
    } else {
        if (builder) {
            load_x(xa, 0);
            if (nseg > 1)
                load_x(xb, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        if (builder)
            build(xa, 0);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        // during segment s: prefetch x of s + 2, build the pieces of s + 1
        for (int sg = 0; sg < nseg; sg += 2) {
            if (builder) {
                if (sg + 2 < nseg)
                    load_x(xa, sg + 2);
                if (sg + 1 < nseg)
                    build(xb, 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
            if (sg + 1 < nseg) {
                if (builder) {
                    if (sg + 3 < nseg)
                        load_x(xb, sg + 3);
                    if (sg + 2 < nseg)
                        build(xa, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                lds_barrier();
            }
        }
        lds_barrier(); // the slices' totals are written
    }
}

template <int FMT, int NC, int SWS> int launch_mfma_seg(const ColsArgs &c, int RT, int kseg, hipStream_t s)
{
    const void *fn = reinterpret_cast<const void *>(&gemv_cols_mfma_seg_kernel<FMT, NC, SWS>);
    const int64_t lds = 2 * seg_buf_bytes<NC>(kseg) + 2 * NC * 4;
    if (lds > 64 * 1024) {
        static std::once_flag once;
        static hipError_t attr_err = hipSuccess;
        std::call_once(once, [&] { attr_err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds); });
        if (attr_err != hipSuccess)
            return (int)attr_err;
    }
    const int grid = (c.N + 16 * RT - 1) / (16 * RT);
    const unsigned char *W = c.W;
    const float *x = c.x;
    int N = c.N, K = c.K, rt = RT, ks = kseg, act = c.act;
    const float *m = c.m, *r = c.r;
    float *dst = c.dst;
    void *args[] = {&W, &x, &N, &K, &rt, &ks, &act, &m, &r, &dst};
    return (int)hipLaunchKernel(fn, dim3(grid), dim3(kWG * kWave), args, (size_t)lds, s);
}

template <int FMT, int NC, int SW, int VO> int launch_mfma(const ColsArgs &c, int RT, hipStream_t s)
{
    const void *fn = reinterpret_cast<const void *>(&gemv_cols_mfma_kernel<FMT, NC, SW, VO>);
    const int64_t lds = mfma_union_bytes(pieces_bytes<NC>(c.K)) + kMW * 4;
    if (lds > 64 * 1024) {
        static std::once_flag once;
        static hipError_t attr_err = hipSuccess;
        std::call_once(once, [&] { attr_err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds); });
        if (attr_err != hipSuccess)
            return (int)attr_err;
    }
    const int grid = (c.N + 16 * RT - 1) / (16 * RT);
    const unsigned char *W = c.W;
    const float *x = c.x;
    int N = c.N, K = c.K, rt = RT, act = c.act;
    const float *m = c.m, *r = c.r;
    float *dst = c.dst;
    void *args[] = {&W, &x, &N, &K, &rt, &act, &m, &r, &dst};
    return (int)hipLaunchKernel(fn, dim3(grid), dim3(kWG * kWave), args, (size_t)lds, s);
}

// Where the matrix-core kernel is taken instead of the vector-ALU column
// kernel (measured on the decode shapes).  Its fixed cost (x read and split
// per workgroup, then the unpack after the pieces are ready) is about 4-6 us
// over the weight stream, while the vector-ALU kernel's time grows with
// every column once the multiply-adds outrun the stream.  f16/bf16: from
// five columns where 4096 <= K <= 6144 (one segment), from seven on
// shorter or segmented rows.  8-bit: from
// four where the matrix is 20 MB or more and the tiles make one round of
// workgroups, from six on 32 MB or more.  4-bit: from three on 16 MB or
// more, from six on smaller matrices.
bool mfma_wins(int wfmt, int NC, int64_t K, int64_t tiles, int64_t cus, int64_t wbytes)
{
    const int64_t MB = 1 << 20;
    if (wfmt == GEMV_W_F16 || wfmt == GEMV_W_BF16)
        return NC >= (K >= 4096 && K <= 6144 ? 5 : 7);
    if (wfmt == GEMV_W_Q8B32)
        return (NC >= 4 && wbytes >= 20 * MB && tiles <= cus) || (NC >= 6 && wbytes >= 32 * MB);
    return NC >= (wbytes >= 16 * MB ? 3 : 6);
}

int64_t row_bytes_of(int wfmt, int64_t K)
{
    return (wfmt == GEMV_W_F16 || wfmt == GEMV_W_BF16) ? 2 * K : (wfmt == GEMV_W_Q8B32 ? K : K / 2);
}

template <int FMT, int NC, int SW> int launch_mfma_vo(const ColsArgs &c, const MfmaPlan &p, hipStream_t s)
{
    if (p.vo <= 4)
        return launch_mfma<FMT, NC, SW, 4>(c, p.rt, s);
    if (p.vo <= 8)
        return launch_mfma<FMT, NC, SW, 8>(c, p.rt, s);
    return launch_mfma<FMT, NC, SW, 12>(c, p.rt, s);
}

template <int FMT, int NC> int launch_mfma_plan(const ColsArgs &c, const MfmaPlan &p, hipStream_t s)
{
    if (p.kseg)
        return launch_mfma_seg<FMT, NC, 8>(c, p.rt, p.kseg, s);
    constexpr int SW1 = Fmt<FMT>::kBlock ? 32 : 16;
    if constexpr (FMT == GEMV_W_Q4B32) {
        if (p.sw > SW1)
            return launch_mfma_vo<FMT, NC, 2 * SW1>(c, p, s);
    }
    return launch_mfma_vo<FMT, NC, SW1>(c, p, s);
}

template <int NC> int launch_mfma_fmt(int wfmt, const ColsArgs &c, const MfmaPlan &p, hipStream_t s)
{
    switch (wfmt) {
    case GEMV_W_F16:
        return launch_mfma_plan<GEMV_W_F16, NC>(c, p, s);
    case GEMV_W_BF16:
        return launch_mfma_plan<GEMV_W_BF16, NC>(c, p, s);
    case GEMV_W_Q8B32:
        return launch_mfma_plan<GEMV_W_Q8B32, NC>(c, p, s);
    default:
        return launch_mfma_plan<GEMV_W_Q4B32, NC>(c, p, s);
    }
}

} // namespace

// Tiles per workgroup (rt): the fewest that make the grid a single round on
// the compute units, as long as a W wave's slice fits its registers (sw
// steps: 16 for f16/bf16, which then need one tile per workgroup; 32 for the
// 8-bit format; 32 or 64 for the 4-bit format); otherwise fewer.  The shape
// must also fit: K a whole number of steps (of scale units, 256 values, for
// the block formats), a column within a builder's registers (K <= 6144),
// the pieces within LDS.
MfmaPlan cols_mfma_plan(int wfmt, int ncols, int64_t N, int64_t K, int64_t cus)
{
    MfmaPlan p{0, 0, 0, 0};
    if (wfmt == GEMV_W_F32 || wfmt < 0 || wfmt > GEMV_W_Q4B32 || ncols < 2 || ncols > 8 || N < 1)
        return p;
    const bool block = wfmt == GEMV_W_Q8B32 || wfmt == GEMV_W_Q4B32;
    if (K < 1 || K % (block ? 256 : 32) != 0 || K >= GEMV_MAX_DIM_EXTENT)
        return p;
    const int64_t tiles = (N + 15) / 16;
    if (!mfma_wins(wfmt, ncols, K, tiles, cus, N * row_bytes_of(wfmt, K)))
        return p;
    int rt1 = 1; // tiles per workgroup for one round of workgroups
    while (rt1 < kMW && tiles > cus * rt1)
        rt1 *= 2;
    // the whole row as one segment
    if (K <= kWave * 8 * 12 && mfma_union_bytes(2 * ncols * piece_row_slots(K) * 16) + kMW * 4 <= kMaxLds) {
        const int sw1 = block ? 32 : 16;
        const int swmax = wfmt == GEMV_W_Q4B32 ? 64 : sw1;
        for (int rt = rt1; rt >= 1; rt /= 2) {
            const int spw = mfma_spw((int)(K / 32), kMW / rt, block);
            if (!block && tiles > cus)
                break;
            if (spw <= swmax) {
                const int64_t vo = (K / 8 + kWave - 1) / kWave; // x octets per builder lane
                p = MfmaPlan{rt, spw <= sw1 ? sw1 : swmax, vo <= 4 ? 4 : (vo <= 8 ? 8 : 12), 0};
                return p;
            }
        }
        return p;
    }
    // segments of kseg = 2048 / rt values, so that every W wave takes 8 steps
    // of each segment (more would not fit its registers beside the second
    // segment in flight); kseg must divide K and two piece buffers fit LDS
    for (int rt = rt1; rt >= 1; rt /= 2) {
        const int kseg = 2048 / rt;
        if (!block && tiles > cus * rt)
            continue;
        if (K % kseg != 0 || 2 * (2 * ncols * piece_row_slots(kseg) * 16) + 2 * ncols * 4 > kMaxLds)
            continue;
        p = MfmaPlan{rt, 8, 4, kseg};
        return p;
    }
    return p;
}

int launch_cols_mfma(int wfmt, int ncols, const ColsArgs &c, void *stream)
{
    const MfmaPlan p = cols_mfma_plan(wfmt, ncols, c.N, c.K, device_cus());
    if (!p.rt)
        return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (ncols) {
    case 2:
        return launch_mfma_fmt<2>(wfmt, c, p, s);
    case 3:
        return launch_mfma_fmt<3>(wfmt, c, p, s);
    case 4:
        return launch_mfma_fmt<4>(wfmt, c, p, s);
    case 5:
        return launch_mfma_fmt<5>(wfmt, c, p, s);
    case 6:
        return launch_mfma_fmt<6>(wfmt, c, p, s);
    case 7:
        return launch_mfma_fmt<7>(wfmt, c, p, s);
    default:
        return launch_mfma_fmt<8>(wfmt, c, p, s);
    }
}

} // namespace gemv

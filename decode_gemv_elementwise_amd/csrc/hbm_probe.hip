// Measurement kernels for the benchmark: a read-only streaming probe and a
// plain copy (see include/hbm_probe.h).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemv_device.h"
#include "hbm_probe.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4 *__restrict__ a, int64_t n16, float *out)
{
    float s = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        u32x4 v = __builtin_nontemporal_load(a + i);
        unsigned d[4] = {v.x, v.y, v.z, v.w};
        s += (__builtin_bit_cast(float, d[0]) + __builtin_bit_cast(float, d[1])) +
             (__builtin_bit_cast(float, d[2]) + __builtin_bit_cast(float, d[3]));
    }
    __shared__ float red[256];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w)
            red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        out[blockIdx.x] = red[0];
}

// One pass, no loop: wave w reads the 8 KiB at [8 KiB w, 8 KiB (w+1)) of the
// buffer, lane l the 16-byte pieces l, l + 64, ..., l + 448 of it, all issued
// before any is used (indices past the end are clamped to the last piece).
// The sum is stored only if it equals a value it never takes, which keeps
// the loads without writing anything.
constexpr int kOnceLoads = 8;
__global__ __launch_bounds__(256) void read_once_kernel(const u32x4 *__restrict__ a, int64_t n16, float *out)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t base = wave * 64 * kOnceLoads;
    u32x4 v[kOnceLoads];
#pragma unroll
    for (int u = 0; u < kOnceLoads; ++u) {
        const int64_t i = base + lane + 64 * u;
        v[u] = __builtin_nontemporal_load(a + (i < n16 ? i : n16 - 1));
    }
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < kOnceLoads; ++u)
        s += __builtin_bit_cast(float, v[u].x) + __builtin_bit_cast(float, v[u].w);
    if (s == -1234.5f)
        out[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *__restrict__ a, u32x4 *__restrict__ b, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        b[i] = a[i];
}

// Floor probes of other launch shapes: every wave stores one result, so each
// is a read of the bytes plus what a GEMV launch must end with.  One pass
// (every wave issues its L loads per lane at once, NW waves per workgroup),
// or a resident grid whose waves walk units of 64 L pieces.
template <int L, int NW>
__global__ __launch_bounds__(NW * 64) void floor_once_kernel(const u32x4 *__restrict__ a, int64_t n16, float *out)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * NW + (threadIdx.x >> 6);
    const int64_t base = wave * 64 * L;
    u32x4 v[L];
#pragma unroll
    for (int u = 0; u < L; ++u) {
        const int64_t i = base + lane + 64 * u;
        v[u] = __builtin_nontemporal_load(a + (i < n16 ? i : n16 - 1));
    }
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < L; ++u)
        s += __builtin_bit_cast(float, v[u].x) + __builtin_bit_cast(float, v[u].w);
    for (int o = 32; o > 0; o >>= 1)
        s += __shfl_xor(s, o);
    if (lane == 0)
        out[wave] = s;
}

template <int L, int NW>
__global__ __launch_bounds__(NW * 64) void floor_resident_kernel(const u32x4 *__restrict__ a, int64_t n16, float *out)
{
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * NW;
    const int64_t wave = (int64_t)blockIdx.x * NW + (threadIdx.x >> 6);
    const int64_t per = 64 * L;
    const int64_t nunits = (n16 + per - 1) / per;
    float s = 0.0f;
    for (int64_t t = wave; t < nunits; t += nwaves) {
        u32x4 v[L];
#pragma unroll
        for (int u = 0; u < L; ++u) {
            const int64_t i = t * per + lane + 64 * u;
            v[u] = __builtin_nontemporal_load(a + (i < n16 ? i : n16 - 1));
        }
#pragma unroll
        for (int u = 0; u < L; ++u)
            s += __builtin_bit_cast(float, v[u].x) + __builtin_bit_cast(float, v[u].w);
    }
    for (int o = 32; o > 0; o >>= 1)
        s += __shfl_xor(s, o);
    if (lane == 0)
        out[wave] = s;
}

constexpr int kFloorShapes = 3;

struct FloorShape {
    const void *fn;
    int waves, loads;
    bool resident;
};

FloorShape floor_shape(int shape)
{
    switch (shape) {
    case 0:
        return {reinterpret_cast<const void *>(&floor_once_kernel<8, 4>), 4, 8, false};
    case 1:
        return {reinterpret_cast<const void *>(&floor_once_kernel<4, 16>), 16, 4, false};
    default:
        return {reinterpret_cast<const void *>(&floor_resident_kernel<4, 16>), 16, 4, true};
    }
}

int device_cu_count()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

int64_t floor_grid(int64_t nbytes, const FloorShape &f)
{
    if (f.resident)
        return 2 * (int64_t)device_cu_count();
    const int64_t n16 = nbytes / 16;
    const int64_t waves = (n16 + 64 * f.loads - 1) / (64 * f.loads);
    return (waves + f.waves - 1) / f.waves;
}

// The one-column kernels' arithmetic alone: per row, U chunks of 16 bytes
// decoded and multiplied into f32 sums exactly as the GEMV does (the same
// Fmt<>::dot), then the wave reduction, one row per wave in 8-wave
// workgroups; the 16-byte words are made from the lane and row numbers in
// registers, so no W byte is read.  Its launch time is the floor the vector
// ALUs set for a call of that shape.
template <int FMT>
__global__ __launch_bounds__(512) void valu_floor_kernel(const float *__restrict__ x, int N, int U, float *out)
{
    using F = gemv::Fmt<FMT>;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 8 + (threadIdx.x >> 6);
    float xv[F::E];
#pragma unroll
    for (int i = 0; i < F::E; ++i)
        xv[i] = x[(lane + i) & 63];
    float acc = 0.0f;
    for (int u = 0; u < U; ++u) {
        const unsigned s = (unsigned)lane * 0x01010101u + (unsigned)u * 0x11111111u + (unsigned)row;
        const u32x4 q = {s & 0x3F7F7F7Fu, (s ^ 0x5A5A5A5Au) & 0x3F7F7F7Fu, (s + 0x12345678u) & 0x3F7F7F7Fu,
                         (s * 3u) & 0x3F7F7F7Fu};
        if constexpr (F::kBlock)
            acc = F::dot(q, xv, (_Float16)0.01f, acc);
        else
            acc = F::dot(q, xv, acc);
    }
    const float t = gemv::wave_sum(acc);
    if (lane == 0 && row < N)
        out[row] = t;
}

bool ok16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

} // namespace

extern "C" {

int hbm_read_probe(const void *buf, int64_t nbytes, float *out, int blocks, void *hip_stream)
{
    if (!buf || !out || nbytes <= 0 || nbytes % 16 || !ok16(buf) || blocks < 1 || blocks > (1 << 20))
        return -1;
    int64_t n16 = nbytes / 16;
    const u32x4 *a = static_cast<const u32x4 *>(buf);
    void *args[] = {&a, &n16, &out};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&read_probe_kernel), dim3(blocks), dim3(256), args,
                                   0, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? 0 : (int)e;
}

int hbm_read_once_blocks(int64_t nbytes) { return nbytes <= 0 ? -1 : (int)((nbytes / 16 + 64 * kOnceLoads * 4 - 1) / (64 * kOnceLoads * 4)); }

int hbm_read_once(const void *buf, int64_t nbytes, float *out, void *hip_stream)
{
    if (!buf || !out || nbytes <= 0 || nbytes % 16 || !ok16(buf) || nbytes > (int64_t(1) << 40))
        return -1;
    int64_t n16 = nbytes / 16;
    const u32x4 *a = static_cast<const u32x4 *>(buf);
    void *args[] = {&a, &n16, &out};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&read_once_kernel), dim3(hbm_read_once_blocks(nbytes)),
                                   dim3(256), args, 0, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? 0 : (int)e;
}

int hbm_copy(const void *src, void *dst, int64_t nbytes, void *hip_stream)
{
    if (!src || !dst || nbytes <= 0 || nbytes % 16 || !ok16(src) || !ok16(dst))
        return -1;
    const char *s = static_cast<const char *>(src);
    char *d = static_cast<char *>(dst);
    if (s < d + nbytes && d < s + nbytes)
        return -1;
    int64_t n16 = nbytes / 16;
    int64_t want = (n16 + 255) / 256;
    int blocks = (int)(want < 8192 ? want : 8192);
    const u32x4 *a = static_cast<const u32x4 *>(src);
    u32x4 *b = static_cast<u32x4 *>(dst);
    void *args[] = {&a, &b, &n16};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&copy_kernel), dim3(blocks), dim3(256), args, 0,
                                   static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? 0 : (int)e;
}

int hbm_read_floor_shapes(void) { return kFloorShapes; }

int64_t hbm_read_floor_out_floats(int64_t nbytes, int shape)
{
    if (nbytes <= 0 || shape < 0 || shape >= kFloorShapes)
        return -1;
    const FloorShape f = floor_shape(shape);
    return floor_grid(nbytes, f) * f.waves;
}

int hbm_read_floor(const void *buf, int64_t nbytes, float *out, int shape, void *hip_stream)
{
    if (!buf || !out || nbytes <= 0 || nbytes % 16 || !ok16(buf) || nbytes > (int64_t(1) << 40) || shape < 0 ||
        shape >= kFloorShapes)
        return -1;
    const FloorShape f = floor_shape(shape);
    int64_t n16 = nbytes / 16;
    const u32x4 *a = static_cast<const u32x4 *>(buf);
    void *args[] = {&a, &n16, &out};
    hipError_t e = hipLaunchKernel(f.fn, dim3((unsigned)floor_grid(nbytes, f)), dim3(f.waves * 64), args, 0,
                                   static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? 0 : (int)e;
}

int gemv_valu_floor(int wfmt, int64_t N, int64_t K, const float *x, float *out, void *hip_stream)
{
    static const int kE[] = {4, 8, 8, 16, 32};
    if (!x || !out || wfmt < GEMV_W_F32 || wfmt > GEMV_W_Q4B32 || N < 1 || K < 1 || N > (int64_t(1) << 30) ||
        K > (int64_t(1) << 30))
        return -1;
    const int64_t nchunks = (K + kE[wfmt] - 1) / kE[wfmt];
    int U = (int)((nchunks + 63) / 64), n = (int)N;
    const void *fn = nullptr;
    switch (wfmt) {
    case GEMV_W_F32:
        fn = reinterpret_cast<const void *>(&valu_floor_kernel<GEMV_W_F32>);
        break;
    case GEMV_W_F16:
        fn = reinterpret_cast<const void *>(&valu_floor_kernel<GEMV_W_F16>);
        break;
    case GEMV_W_BF16:
        fn = reinterpret_cast<const void *>(&valu_floor_kernel<GEMV_W_BF16>);
        break;
    case GEMV_W_Q8B32:
        fn = reinterpret_cast<const void *>(&valu_floor_kernel<GEMV_W_Q8B32>);
        break;
    default:
        fn = reinterpret_cast<const void *>(&valu_floor_kernel<GEMV_W_Q4B32>);
        break;
    }
    void *args[] = {&x, &n, &U, &out};
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)((N + 7) / 8)), dim3(512), args, 0,
                                   static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? 0 : (int)e;
}

} // extern "C"

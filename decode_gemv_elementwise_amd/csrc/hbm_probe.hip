// Measurement kernels for the benchmark: a read-only streaming probe and a
// plain copy (see include/hbm_probe.h).
#include <hip/hip_runtime.h>

#include <cstdint>

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

// The same one-pass read, then what every GEMV ends with: one 4-byte store
// per wave (the wave's sum, reduced over its lanes so that every lane's loads
// are used), to out[wave].  A launch ends only when its stores are
// acknowledged, so this is the floor for a kernel that reads the bytes and
// writes one result per wave.
__global__ __launch_bounds__(256) void read_once_store_kernel(const u32x4 *__restrict__ a, int64_t n16, float *out)
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
    for (int o = 32; o > 0; o >>= 1)
        s += __shfl_xor(s, o);
    if (lane == 0)
        out[wave] = s;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *__restrict__ a, u32x4 *__restrict__ b, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        b[i] = a[i];
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

int hbm_read_once_store(const void *buf, int64_t nbytes, float *out, void *hip_stream)
{
    if (!buf || !out || nbytes <= 0 || nbytes % 16 || !ok16(buf) || nbytes > (int64_t(1) << 40))
        return -1;
    int64_t n16 = nbytes / 16;
    const u32x4 *a = static_cast<const u32x4 *>(buf);
    void *args[] = {&a, &n16, &out};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&read_once_store_kernel),
                                   dim3(hbm_read_once_blocks(nbytes)), dim3(256), args, 0,
                                   static_cast<hipStream_t>(hip_stream));
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

} // extern "C"

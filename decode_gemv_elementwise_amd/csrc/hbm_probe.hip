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

// qk_probe.hip — measurement probes run next to the GEMVs in the same run:
// * a streaming read: the HBM read rate a plain kernel reaches on this
//   device. Every byte of the buffer is read once with 16-byte loads, several
//   in flight per lane; the XOR of all words is written per workgroup so that
//   nothing is optimised away.
// * a plain copy of known size, whose hardware counters (bytes fetched from
//   and written to HBM) calibrate the counters taken on the GEMV kernels.
#include "../../include/qk_probe.h"
#include "qk_formats.h"

namespace {

__global__ __launch_bounds__(256) void read_probe_kernel(const qk::u32x4 *__restrict__ p, int64_t n16,
                                                         uint32_t *__restrict__ out) {
    constexpr int UNROLL = 8;
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
        qk::u32x4 v[UNROLL];
#pragma unroll
        for (int k = 0; k < UNROLL; k++) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
        for (int k = 0; k < UNROLL; k++) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (; i < n16; i += stride) {
        const qk::u32x4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int m = 32; m > 0; m >>= 1) acc ^= __shfl_xor(acc, m);
    __shared__ uint32_t s[4];
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

__global__ __launch_bounds__(256) void copy_probe_kernel(const qk::u32x4 *__restrict__ src,
                                                        qk::u32x4 *__restrict__ dst, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

int cu_count() {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    return cus > 0 ? cus : 256;
}

}  // namespace

extern "C" int qk_probe_copy(const void *src, void *dst, int64_t bytes, void *stream) {
    if (!src || !dst || bytes <= 0 || (bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return -1;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (s0 < d0 + (uintptr_t)bytes && d0 < s0 + (uintptr_t)bytes) return -1;  // overlapping buffers
    const int64_t grid = (int64_t)cu_count() * 8;
    hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const qk::u32x4 *>(src), static_cast<qk::u32x4 *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int qk_probe_read(const void *buf, int64_t bytes, uint32_t *out, int64_t out_len, void *stream) {
    if (!buf || !out || bytes <= 0 || (bytes & 15) || ((uintptr_t)buf & 15) || out_len < 1) return -1;
    int64_t grid = (int64_t)cu_count() * 8;
    if (grid > out_len) grid = out_len;
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const qk::u32x4 *>(buf), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// qk_dequant.hip — qk_dequantize_row: blocks -> fp32, bit-exact.
//
// One thread writes four consecutive weights (one 16-byte store), so the
// fp32 output — the dominant traffic, 4 bytes per weight against at most
// 1.125 bytes read — is written fully coalesced. Built with
// -ffp-contract=off; decode4 also uses explicit round-to-nearest operations.
#include "qk_decode.h"
#include "qk_launch.h"

namespace qk {

template <int F>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ blocks, int64_t n4,
                                                      float *__restrict__ out) {
    constexpr int QK = Layout<F>::QK, BYTES = Layout<F>::BYTES;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n4;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = 4 * t;
        const int64_t b = i / QK;
        float w[4];
        decode4<F>(blocks + b * BYTES, (int)(i % QK), w);
        if (((uintptr_t)out & 15u) == 0) {
            *reinterpret_cast<float4 *>(out + i) = make_float4(w[0], w[1], w[2], w[3]);
        } else {
            out[i] = w[0];
            out[i + 1] = w[1];
            out[i + 2] = w[2];
            out[i + 3] = w[3];
        }
    }
}

hipError_t launch_dequant(int type, const void *blocks, int64_t n, float *out, hipStream_t stream) {
    const int64_t n4 = n / 4;
    const int threads = 256;
    int64_t grid = (n4 + threads - 1) / threads;
    if (grid > 65536) grid = 65536;
    const uint8_t *src = static_cast<const uint8_t *>(blocks);
    switch (type) {
    case Q4_K: hipLaunchKernelGGL(dequant_kernel<Q4_K>, dim3((unsigned)grid), dim3(threads), 0, stream, src, n4, out); break;
    case Q6_K: hipLaunchKernelGGL(dequant_kernel<Q6_K>, dim3((unsigned)grid), dim3(threads), 0, stream, src, n4, out); break;
    case Q8_0: hipLaunchKernelGGL(dequant_kernel<Q8_0>, dim3((unsigned)grid), dim3(threads), 0, stream, src, n4, out); break;
    case Q4_0: hipLaunchKernelGGL(dequant_kernel<Q4_0>, dim3((unsigned)grid), dim3(threads), 0, stream, src, n4, out); break;
    case Q8_0_F16: hipLaunchKernelGGL(dequant_kernel<Q8_0_F16>, dim3((unsigned)grid), dim3(threads), 0, stream, src, n4, out); break;
    case Q5_1: hipLaunchKernelGGL(dequant_kernel<Q5_1>, dim3((unsigned)grid), dim3(threads), 0, stream, src, n4, out); break;
    case Q5_K: hipLaunchKernelGGL(dequant_kernel<Q5_K>, dim3((unsigned)grid), dim3(threads), 0, stream, src, n4, out); break;
    case Q2_K: hipLaunchKernelGGL(dequant_kernel<Q2_K>, dim3((unsigned)grid), dim3(threads), 0, stream, src, n4, out); break;
    case Q3_K: hipLaunchKernelGGL(dequant_kernel<Q3_K>, dim3((unsigned)grid), dim3(threads), 0, stream, src, n4, out); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qk

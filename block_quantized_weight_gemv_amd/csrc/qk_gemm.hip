// qk_gemm.hip — Y = X W^T for M activation rows (bf16 X, fp32 Y).
//
// Batched path: one wave per weight row; lanes walk the row four weights at a
// time with the bit-exact decoder and accumulate up to MB activation rows at
// once, so W is streamed once per MB rows of X.
#include "qk_decode.h"
#include "qk_launch.h"

namespace qk {

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }

template <int F, int MB>
__global__ __launch_bounds__(256) void gemm_rows_kernel(const uint8_t *__restrict__ W, int64_t rows, int64_t cols,
                                                        int64_t row_bytes, const uint16_t *__restrict__ X,
                                                        int64_t M, float *__restrict__ Y) {
    constexpr int QK = Layout<F>::QK, BYTES = Layout<F>::BYTES;
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t mchunks = (M + MB - 1) / MB;
    for (int64_t job = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); job < rows * mchunks;
         job += nwaves) {
        const int64_t r = job % rows, m0 = (job / rows) * MB;
        const uint8_t *row = W + r * row_bytes;
        float acc[MB];
#pragma unroll
        for (int m = 0; m < MB; m++) acc[m] = 0.f;
        for (int64_t c = 4 * (int64_t)lane; c < cols; c += 256) {
            float w[4];
            decode4<F>(row + (c / QK) * BYTES, (int)(c % QK), w);
#pragma unroll
            for (int m = 0; m < MB; m++) {
                if (m0 + m < M) {
                    const uint2 xv = *reinterpret_cast<const uint2 *>(X + (m0 + m) * cols + c);
                    acc[m] += w[0] * bf16_lo(xv.x) + w[1] * bf16_hi(xv.x) + w[2] * bf16_lo(xv.y) +
                              w[3] * bf16_hi(xv.y);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MB; m++) {
            float a = acc[m];
            for (int s = 32; s > 0; s >>= 1) a += __shfl_xor(a, s);
            if (lane == 0 && m0 + m < M) Y[(m0 + m) * rows + r] = a;
        }
    }
}

template <int F>
static hipError_t launch_gemm_t(const uint8_t *W, int64_t rows, int64_t cols, const uint16_t *X, int64_t M, float *Y,
                                hipStream_t stream) {
    constexpr int QK = Layout<F>::QK, BYTES = Layout<F>::BYTES;
    const int64_t row_bytes = cols / QK * BYTES;
    constexpr int MB = 8;
    const int64_t jobs = rows * ((M + MB - 1) / MB);
    int64_t grid = (jobs + 3) / 4;
    const int64_t cap = (int64_t)device_cu_count() * 16;
    if (grid > cap) grid = cap;
    hipLaunchKernelGGL((gemm_rows_kernel<F, MB>), dim3((unsigned)grid), dim3(256), 0, stream, W, rows, cols, row_bytes,
                       X, M, Y);
    return hipGetLastError();
}

hipError_t launch_gemm(int type, const void *W, int64_t rows, int64_t cols, const uint16_t *X, int64_t M, float *Y,
                       hipStream_t stream) {
    const uint8_t *w = static_cast<const uint8_t *>(W);
    switch (type) {
    case Q4_K: return launch_gemm_t<Q4_K>(w, rows, cols, X, M, Y, stream);
    case Q6_K: return launch_gemm_t<Q6_K>(w, rows, cols, X, M, Y, stream);
    case Q8_0: return launch_gemm_t<Q8_0>(w, rows, cols, X, M, Y, stream);
    case Q4_0: return launch_gemm_t<Q4_0>(w, rows, cols, X, M, Y, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qk

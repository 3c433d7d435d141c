// qk_dequant.hip — qk_dequantize_row: blocks -> fp32, bit-exact.
//
// The fp32 output is the dominant traffic (4 bytes per weight against at
// most 1.125 read). A workgroup takes 4096 consecutive weights: their blocks
// (a multiple of 16 bytes for every format) go to LDS with coalesced 16-byte
// loads, so each input byte is read from memory once, and each thread then
// decodes four weights at a time from LDS, at positions 1024 weights apart,
// so that every store instruction of a wave writes 1 KiB contiguous. Calls
// that would give fewer than two such workgroups per CU take 2048 weights
// per workgroup (twice the workgroups for the same latency). Built
// with -ffp-contract=off; decode4 also uses explicit round-to-nearest
// operations.
#include "qk_decode.h"
#include "qk_launch.h"

namespace qk {

// WPG: weights per workgroup (4096 or 2048, multiples of every block size).
// A16: out is 16-byte aligned (one 16-byte store per four weights; a run-time
// choice inside the kernel lets the compiler split that store).
template <int F, int WPG, bool A16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ blocks, int64_t n,
                                                      float *__restrict__ out) {
    constexpr int QK = Layout<F>::QK, BYTES = Layout<F>::BYTES;
    constexpr int SB = WPG / QK * BYTES;  // bytes of a workgroup's blocks
    static_assert(WPG % QK == 0 && SB % 16 == 0, "a workgroup's blocks are whole 16-byte pieces");
    __shared__ __attribute__((aligned(16))) uint8_t sb[SB];
    const int64_t w0 = (int64_t)blockIdx.x * WPG;
    const int nw = (int)(n - w0 < WPG ? n - w0 : WPG);  // a multiple of QK
    const int nbytes = nw / QK * BYTES;
    const uint8_t *src = blocks + (int64_t)blockIdx.x * SB;  // 16-byte aligned (blocks is)
    for (int c = threadIdx.x; 16 * c < nbytes; c += blockDim.x) {
        if (16 * c + 16 <= nbytes) {
            *reinterpret_cast<uint4 *>(sb + 16 * c) = *reinterpret_cast<const uint4 *>(src + 16 * c);
        } else {
            for (int b = 16 * c; b < nbytes; b++) sb[b] = src[b];  // the last workgroup's last piece
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < WPG / 1024; k++) {
        const int i = 4 * (threadIdx.x + 256 * k);
        if (i < nw) {
            float w[4];
            decode4<F>(sb + (i / QK) * BYTES, i % QK, w);
            float *o = out + w0 + i;
            if constexpr (A16) {
                *reinterpret_cast<float4 *>(o) = make_float4(w[0], w[1], w[2], w[3]);
            } else {
                o[0] = w[0];
                o[1] = w[1];
                o[2] = w[2];
                o[3] = w[3];
            }
        }
    }
}

hipError_t launch_dequant(int type, const void *blocks, int64_t n, float *out, hipStream_t stream) {
    const int threads = 256;
    const bool big = n >= (int64_t)4096 * 2 * device_cu_count();
    const int wpg = big ? 4096 : 2048;
    const int64_t grid = (n + wpg - 1) / wpg;
    const uint8_t *src = static_cast<const uint8_t *>(blocks);
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, stream, src, n, out); };
    const bool a16 = ((uintptr_t)out & 15u) == 0;
#define QK_DQ(F)                                                                                   \
    (big ? (a16 ? go(dequant_kernel<F, 4096, true>) : go(dequant_kernel<F, 4096, false>))          \
         : (a16 ? go(dequant_kernel<F, 2048, true>) : go(dequant_kernel<F, 2048, false>)))
    switch (type) {
    case Q4_K: QK_DQ(Q4_K); break;
    case Q6_K: QK_DQ(Q6_K); break;
    case Q8_0: QK_DQ(Q8_0); break;
    case Q4_0: QK_DQ(Q4_0); break;
    case Q8_0_F16: QK_DQ(Q8_0_F16); break;
    case Q5_1: QK_DQ(Q5_1); break;
    case Q5_K: QK_DQ(Q5_K); break;
    case Q2_K: QK_DQ(Q2_K); break;
    case Q3_K: QK_DQ(Q3_K); break;
    default: return hipErrorInvalidValue;
    }
#undef QK_DQ
    return hipGetLastError();
}

}  // namespace qk

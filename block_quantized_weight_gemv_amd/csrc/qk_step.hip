// qk_step.hip — the operations of one decode step around the GEMVs
// (include/qk_step.h) and the q8_0 / q4_0 encoder.
//
// The step of "picoLM, in Python" §4 (model_forward) on the GPU: RMSNorm
// (with the residual add of the previous projection fused in), RoPE on q and
// k with the fp16 KV-cache store, attention over the cache with a running
// maximum and sum (the online softmax the page's C uses; no score array;
// the positions split into chunks over many workgroups, whose states a
// second launch merges), SwiGLU. These are small, latency-bound launches next to the weight
// GEMVs; each is one launch so that a whole step can be captured in one HIP
// graph, and the position is read from device memory so that the graph
// replays for every position.
#include <math.h>
#include <stdio.h>

#include <mutex>

#include "../../include/qk_step.h"
#include "qk_launch.h"

namespace qk {

// ------------------------------------------------------------------ norms

// Sum over the workgroup; every thread gets the total (the wave totals are
// added in wave order, so the result does not depend on timing).
__device__ __forceinline__ float block_sum(float v, float *sh) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); i++) t += sh[i];
    __syncthreads();
    return t;
}

__device__ __forceinline__ float block_max(float v, float *sh) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    float t = -INFINITY;
    for (int i = 0; i < (int)(blockDim.x >> 6); i++) t = fmaxf(t, sh[i]);
    __syncthreads();
    return t;
}

// One workgroup: x += r (when r is given), then out = w * x / sqrt(mean(x^2)
// + eps). Each thread reads back only the x values it wrote.
__global__ __launch_bounds__(1024) void rmsnorm_kernel(float *x, const float *__restrict__ r,
                                                       const float *__restrict__ w, int n, float eps, float *out) {
    __shared__ float sh[16];
    float ss = 0.f;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        float v = x[i];
        if (r) {
            v += r[i];
            x[i] = v;
        }
        ss += v * v;
    }
    const float tot = block_sum(ss, sh);
    const float inv = 1.0f / sqrtf(tot / (float)n + eps);
    for (int i = threadIdx.x; i < n; i += blockDim.x) out[i] = w[i] * (x[i] * inv);
}

// ------------------------------------------------------------------ RoPE

__global__ void rope_table_kernel(int64_t max_pos, int half, int head_dim, double base, float *c, float *s) {
    const int64_t total = max_pos * half;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = idx / half;
        const int i = (int)(idx - p * half);
        const double theta = pow(base, -2.0 * (double)i / (double)head_dim);
        const double a = (double)p * theta;
        c[idx] = (float)cos(a);
        s[idx] = (float)sin(a);
    }
}

__device__ __forceinline__ uint16_t to_half_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32: round to nearest even
}

// q heads, then k heads, then the v copy: one thread per rotated pair or per
// v value. The pair (x[2i], x[2i+1]) of each head turns by the table row of
// the position ("picoLM, in Python", the RoPE layout llama.cpp uses).
__global__ __launch_bounds__(256) void rope_kv_kernel(float *q, float *k, const float *__restrict__ v,
                                                      const int32_t *pos, int64_t max_pos,
                                                      const float *__restrict__ ct, const float *__restrict__ st,
                                                      int nh, int nkv, int hd, uint16_t *kc, uint16_t *vc,
                                                      int64_t kv_stride) {
    const int p = *pos;
    if (p < 0 || (int64_t)p >= max_pos) return;
    const int half = hd >> 1;
    const float *c = ct + (int64_t)p * half;
    const float *s = st + (int64_t)p * half;
    const int nq = nh * half, nk = nkv * half, nv = nkv * hd;
    uint16_t *krow = kc + (int64_t)p * kv_stride;
    uint16_t *vrow = vc + (int64_t)p * kv_stride;
    for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < nq + nk + nv; idx += gridDim.x * blockDim.x) {
        if (idx < nq + nk) {
            const bool isq = idx < nq;
            const int j = isq ? idx : idx - nq;
            const int h = j / half, i = j - h * half;
            float *x = (isq ? q : k) + (int64_t)h * hd + 2 * i;
            const float x0 = x[0], x1 = x[1];
            const float r0 = x0 * c[i] - x1 * s[i];
            const float r1 = x0 * s[i] + x1 * c[i];
            x[0] = r0;
            x[1] = r1;
            if (!isq) {
                krow[h * hd + 2 * i] = to_half_bits(r0);
                krow[h * hd + 2 * i + 1] = to_half_bits(r1);
            }
        } else {
            const int j = idx - nq - nk;
            vrow[j] = to_half_bits(v[j]);
        }
    }
}

// ------------------------------------------------------------------ attention

__device__ __forceinline__ void halves8(const uint16_t *p, float *f) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
        f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    }
}

// Positions are split into chunks of `chunk` positions (a power of two of
// at least 64, chosen from the cache's capacity so that there are at most
// kAttMaxChunks of them); workgroup (chunk c, head h) covers positions
// [c * chunk, (c + 1) * chunk) up to the current one. The lanes split the
// head dimension: a group of HD / 8 lanes takes one position at a time, lane
// lo of the group holding dimensions 8 lo .. 8 lo + 7 (one 16-byte read of
// K and one of V per position: a cache row is read by neighbouring lanes),
// so the 256 threads work on 32 (HD 64) or 16 (HD 128) positions at once.
// Each group runs the online softmax over positions g, g + groups, ... of
// the chunk: a running maximum m, the running sum l of exp(s - m) and, per
// lane, the running sums acc of exp(s - m) * V[t] over its 8 dimensions, the
// next position's K and V loaded while one is added. The groups' states are
// brought to the workgroup's maximum and summed in a fixed order (across the
// groups of a wave with lane exchanges, then the four waves through LDS),
// and the chunk's (m, l, acc) goes to the workspace;
// attention_merge_kernel then combines the chunks of each head in chunk
// order. The grid covers the cache's capacity (it cannot depend on the
// position, which lives in device memory); chunks past the position write an
// empty state (m = -inf). (A single launch in which the last workgroup of a
// head to finish merges its chunks measured ~20 us slower per call: the
// device-scope release/acquire of every workgroup writes back and
// invalidates L2.)
constexpr int kAttMinChunk = 64;

// The chunks of head h that hold positions (0 .. p / chunk), merged:
// out_i = sum_c acc_c[i] e^(m_c - M) / sum_c l_c e^(m_c - M), M the largest
// chunk maximum. The chunks' (m, l) go through LDS; thread (i, j) of the 256
// adds acc_c[i] over chunks c = j, j + 256 / HD, ... (independent loads, the
// first 8 of them issued with the (m, l) loads), and the 256 / HD partial
// sums are added in j order.
constexpr int kAttMaxChunks = 256;
constexpr int64_t kAttMaxPos = 65536;  // chunks of up to 256 positions

// Positions per chunk for a cache of max_pos rows (1 <= max_pos <= kAttMaxPos).
inline int att_chunk(int64_t max_pos) {
    int c = kAttMinChunk;
    while ((int64_t)c * kAttMaxChunks < max_pos) c *= 2;
    return c;
}

template <int HD>
__device__ __forceinline__ void attention_merge(const float *part, int ncur, float *out) {
    constexpr int NJ = 256 / HD;
    __shared__ float fm[kAttMaxChunks], fl[kAttMaxChunks];
    __shared__ float shm[16];
    __shared__ float red[NJ][HD];
    const int i = threadIdx.x % HD, j = threadIdx.x / HD;
    float av[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const int c = j + k * NJ;
        av[k] = c < ncur ? part[c * (HD + 2) + 2 + i] : 0.f;
    }
    float mx = -INFINITY;
    for (int c = threadIdx.x; c < ncur; c += blockDim.x) {
        fm[c] = part[c * (HD + 2)];
        fl[c] = part[c * (HD + 2) + 1];
        mx = fmaxf(mx, fm[c]);
    }
    const float M = block_max(mx, shm);  // (its barrier also publishes fm, fl)
    float lp = 0.f;
    for (int c = threadIdx.x; c < ncur; c += blockDim.x) {
        fm[c] = expf(fm[c] - M);
        lp += fl[c] * fm[c];
    }
    const float L = block_sum(lp, shm);  // (and publishes the factors)
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const int c = j + k * NJ;
        if (c < ncur) a += av[k] * fm[c];
    }
#pragma unroll 4
    for (int c = j + 8 * NJ; c < ncur; c += NJ) a += part[c * (HD + 2) + 2 + i] * fm[c];
    red[j][i] = a;
    __syncthreads();
    if (j == 0) {
        float t = red[0][i];
#pragma unroll
        for (int k = 1; k < NJ; k++) t += red[k][i];
        out[i] = t / L;
    }
}

// ROPE: the kernel also does the work of rope_kv_kernel for the current
// position p (q arrives unrotated; k and v arrive as projected): each
// workgroup rotates its head's q, the workgroup whose chunk holds p rotates
// k and rounds k and v to fp16 in LDS and uses them for position p instead
// of reading the cache, and one workgroup per KV head (h % grp == 0) writes
// that cache row. No workgroup of the launch reads row p from the cache.
template <int HD, bool ROPE>
__global__ __launch_bounds__(256) void attention_chunk_kernel(const float *__restrict__ q,
                                                              const uint16_t *kc, const uint16_t *vc,
                                                              const int32_t *pos, int64_t max_pos, int grp,
                                                              int64_t kv_stride, float *__restrict__ ws,
                                                              const float *__restrict__ kraw,
                                                              const float *__restrict__ vraw,
                                                              const float *__restrict__ ct,
                                                              const float *__restrict__ st, int chunk) {
    __shared__ __attribute__((aligned(16))) float qs[HD];
    __shared__ float red[4][HD];
    __shared__ __attribute__((aligned(16))) uint16_t kp[ROPE ? HD : 8], vp[ROPE ? HD : 8];
    const int p = *pos;
    if (p < 0 || (int64_t)p >= max_pos) return;
    const int npos = p + 1;
    const int nchunk = gridDim.x;
    const int c = blockIdx.x, h = blockIdx.y, g = h / grp;
    float *part_h = ws + (int64_t)h * nchunk * (HD + 2);
    float *part = part_h + (int64_t)c * (HD + 2);  // m, l, acc[HD]
    const int t0 = c * chunk, t1 = min(npos, t0 + chunk);
    if (t0 >= t1) {
        if (threadIdx.x == 0) {
            part[0] = -INFINITY;
            part[1] = 0.f;
        }
        return;
    }
    const float scale = 1.0f / sqrtf((float)HD);
    const bool has_p = ROPE && t1 == npos;  // this chunk holds the current position (the last one)
    constexpr int LPP = HD / 8;        // lanes per position
    constexpr int NG = 256 / LPP;      // position groups per workgroup
    const int lane = threadIdx.x & 63;
    const int lo = lane & (LPP - 1);   // dimensions 8 lo .. 8 lo + 7
    const int gi = threadIdx.x / LPP;  // this lane's group
    const int64_t col = (int64_t)g * HD + 8 * lo;
    auto krow = [&](int t) { return *reinterpret_cast<const uint4 *>(kc + (int64_t)t * kv_stride + col); };
    auto vrow = [&](int t) { return *reinterpret_cast<const uint4 *>(vc + (int64_t)t * kv_stride + col); };
    const int tend = has_p ? t1 - 1 : t1;  // with ROPE, position p comes from LDS
    // the group's first cache row, requested before q is read and rotated
    // so that the two round trips overlap
    int t = t0 + gi;
    uint4 kn = uint4{0u, 0u, 0u, 0u}, vn = uint4{0u, 0u, 0u, 0u};
    if (t < tend) {
        kn = krow(t);
        vn = vrow(t);
    }
    if constexpr (ROPE) {
        const float *cs = ct + (int64_t)p * (HD / 2);
        const float *sn = st + (int64_t)p * (HD / 2);
        for (int i = threadIdx.x; i < HD / 2; i += blockDim.x) {
            const float x0 = q[(int64_t)h * HD + 2 * i], x1 = q[(int64_t)h * HD + 2 * i + 1];
            const float r0 = x0 * cs[i] - x1 * sn[i];
            const float r1 = x0 * sn[i] + x1 * cs[i];
            qs[2 * i] = r0 * scale;
            qs[2 * i + 1] = r1 * scale;
            if (has_p) {
                const float k0 = kraw[(int64_t)g * HD + 2 * i], k1 = kraw[(int64_t)g * HD + 2 * i + 1];
                kp[2 * i] = to_half_bits(k0 * cs[i] - k1 * sn[i]);
                kp[2 * i + 1] = to_half_bits(k0 * sn[i] + k1 * cs[i]);
            }
        }
        if (has_p)
            for (int i = threadIdx.x; i < HD; i += blockDim.x) vp[i] = to_half_bits(vraw[(int64_t)g * HD + i]);
        __syncthreads();
        if (has_p && h % grp == 0) {
            uint16_t *kw = const_cast<uint16_t *>(kc) + (int64_t)p * kv_stride + (int64_t)g * HD;
            uint16_t *vw = const_cast<uint16_t *>(vc) + (int64_t)p * kv_stride + (int64_t)g * HD;
            for (int i = threadIdx.x; i < HD; i += blockDim.x) {
                kw[i] = kp[i];
                vw[i] = vp[i];
            }
        }
    } else {
        for (int i = threadIdx.x; i < HD; i += blockDim.x) qs[i] = q[(int64_t)h * HD + i] * scale;
        __syncthreads();
    }

    float qv[8];
#pragma unroll
    for (int i = 0; i < 8; i++) qv[i] = qs[8 * lo + i];

    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = 0.f;
    // one position: its score (the group's partial dots summed over its
    // LPP lanes), then the running state
    auto visit = [&](const uint4 &ku, const uint4 &vu) {
        float kf[8], vf[8];
        halves8(reinterpret_cast<const uint16_t *>(&ku), kf);
        halves8(reinterpret_cast<const uint16_t *>(&vu), vf);
        float sdot = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) sdot += kf[i] * qv[i];
#pragma unroll
        for (int o = 1; o < LPP; o <<= 1) sdot += __shfl_xor(sdot, o);
        const float mn = fmaxf(m, sdot);
        const float corr = expf(m - mn);  // 0 for the first position (m = -inf)
        const float e = expf(sdot - mn);
        l = l * corr + e;
#pragma unroll
        for (int i = 0; i < 8; i++) acc[i] = acc[i] * corr + e * vf[i];
        m = mn;
    };
    if (t < tend) {  // uniform per group; groups differ only in their trip counts
        for (; t < tend; t += NG) {
            const uint4 ku = kn, vu = vn;
            const int tn = min(t + NG, tend - 1);  // the next position (the last one again at the end)
            kn = krow(tn);
            vn = vrow(tn);
            visit(ku, vu);
        }
    }
    if constexpr (ROPE) {
        if (has_p && gi == (p - t0) % NG)
            visit(*reinterpret_cast<const uint4 *>(kp + 8 * lo), *reinterpret_cast<const uint4 *>(vp + 8 * lo));
    }

    // The groups' states, combined in a fixed order with one barrier: each
    // wave brings its groups to the wave's maximum mw and sums them with
    // lane exchanges; the four wave states are then brought to the
    // workgroup's maximum.
    __shared__ float wm[4], wl[4];
    float mw = m;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mw = fmaxf(mw, __shfl_xor(mw, o));
    const float f = m == -INFINITY ? 0.f : expf(m - mw);
    float lw = lo == 0 ? l * f : 0.f;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lw += __shfl_xor(lw, o);
#pragma unroll
    for (int i = 0; i < 8; i++) {
        float a = acc[i] * f;
#pragma unroll
        for (int o = LPP; o < 64; o <<= 1) a += __shfl_xor(a, o);
        acc[i] = a;
    }
    const int w = threadIdx.x >> 6;
    if (lane < LPP) {
#pragma unroll
        for (int i = 0; i < 8; i++) red[w][8 * lane + i] = acc[i];
    }
    if (lane == 0) {
        wm[w] = mw;
        wl[w] = lw;
    }
    __syncthreads();
    const float M = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
    float fw[4];
#pragma unroll
    for (int k = 0; k < 4; k++) fw[k] = wm[k] == -INFINITY ? 0.f : expf(wm[k] - M);
    for (int i = threadIdx.x; i < HD; i += blockDim.x)
        part[2 + i] = ((red[0][i] * fw[0] + red[1][i] * fw[1]) + red[2][i] * fw[2]) + red[3][i] * fw[3];
    if (threadIdx.x == 0) {
        part[0] = M;
        part[1] = ((wl[0] * fw[0] + wl[1] * fw[1]) + wl[2] * fw[2]) + wl[3] * fw[3];
    }
}

template <int HD>
__global__ __launch_bounds__(256) void attention_merge_kernel(const int32_t *pos, int64_t max_pos, int chunk,
                                                              int nchunk, const float *__restrict__ ws,
                                                              float *__restrict__ out) {
    const int p = *pos;
    if (p < 0 || (int64_t)p >= max_pos) return;
    const int h = blockIdx.x;
    attention_merge<HD>(ws + (int64_t)h * nchunk * (HD + 2), min(nchunk, p / chunk + 1), out + (int64_t)h * HD);
}

// ------------------------------------------------------------------ SwiGLU

__global__ void swiglu_kernel(const float *gate, const float *up, int64_t n, float *out) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const float g = gate[i];
        out[i] = g / (1.0f + expf(-g)) * up[i];
    }
}

// ------------------------------------------------------------------ encoder

// One thread per 32-weight block; every operation is one IEEE fp32
// operation in the order the header states, so the integer codes are
// decided exactly as written there.
__global__ void quant_q8_0_kernel(const float *__restrict__ x, int64_t nb, uint8_t *__restrict__ out) {
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += (int64_t)gridDim.x * blockDim.x) {
        float v[32];
#pragma unroll
        for (int j = 0; j < 32; j += 4) {
            const float4 t = *reinterpret_cast<const float4 *>(x + b * 32 + j);
            v[j] = t.x;
            v[j + 1] = t.y;
            v[j + 2] = t.z;
            v[j + 3] = t.w;
        }
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 32; j++) amax = fmaxf(amax, fabsf(v[j]));
        const float d = __fdiv_rn(amax, 127.0f);
        const float id = d != 0.f ? __fdiv_rn(1.0f, d) : 0.f;
        uint32_t *blk = reinterpret_cast<uint32_t *>(out + b * 36);  // 36-byte blocks: 4-byte aligned
        blk[0] = __builtin_bit_cast(uint32_t, d);
#pragma unroll
        for (int j = 0; j < 32; j += 4) {
            uint32_t w = 0;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const int qv = (int)roundf(__fmul_rn(v[j + k], id));
                w |= ((uint32_t)qv & 0xFFu) << (8 * k);
            }
            blk[1 + j / 4] = w;
        }
    }
}

__global__ void quant_q4_0_kernel(const float *__restrict__ x, int64_t nb, uint8_t *__restrict__ out) {
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += (int64_t)gridDim.x * blockDim.x) {
        float v[32];
#pragma unroll
        for (int j = 0; j < 32; j += 4) {
            const float4 t = *reinterpret_cast<const float4 *>(x + b * 32 + j);
            v[j] = t.x;
            v[j + 1] = t.y;
            v[j + 2] = t.z;
            v[j + 3] = t.w;
        }
        float amax = 0.f, mval = 0.f;
#pragma unroll
        for (int j = 0; j < 32; j++) {
            const float a = fabsf(v[j]);
            if (a > amax) {  // the first value of largest magnitude
                amax = a;
                mval = v[j];
            }
        }
        float d = __fdiv_rn(mval, -8.0f);
        // d is an fp32 value before it is rounded to fp16: without this the
        // multiply and the conversion fuse into fma(m, -1/8, +0) -> f16,
        // which turns the -0 scale of an all-zero block into +0
        __asm__("" : "+v"(d));
        const float id = d != 0.f ? __fdiv_rn(1.0f, d) : 0.f;
        uint16_t *blk = reinterpret_cast<uint16_t *>(out + b * 18);  // 18-byte blocks: 2-byte aligned
        blk[0] = to_half_bits(d);
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
            uint32_t bytes[2];
#pragma unroll
            for (int k = 0; k < 2; k++) {
                const int c0 = min(15, (int)__fadd_rn(__fmul_rn(v[j + k], id), 8.5f));
                const int c1 = min(15, (int)__fadd_rn(__fmul_rn(v[j + k + 16], id), 8.5f));
                bytes[k] = (uint32_t)(c0 | (c1 << 4));
            }
            blk[1 + j / 2] = (uint16_t)(bytes[0] | (bytes[1] << 8));
        }
    }
}

static unsigned grid_for(int64_t n, int threads, int64_t cap) {
    int64_t g = (n + threads - 1) / threads;
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return (unsigned)g;
}

}  // namespace qk

// ------------------------------------------------------------------ C ABI

namespace {

bool al(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return QK_OK;
    char msg[256];
    snprintf(msg, sizeof msg, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
    return qk::set_last_error(QK_EHIP, msg);
}

int bad(int status, const char *msg) { return qk::set_last_error(status, msg); }

}  // namespace

extern "C" {

int qk_rmsnorm(const float *x, const float *w, int64_t n, float eps, float *out, void *stream) {
    if (!x || !w || !out) return bad(QK_EINVAL_PTR, "qk_rmsnorm: null pointer");
    if (n < 1 || n > 65536) return bad(QK_EINVAL_SHAPE, "qk_rmsnorm: n must be 1..65536");
    hipLaunchKernelGGL(qk::rmsnorm_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, const_cast<float *>(x),
                       nullptr, w, (int)n, eps, out);
    return hip_status(hipGetLastError(), "qk_rmsnorm launch");
}

int qk_add_rmsnorm(float *x, const float *r, const float *w, int64_t n, float eps, float *out, void *stream) {
    if (!x || !r || !w || !out) return bad(QK_EINVAL_PTR, "qk_add_rmsnorm: null pointer");
    if (n < 1 || n > 65536) return bad(QK_EINVAL_SHAPE, "qk_add_rmsnorm: n must be 1..65536");
    if (out == x || out == r) return bad(QK_EINVAL_PTR, "qk_add_rmsnorm: out must not alias x or r");
    hipLaunchKernelGGL(qk::rmsnorm_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, x, r, w, (int)n, eps, out);
    return hip_status(hipGetLastError(), "qk_add_rmsnorm launch");
}

int qk_rope_tables(int64_t max_pos, int head_dim, double base, float *cos_table, float *sin_table, void *stream) {
    if (!cos_table || !sin_table) return bad(QK_EINVAL_PTR, "qk_rope_tables: null pointer");
    if (max_pos < 1 || max_pos > (int64_t(1) << 24) || head_dim < 2 || head_dim > 1024 || head_dim % 2 ||
        !(base > 0.0))
        return bad(QK_EINVAL_SHAPE, "qk_rope_tables: bad size or base");
    const int half = head_dim / 2;
    hipLaunchKernelGGL(qk::rope_table_kernel, dim3(qk::grid_for(max_pos * half, 256, 4096)), dim3(256), 0,
                       (hipStream_t)stream, max_pos, half, head_dim, base, cos_table, sin_table);
    return hip_status(hipGetLastError(), "qk_rope_tables launch");
}

int qk_rope_kv(float *q, float *k, const float *v, const int32_t *pos, int64_t max_pos, const float *cos_table,
               const float *sin_table, int n_heads, int n_kv_heads, int head_dim, uint16_t *k_cache,
               uint16_t *v_cache, int64_t kv_stride, void *stream) {
    if (!q || !k || !v || !pos || !cos_table || !sin_table || !k_cache || !v_cache)
        return bad(QK_EINVAL_PTR, "qk_rope_kv: null pointer");
    if (n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads || head_dim < 2 || head_dim > 1024 || head_dim % 2 ||
        max_pos < 1 || kv_stride < (int64_t)n_kv_heads * head_dim || n_heads > 4096)
        return bad(QK_EINVAL_SHAPE, "qk_rope_kv: bad sizes");
    const int64_t work = (int64_t)n_heads * (head_dim / 2) + (int64_t)n_kv_heads * (head_dim / 2) +
                         (int64_t)n_kv_heads * head_dim;
    hipLaunchKernelGGL(qk::rope_kv_kernel, dim3(qk::grid_for(work, 256, 1024)), dim3(256), 0, (hipStream_t)stream, q,
                       k, v, pos, max_pos, cos_table, sin_table, n_heads, n_kv_heads, head_dim, k_cache, v_cache,
                       kv_stride);
    return hip_status(hipGetLastError(), "qk_rope_kv launch");
}

// Workspace: the chunk states, n_heads x nchunk x (head_dim + 2) floats.
int64_t qk_attention_workspace_bytes(int n_heads, int head_dim, int64_t max_pos) {
    if (n_heads < 1 || head_dim < 1 || max_pos < 1 || max_pos > qk::kAttMaxPos) return QK_EINVAL_SHAPE;
    const int chunk = qk::att_chunk(max_pos);
    const int64_t nchunk = (max_pos + chunk - 1) / chunk;
    return (int64_t)n_heads * nchunk * (head_dim + 2) * (int64_t)sizeof(float);
}

// ------------------------------------------------ attention without a workspace
//
// For callers that cannot allocate device memory: the chunk states live in a
// file-scope device array (one per GPU, kept until the process ends). Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in symbol): its device address is looked up once per device with
// hipGetSymbolAddress and that address is what the kernels receive.
constexpr int64_t kAttScratchBytes = int64_t(8) << 20;
static __device__ __align__(256) float scratch[kAttScratchBytes / sizeof(float)];

namespace {
// Device address of `scratch` on the current device (looked up on the first
// call per device; nullptr and a HIP error on failure).
hipError_t att_scratch(float **out) {
    static std::mutex mu;
    static float *addr[64] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<float *>(ptr);
    }
    *out = addr[dev];
    return hipSuccess;
}
}  // namespace

// With noalloc the chunk states go to the static scratch (workspace and
// workspace_bytes are ignored); every argument is checked before any HIP call.
static int attention_launch(const float *q, const float *k, const float *v, const float *ct, const float *st,
                            uint16_t *k_cache, uint16_t *v_cache, const int32_t *pos, int64_t max_pos, int n_heads,
                            int n_kv_heads, int head_dim, int64_t kv_stride, float *workspace,
                            int64_t workspace_bytes, float *out, void *stream, bool rope, bool noalloc = false) {
    if (noalloc) {
        const int64_t need = qk_attention_workspace_bytes(n_heads, head_dim, max_pos);
        if (need > kAttScratchBytes)
            return bad(QK_EINVAL_SHAPE, "qk_attention_rope_noalloc: these sizes need more chunk-state scratch than "
                                        "the library's static 8 MiB (use qk_attention_rope with a workspace)");
        workspace = nullptr;
        workspace_bytes = kAttScratchBytes;
    }
    if (!q || !k_cache || !v_cache || !pos || !out || (!workspace && !noalloc))
        return bad(QK_EINVAL_PTR, "qk_attention: null pointer");
    if (rope && (!k || !v || !ct || !st)) return bad(QK_EINVAL_PTR, "qk_attention_rope: null pointer");
    if (n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads || (head_dim != 64 && head_dim != 128) ||
        max_pos < 1 || max_pos > qk::kAttMaxPos || kv_stride < (int64_t)n_kv_heads * head_dim ||
        n_heads > 65535)
        return bad(QK_EINVAL_SHAPE, "qk_attention: bad sizes (head_dim 64 or 128)");
    if (!al(k_cache, 16) || !al(v_cache, 16) || kv_stride % 8)
        return bad(QK_EALIGN, "qk_attention: caches 16-byte aligned, kv_stride a multiple of 8");
    if (workspace_bytes < qk_attention_workspace_bytes(n_heads, head_dim, max_pos))
        return bad(QK_EINVAL_SHAPE, "qk_attention: workspace smaller than qk_attention_workspace_bytes()");
    if (noalloc) {
        const hipError_t e = att_scratch(&workspace);
        if (e != hipSuccess) return hip_status(e, "qk_attention_rope_noalloc: scratch address");
    }
    if (!al(workspace, 16)) return bad(QK_EALIGN, "qk_attention: workspace 16-byte aligned");
    const int grp = n_heads / n_kv_heads;
    const int chunk = qk::att_chunk(max_pos);
    const int nchunk = (int)((max_pos + chunk - 1) / chunk);
    const hipStream_t s = (hipStream_t)stream;
    const dim3 grid(nchunk, n_heads);
#define QK_ATT(HD, R)                                                                                               \
    hipLaunchKernelGGL((qk::attention_chunk_kernel<HD, R>), grid, dim3(256), 0, s, q, k_cache, v_cache, pos, max_pos, \
                       grp, kv_stride, workspace, k, v, ct, st, chunk);                                             \
    hipLaunchKernelGGL(qk::attention_merge_kernel<HD>, dim3(n_heads), dim3(256), 0, s, pos, max_pos, chunk, nchunk,\
                       workspace, out)
    if (head_dim == 64) {
        if (rope) { QK_ATT(64, true); } else { QK_ATT(64, false); }
    } else {
        if (rope) { QK_ATT(128, true); } else { QK_ATT(128, false); }
    }
#undef QK_ATT
    return hip_status(hipGetLastError(), "qk_attention launch");
}

int qk_attention(const float *q, const uint16_t *k_cache, const uint16_t *v_cache, const int32_t *pos,
                 int64_t max_pos, int n_heads, int n_kv_heads, int head_dim, int64_t kv_stride, float *workspace,
                 int64_t workspace_bytes, float *out, void *stream) {
    return attention_launch(q, nullptr, nullptr, nullptr, nullptr, const_cast<uint16_t *>(k_cache),
                            const_cast<uint16_t *>(v_cache), pos, max_pos, n_heads, n_kv_heads, head_dim, kv_stride,
                            workspace, workspace_bytes, out, stream, false);
}

int qk_attention_rope(const float *q, const float *k, const float *v, const int32_t *pos, int64_t max_pos,
                      const float *cos_table, const float *sin_table, int n_heads, int n_kv_heads, int head_dim,
                      uint16_t *k_cache, uint16_t *v_cache, int64_t kv_stride, float *workspace,
                      int64_t workspace_bytes, float *out, void *stream) {
    return attention_launch(q, k, v, cos_table, sin_table, k_cache, v_cache, pos, max_pos, n_heads, n_kv_heads,
                            head_dim, kv_stride, workspace, workspace_bytes, out, stream, true);
}

int64_t qk_attention_scratch_limit(void) { return kAttScratchBytes; }

int qk_attention_rope_noalloc(const float *q, const float *k, const float *v, const int32_t *pos, int64_t max_pos,
                              const float *cos_table, const float *sin_table, int n_heads, int n_kv_heads,
                              int head_dim, uint16_t *k_cache, uint16_t *v_cache, int64_t kv_stride, float *out,
                              void *stream) {
    return attention_launch(q, k, v, cos_table, sin_table, k_cache, v_cache, pos, max_pos, n_heads, n_kv_heads,
                            head_dim, kv_stride, nullptr, 0, out, stream, true, true);
}

int qk_swiglu(const float *gate, const float *up, int64_t n, float *out, void *stream) {
    if (!gate || !up || !out) return bad(QK_EINVAL_PTR, "qk_swiglu: null pointer");
    if (n < 0) return bad(QK_EINVAL_SHAPE, "qk_swiglu: negative size");
    if (n == 0) return QK_OK;
    hipLaunchKernelGGL(qk::swiglu_kernel, dim3(qk::grid_for(n, 256, 4096)), dim3(256), 0, (hipStream_t)stream, gate,
                       up, n, out);
    return hip_status(hipGetLastError(), "qk_swiglu launch");
}

int qk_quantize_row(int type, const float *x, int64_t n, void *blocks, void *stream) {
    if (type != QK_Q8_0 && type != QK_Q4_0) return bad(QK_EINVAL_TYPE, "qk_quantize_row: q8_0 or q4_0");
    if (n < 0 || n % 32) return bad(QK_EINVAL_SHAPE, "qk_quantize_row: n must be a multiple of 32");
    if (n == 0) return QK_OK;
    if (!x || !blocks) return bad(QK_EINVAL_PTR, "qk_quantize_row: null pointer");
    if (!al(x, 16) || !al(blocks, 16)) return bad(QK_EALIGN, "qk_quantize_row: x and blocks 16-byte aligned");
    const int64_t nb = n / 32;
    const unsigned grid = qk::grid_for(nb, 256, 8192);
    uint8_t *dst = static_cast<uint8_t *>(blocks);
    if (type == QK_Q8_0)
        hipLaunchKernelGGL(qk::quant_q8_0_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, x, nb, dst);
    else
        hipLaunchKernelGGL(qk::quant_q4_0_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, x, nb, dst);
    return hip_status(hipGetLastError(), "qk_quantize_row launch");
}

}  // extern "C"

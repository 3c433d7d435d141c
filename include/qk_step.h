/*
 * qk_step.h — the operations of one decode step around the GEMVs of qk.h,
 * and the encoder that writes q8_0 / q4_0 blocks, on one AMD MI355X.
 *
 * One token's forward pass ("picoLM, in Python", §4 "The forward pass"):
 * the token's embedding row is dequantised (qk_dequantize_row); each layer
 * normalises x (RMSNorm), projects q, k, v (qk_gemv / qk_gemv_batch),
 * rotates q and k with the position's cos/sin (RoPE, the interleaved pairs
 * of §3 "The RoPE layout is not the one you learned"), stores k and v in an
 * fp16 cache at `pos` (k after the rotation), lets every query head attend
 * over positions 0..pos of the KV head it shares (n_kv_heads < n_heads),
 * projects the result (qk_gemv), adds it to x, normalises again, runs
 * gate/up (qk_gemv_batch), SwiGLU, down (qk_gemv) and adds that to x; a last
 * RMSNorm and the output matrix give the logits. PETIT's README names the
 * same block (RMSNorm, RoPE with base 10000 per head, KV cache, SwiGLU) and
 * an exporter that quantises fp32 weights into q8_0 / q4_0 blocks.
 *
 * Readings where the pages leave a step open: RMSNorm out_i = w_i * x_i /
 * sqrt(mean(x^2) + eps); RoPE theta_i = base^(-2i/head_dim); attention
 * scale 1/sqrt(head_dim), query head h reads KV head h / (n_heads /
 * n_kv_heads); SwiGLU silu(gate) * up; the encoder's rounding rule (below).
 *
 * Position on the device: the RoPE/cache and attention calls read the
 * position from a device int32 (`pos`), so a captured HIP graph of a whole
 * step replays for every position; the caller advances that int between
 * replays. A position outside [0, max_pos) makes those calls write nothing
 * (the host cannot check a device value; the kernels do).
 *
 * Memory: every pointer is device memory owned by the caller; nothing is
 * allocated (attention's partial results go to a workspace the caller
 * passes). All vectors are fp32 unless stated; the KV cache is fp16 (bit
 * patterns in uint16): one layer's K (and V) cache holds max_pos rows, row t
 * with n_kv_heads * head_dim values starting at t * kv_stride; the RoPE
 * tables hold max_pos rows of head_dim/2 values. Calls enqueue on `stream` (a
 * hipStream_t as void*, NULL the null stream) and return qk_status codes
 * (qk.h); arguments are checked on the host first and a failed check
 * launches nothing.
 */
#ifndef QK_STEP_H
#define QK_STEP_H

#include <stdint.h>

#include "qk.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out = RMSNorm(x) * w over n values (n >= 1, n <= 65536): out_i = w_i * x_i
 * / sqrt(mean(x^2) + eps). out may alias x. */
int qk_rmsnorm(const float *x, const float *w, int64_t n, float eps, float *out, void *stream);

/* The residual step and the next norm in one launch: x += r (in place),
 * then out = RMSNorm(x) * w. out must not alias x or r. */
int qk_add_rmsnorm(float *x, const float *r, const float *w, int64_t n, float eps, float *out, void *stream);

/* RoPE tables for positions 0..max_pos-1: cos/sin[p * (head_dim/2) + i] of
 * p * base^(-2i/head_dim), computed in fp64 and rounded to fp32. head_dim
 * even, 2..1024. */
int qk_rope_tables(int64_t max_pos, int head_dim, double base, float *cos_table, float *sin_table, void *stream);

/* For the position *pos: rotate q (n_heads heads) and k (n_kv_heads heads)
 * in place, each pair (x[2i], x[2i+1]) of a head by the table row *pos, and
 * store the rotated k and v, rounded to fp16 (nearest even), in row *pos of
 * the layer's caches. n_heads a multiple of n_kv_heads; head_dim even,
 * 2..1024; kv_stride >= n_kv_heads * head_dim. */
int qk_rope_kv(float *q, float *k, const float *v, const int32_t *pos, int64_t max_pos, const float *cos_table,
               const float *sin_table, int n_heads, int n_kv_heads, int head_dim, uint16_t *k_cache,
               uint16_t *v_cache, int64_t kv_stride, void *stream);

/* Attention of one position's queries over cache rows 0..*pos:
 * out[h*head_dim + i] = sum_t p_t V[t, g, i] with p = softmax_t(q_h . K[t, g]
 * / sqrt(head_dim)), g = h / (n_heads / n_kv_heads). One pass over the cache
 * with a running maximum and sum (no score array): the positions are split
 * into chunks (64 positions, or more for caches of over 16384 rows: at most
 * 256 chunks) handled by separate workgroups, each of which leaves its
 * chunk's (maximum, sum, weighted V sum) in `workspace`; a second launch on
 * the same stream merges them in chunk order. max_pos <= 65536; head_dim 64
 * or 128; k/v caches
 * 16-byte aligned with kv_stride a multiple of 8. workspace: caller-owned
 * device memory, 16-byte aligned, of at least
 * qk_attention_workspace_bytes(n_heads, head_dim, max_pos) bytes (scratch:
 * no initial contents needed; calls that overlap on one workspace race). */
int64_t qk_attention_workspace_bytes(int n_heads, int head_dim, int64_t max_pos);
int qk_attention(const float *q, const uint16_t *k_cache, const uint16_t *v_cache, const int32_t *pos,
                 int64_t max_pos, int n_heads, int n_kv_heads, int head_dim, int64_t kv_stride, float *workspace,
                 int64_t workspace_bytes, float *out, void *stream);

/* qk_rope_kv and qk_attention in one: q, k, v arrive as projected (q and k
 * unrotated; none is modified); the rotation of q, the rotation of k, the
 * fp16 rounding of k and v and the write of cache row *pos happen inside
 * the attention launch (the workgroups that cover *pos use the new row from
 * on-chip memory). The cache row *pos and out are what qk_rope_kv followed
 * by qk_attention give (up to the fusing of the rotation's products). */
int qk_attention_rope(const float *q, const float *k, const float *v, const int32_t *pos, int64_t max_pos,
                      const float *cos_table, const float *sin_table, int n_heads, int n_kv_heads, int head_dim,
                      uint16_t *k_cache, uint16_t *v_cache, int64_t kv_stride, float *workspace,
                      int64_t workspace_bytes, float *out, void *stream);

/* qk_attention_rope for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that must not call hipMalloc,
 * harnesses that forbid allocation): the same call without a workspace. The
 * chunk states go to a static scratch array of the library, one per GPU,
 * held until the process ends, of qk_attention_scratch_limit() bytes (8 MiB:
 * any max_pos <= 65536 with up to 32 heads of 128 or 64 heads of 64); sizes
 * whose qk_attention_workspace_bytes() exceed it are QK_EINVAL_SHAPE before
 * anything is launched. It allocates nothing and frees nothing; its device
 * address is looked up on the first call on each device (make that first
 * call outside graph capture). Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams, other
 * threads) race and give wrong results; calls ordered on one stream do not.
 * Nothing needs to start at zero: each call writes every chunk state it
 * reads. Results are bit-identical to qk_attention_rope's. */
int64_t qk_attention_scratch_limit(void);
int qk_attention_rope_noalloc(const float *q, const float *k, const float *v, const int32_t *pos, int64_t max_pos,
                              const float *cos_table, const float *sin_table, int n_heads, int n_kv_heads,
                              int head_dim, uint16_t *k_cache, uint16_t *v_cache, int64_t kv_stride, float *out,
                              void *stream);

/* out_i = silu(gate_i) * up_i, silu(g) = g / (1 + exp(-g)). out may alias
 * gate or up. */
int qk_swiglu(const float *gate, const float *up, int64_t n, float *out, void *stream);

/* A transform of the input of a GEMV, done by the GEMV kernel as it stages
 * x (the norm or the SwiGLU that feeds a projection, without a launch of its
 * own). */
typedef enum {
    QK_INPUT_PLAIN = 0,       /* x as given */
    QK_INPUT_ADD_RMSNORM = 1, /* x' = RMSNorm(x + aux) * norm_w (eps), and
                                 x + aux written to x_out: the residual add
                                 and the next norm of the forward pass */
    QK_INPUT_SWIGLU = 2       /* x' = silu(x) * aux: gate in x, up in aux */
} qk_input_kind;

typedef struct qk_gemv_input {
    int kind;             /* qk_input_kind */
    const float *aux;     /* fp32[cols]: the residual (kind 1) or up (kind 2) */
    const float *norm_w;  /* fp32[cols] (kind 1) */
    float eps;            /* (kind 1) */
    float *x_out;         /* fp32[cols] receives x + aux (kind 1); must not
                             overlap x, aux, norm_w or any output */
} qk_gemv_input;

/* 1 if qk_gemv_batch_input takes this format and shape (the fused GEMV
 * kernels of Q4_K, Q6_K, q4_0 and q8_0, with their limits as described for
 * qk_gemv), else 0. */
int qk_gemv_input_supported(int type, int64_t rows, int64_t cols);

/* 1 to 4 GEMVs that share cols and x, in one launch, each computing
 * y = W x' with x' the transform `in` of x (the same x' for all). Every
 * descriptor needs rows >= 1 and qk_gemv_input_supported; their formats
 * must share a launch as in qk_gemv_batch. Within the tolerance of qk_gemv
 * against W applied to x' computed in fp64; x' itself equals what
 * qk_add_rmsnorm / qk_swiglu compute up to the order of the sum of squares.
 * x + aux in x_out is exact (fp32 additions). aux, norm_w, x_out 16-byte
 * aligned. */
int qk_gemv_batch_input(const qk_gemv_desc *descs, int n, const qk_gemv_input *in, void *stream);

/* The encoder (PETIT README, "How the pieces match": the exporter writes
 * q8_0 / q4_0 blocks from fp32 weights). n a multiple of 32; type QK_Q8_0
 * or QK_Q4_0; blocks receives n/32 blocks. Rule (a reading; the pages give
 * only the formats), each step one fp32 operation rounded to nearest even:
 * q8_0 amax = max |x|, d = amax / 127, id = d ? 1/d : 0, q = round half away
 * from zero (x * id), block = fp32 d, int8 q[32]; q4_0 m = the first value
 * of largest magnitude, d = m / -8, id = d ? 1/d : 0, code = min(15,
 * trunc(x * id + 8.5)), block = fp16(d), byte j = code j | code j+16 << 4. */
int qk_quantize_row(int type, const float *x, int64_t n, void *blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QK_STEP_H */

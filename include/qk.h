/*
 * qk.h — C ABI of libqk.so: block-quantized LLM weights decoded and
 * multiplied on one AMD MI355X (gfx950) GPU.
 *
 * Formats (block = weights sharing one set of scales; W is stored out x in,
 * row-major, each row a run of whole blocks with no padding between rows):
 *
 *   QK_Q4_K  256 weights in 144 bytes: fp16 d, fp16 dmin, eight 6-bit
 *            scales and eight 6-bit mins bit-packed into 12 bytes, 128 bytes
 *            of nibbles; weight = d*scale*q - dmin*min.
 *            ("picoLM, in Python", section "§2 — K-quants")
 *   QK_Q6_K  256 weights in 210 bytes: ql[128] (low 4 bits), qh[64] (high 2
 *            bits), int8 scales[16] (one per 16 weights), fp16 d;
 *            weight = d*scale*(code - 32).
 *            ("PicoLM Q6_K量化Bug调试全记录", section 原理)
 *   QK_Q8_0  32 weights in 36 bytes: fp32 scale, 32 int8; weight = scale*q.
 *   QK_Q4_0  32 weights in 18 bytes: fp16 scale, 16 bytes of nibbles; byte j
 *            holds weight j (low nibble) and weight j+16 (high nibble);
 *            weight = d*(nibble - 8).
 *            (PETIT README, "What makes it fast & small" and "How the pieces
 *            match": fp32-scale q8_0 and fp16-scale q4_0 blocks, weights
 *            stored transposed out x in, padded to a multiple of 32)
 *
 * The ggml-specification formats that "picoLM, in Python" names (§2 K-quants,
 * "Verify against the spec, because even the C can be wrong", which gives
 * Q2_K's size and takes the ggml specification as the formats' source of
 * truth; "Exercises" names Q5_K and Q5_1), in the specification's layouts:
 *
 *   QK_Q8_0_F16  32 weights in 34 bytes: fp16 d, 32 int8; weight = d*q
 *            (GGUF's Q8_0; QK_Q8_0 above is PETIT's fp32-scale block).
 *   QK_Q5_1  32 weights in 24 bytes: fp16 d, fp16 m, uint32 qh, 16 nibble
 *            bytes; byte j holds weight j (low nibble, fifth bit = bit j of
 *            qh) and weight j+16 (high nibble, bit j+16); weight = q*d + m.
 *   QK_Q5_K  256 weights in 176 bytes: Q4_K's fp16 d, fp16 dmin and 12
 *            packed scale/min bytes, qh[32], 128 nibble bytes; weight 64g+l
 *            (low nibble of byte 32g+l) takes bit 2g of qh[l] as its fifth
 *            bit, weight 64g+32+l (high nibble) bit 2g+1; weight =
 *            d*scale*q - dmin*min per 32 weights.
 *   QK_Q2_K  256 weights in 84 bytes: scales[16] (low nibble scale, high
 *            nibble min, one per 16 weights), qs[64], fp16 d, fp16 dmin;
 *            weight 128h+32j+l = bits 2j..2j+1 of qs[32h+l];
 *            weight = d*scale*q - dmin*min.
 *   QK_Q3_K  256 weights in 110 bytes: hmask[32], qs[64], 12 bytes of
 *            sixteen packed 6-bit scales, fp16 d; weight 128h+32j+l =
 *            (bits 2j..2j+1 of qs[32h+l]) - 4 unless bit 4h+j of hmask[l]
 *            is set; scale s (one per 16 weights) has its low 4 bits in
 *            byte s (s < 8) or the high nibble of byte s-8 and its top 2
 *            bits at bit 2(s/4) of byte 8 + s%4, stored plus 32;
 *            weight = d*scale*q.
 * All multi-byte fields are little-endian.
 *
 * Memory: every pointer argument of the compute calls is device memory (or
 * memory the current HIP device can access) owned by the caller. The library
 * never allocates, frees or keeps caller memory, and the compute calls
 * allocate nothing. Pointers into one call must not alias its outputs.
 * Calls work on the current HIP device.
 *
 * Streams: `stream` is a hipStream_t passed as void*; NULL is the null
 * (legacy default) stream. Compute calls only enqueue work: they return
 * before the GPU finishes, and a fault inside a kernel surfaces at the
 * caller's next synchronisation on that stream.
 *
 * Errors: every call returns a qk_status. Arguments are checked on the host
 * before any HIP call; a failed check launches nothing and writes nothing.
 * A HIP error at launch returns QK_EHIP; qk_last_hip_error() then describes
 * it.
 */
#ifndef QK_H
#define QK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Format ids (this library's own numbering; a GGUF loader maps ggml types
 * to these). */
typedef enum {
    QK_Q4_0 = 1,
    QK_Q8_0 = 2,
    QK_Q4_K = 3,
    QK_Q6_K = 4,
    QK_Q8_0_F16 = 5,
    QK_Q5_1 = 6,
    QK_Q5_K = 7,
    QK_Q2_K = 8,
    QK_Q3_K = 9
} qk_type;

typedef enum {
    QK_OK = 0,
    QK_EINVAL_TYPE = -1,  /* unknown format id */
    QK_EINVAL_SHAPE = -2, /* negative size, or a weight count that is not a
                             whole number of blocks */
    QK_EINVAL_PTR = -3,   /* NULL pointer where data is needed */
    QK_EALIGN = -4,       /* W/blocks, x or X not 16-byte aligned; y, Y or
                             out not 4-byte aligned */
    QK_EHIP = -5,         /* the HIP runtime reported an error */
    QK_EIO = -6,          /* a file could not be opened or mapped (qk_gguf.h) */
    QK_EFORMAT = -7,      /* a file is not a well-formed GGUF file (qk_gguf.h) */
    QK_ENOTFOUND = -8,    /* no such tensor or metadata entry (qk_gguf.h) */
    QK_ENOMEM = -9        /* host memory ran out while reading a file's tables
                             (qk_gguf.h) */
} qk_status;

/* Weights per block: 256 (Q4_K, Q6_K, Q5_K, Q2_K, Q3_K) or 32 (Q4_0, Q8_0,
 * Q8_0_F16, Q5_1); QK_EINVAL_TYPE for an unknown id. */
int qk_block_elems(int type);

/* Bytes per block: 144 (Q4_K), 210 (Q6_K), 18 (Q4_0), 36 (Q8_0), 34
 * (Q8_0_F16), 24 (Q5_1), 176 (Q5_K), 84 (Q2_K), 110 (Q3_K); QK_EINVAL_TYPE
 * for an unknown id. */
int qk_block_bytes(int type);

/* Bytes of one row of `cols` weights (cols / block_elems * block_bytes);
 * a negative qk_status for an unknown type or a cols that is negative or not
 * a whole number of blocks. */
int64_t qk_row_bytes(int type, int64_t cols);

/* Dequantise n weights held in n / block_elems consecutive blocks into
 * out[n] (fp32). Every output is bit-identical to the format's definition
 * evaluated in fp32 in the pages' order (Q4_K: (d*scale)*q - dmin*min;
 * Q6_K: (d*scale)*q; Q8_0: scale*q; Q4_0: d*(nibble-8)). This is the
 * pages' dequantize_row(src, dst, n, type), used for an embedding row
 * ("picoLM, in Python", section "§4 — The forward pass").
 * n == 0 is a no-op. Enqueued on the null stream. */
int qk_dequantize_row(int type, const void *blocks, int64_t n, float *out);

/* As qk_dequantize_row, on `stream`. */
int qk_dequantize_row_async(int type, const void *blocks, int64_t n, float *out, void *stream);

/* y = W x: y[r] = sum_c w[r][c] * x[c] for r < rows, with W rows x cols of
 * format `type` (rows x cols/block_elems blocks, row-major), x fp32[cols],
 * y fp32[rows] (overwritten). The weights are decoded on the fly and never
 * written out in fp32: the fused dequantise-and-dot of the pages' matmul
 * ("picoLM, in Python", section "§3 — Tensor ops"; the fused vec_dot of
 * "PicoLM Q6_K量化Bug调试全记录"). Accumulation is fp32; each output is
 * within 1e-4 * sum_c |w[r][c] * x[c]| + 1e-6 of the exact sum.
 * Any shape is accepted; the fused kernels take rows of up to 512 units of
 * 64 weights (K-quants: 32768 columns) or 32 weights (the 32-weight formats:
 * 16384 columns), whose x fits one workgroup's LDS, with an even block count
 * per row for q4_0 and Q8_0_F16 and, for Q3_K, an even block count or an
 * even row count; other shapes run a slower generic kernel with the same
 * result bound. Results are deterministic (a fixed summation order).
 * y must not overlap W or x (QK_EINVAL_PTR): every workgroup reads all of x
 * when it starts, after others may have written y.
 * rows == 0 is a no-op; cols == 0 writes y = 0. */
int qk_gemv(int type, const void *W, int64_t rows, int64_t cols,
            const float *x, float *y, void *stream);

/* Which kernel qk_gemv runs for this format and shape: a host-side query of
 * the type-dispatch table that launches nothing. QK_PATH_GENERIC, the
 * generic kernel; QK_PATH_FUSED, the fused GEMV reading rows straight into
 * registers; QK_PATH_STREAMED, the fused GEMV streaming row groups through
 * LDS (launches of 128 MiB or more whose rows one wave covers, not q4_0);
 * QK_PATH_WIDE, the wide-row kernel (6145 to 32768 columns). The tuning key
 * QK_TUNE_GEMV_STREAM overrides the streamed choice here as in qk_gemv.
 * Returns QK_EINVAL_TYPE or QK_EINVAL_SHAPE (rows < 1, cols < 1 or not a
 * multiple of the block size) otherwise. */
typedef enum { QK_PATH_GENERIC = 0, QK_PATH_FUSED = 1, QK_PATH_STREAMED = 2, QK_PATH_WIDE = 3 } qk_gemv_path;
int qk_gemv_kernel_path(int type, int64_t rows, int64_t cols);

/* One GEMV of a batch (see qk_gemv_batch). */
typedef struct qk_gemv_desc {
    int type;        /* qk_type */
    const void *W;   /* rows x cols of `type`, as for qk_gemv */
    int64_t rows;
    int64_t cols;
    const float *x;  /* fp32[cols] */
    float *y;        /* fp32[rows], overwritten */
} qk_gemv_desc;

/* n independent GEMVs, each exactly as qk_gemv(descs[i]...), enqueued on
 * `stream` with as few launches as possible: GEMVs of the same width that
 * read the same x run in one launch, up to 4 per launch, and Q4_K may share a
 * launch with Q6_K (and q4_0 with q8_0) because their lanes cover rows the
 * same way. This is the grouped decode launch: one launch per dependency
 * stage of a decoder layer instead of one per weight matrix ("picoLM, in
 * Python", section "§4 — The forward pass": q, k and v read the same normed
 * x, gate and up the same one). Every descriptor is checked as qk_gemv checks
 * its arguments before anything is launched; outputs must not overlap each
 * other or any input of the batch (QK_EINVAL_PTR). n == 0 is a no-op. */
int qk_gemv_batch(const qk_gemv_desc *descs, int n, void *stream);

/* A decode-step weight pass in one persistent launch (the device-side work
 * list of the grouped decode launch). The pages' forward pass runs a layer's
 * projections as dependent stages, each stage's x computed from what the
 * stage before produced ("picoLM, in Python", §4 — The forward pass: q, k
 * and v read one normed x, o the attention output, gate and up one normed x,
 * down the SwiGLU product). qk_gemv_batch launches one kernel per stage; a
 * pass runs all the stages in one launch whose workgroups stay resident, and
 * a stage that reads an earlier stage's output starts, on the device, as
 * soon as that output is written.
 *
 * descs[0..n) in stage order; stage[i] is the stage of descs[i], starting at
 * 0 and rising by 0 or 1 from one GEMV to the next. The GEMVs of one stage
 * (at most 4) share one width and one x. Supported: Q4_K and Q6_K matrices
 * of 256 to 6144 columns that the fused GEMV takes (QK_EINVAL_SHAPE
 * otherwise).
 *
 * Each stage computes y = W x' for its GEMVs, with x' its input transform
 * (inputs[s]; inputs NULL: every stage QK_PASS_IN_PLAIN):
 *   QK_PASS_IN_PLAIN    x' = x;
 *   QK_PASS_IN_RMSNORM  x' = norm_w * (x / sqrt(mean(x^2) + eps)) (norm_w
 *                       NULL: weights of 1; eps > 0);
 *   QK_PASS_IN_SWIGLU   x' = silu(x) * aux (x the gate, aux the up values).
 * x and aux are each either exactly the output (y) of a GEMV of an earlier
 * stage whose rows equal the stage's width — the chain: the stage waits on
 * the device until that output is written — or memory that overlaps no
 * output (read as it is; it must not change while a run is in flight).
 * Anything else is QK_EINVAL_PTR, as is an output that overlaps a weight
 * matrix or another output, or a norm_w that overlaps an output. x, aux and
 * norm_w 16-byte aligned.
 *
 * Results: a stage with a plain input is exactly qk_gemv_batch on that x
 * (the same kernels' arithmetic, bit for bit); with a transform, within the
 * tolerance of qk_gemv against W applied to x' computed in fp64 (silu with
 * the hardware exponential and reciprocal, a few ulps). Repeated runs give
 * the same bits.
 *
 * workspace: caller-owned device memory, 256-byte aligned, of at least
 * qk_gemv_pass_workspace_bytes(the same descs, n, stage, inputs) bytes
 * (which checks them as qk_gemv_pass_create does), holding the stage table,
 * the run's words and a mirror of every output that a later stage reads;
 * qk_gemv_pass_create writes it with blocking copies (not under graph
 * capture), and it must stay valid, untouched by anything else and apart
 * from every matrix, input and output, until the pass is destroyed. The pass
 * belongs to the device that is current at creation. Runs of one pass that
 * overlap in time (two streams) race; runs ordered on one stream do not, and
 * a run may be captured in a HIP graph and replayed. qk_gemv_pass_create
 * allocates only the host handle; a run allocates nothing.
 *
 * Every wait in a run is bounded: after qk_gemv_pass_set_spin_limit polls
 * of one piece of an input (default 65536, ~0.07 s) it gives up, marks the
 * run and goes on, so a run always ends; the outputs of a marked run are not
 * to be trusted. qk_gemv_pass_gave_up (synchronous) returns 1 if the last
 * finished run was marked, else 0. qk_gemv_pass_grid returns the run's
 * workgroup count. */
typedef enum { QK_PASS_IN_PLAIN = 0, QK_PASS_IN_RMSNORM = 1, QK_PASS_IN_SWIGLU = 2 } qk_pass_input_kind;
typedef struct qk_gemv_pass_input {
    int kind;             /* qk_pass_input_kind */
    const float *aux;     /* SWIGLU: fp32[cols], the up values */
    const float *norm_w;  /* RMSNORM: fp32[cols] weights, or NULL */
    float eps;            /* RMSNORM */
} qk_gemv_pass_input;
typedef struct qk_gemv_pass qk_gemv_pass;
int64_t qk_gemv_pass_workspace_bytes(const qk_gemv_desc *descs, int n, const int *stage,
                                     const qk_gemv_pass_input *inputs);
int qk_gemv_pass_create(const qk_gemv_desc *descs, int n, const int *stage, const qk_gemv_pass_input *inputs,
                        void *workspace, int64_t workspace_bytes, qk_gemv_pass **out);
int qk_gemv_pass_run(const qk_gemv_pass *pass, void *stream);
int qk_gemv_pass_set_spin_limit(qk_gemv_pass *pass, int64_t polls);
int qk_gemv_pass_gave_up(const qk_gemv_pass *pass);
int qk_gemv_pass_grid(const qk_gemv_pass *pass);
void qk_gemv_pass_destroy(qk_gemv_pass *pass);

/* Y = X W^T for M activation rows: Y[m][r] = sum_c w[r][c] * X[m][c], with
 * X bfloat16 [M][cols] row-major (as uint16 bit patterns), Y fp32 [M][rows]
 * row-major (overwritten). The pages' engines run the prompt one position at
 * a time through the GEMV ("picoLM, in Python", §4 — The forward pass: no
 * batched prefill); with M positions at once the product is a dense
 * contraction, so it runs on the matrix cores for rows of whole 256-column
 * steps (every K-quant row; q8_0, q4_0, Q8_0_F16 and Q5_1 rows of a multiple
 * of 8 blocks): M up to 16 in a batched GEMV that streams W once, larger M in
 * a prefill tile kernel. The operands are exact where the format allows
 * (Q4_K, Q6_K, q8_0, q4_0, Q8_0_F16: integer codes as bf16 with the block
 * scales applied in fp32 in the small-M kernel; Q6_K's sc*(q-32) split into
 * two bf16 and the codes of the 32-weight formats in the prefill kernel);
 * otherwise (Q4_K in the prefill kernel, Q5_K, Q2_K, Q3_K, Q5_1) each fp32
 * weight is split into a bf16 pair within 2^-17 of it. Other rows run a row
 * kernel that reads W once per 8 rows of X.
 * Same tolerance as qk_gemv, per output; repeated calls give identical Y.
 * When few row tiles would leave CUs idle, the small-M kernel runs after a
 * fill that zeroes Y, and two workgroups add their halves of each row's sum
 * into it (two addends: the order does not change the result); Y must not
 * overlap W or X. M == 0 or rows == 0 is a no-op; cols == 0 writes Y = 0. */
int qk_gemm_prefill(int type, const void *W, int64_t rows, int64_t cols,
                    const uint16_t *X, int64_t M, float *Y, void *stream);

/* Which kernel qk_gemm_prefill runs for this format, shape and M (host-side,
 * launches nothing): QK_GEMM_PATH_ROWS, the row kernel (q8_0, q4_0,
 * Q8_0_F16 and Q5_1 rows that are not whole 256-column steps, and rows of
 * 2^26 columns or more);
 * QK_GEMM_PATH_FEW, the few-token kernel (M <= 16: W streams once through
 * the matrix cores); QK_GEMM_PATH_PREFILL, the prefill kernel (M > 16). The
 * tuning key QK_TUNE_GEMM_PATH forces a kernel where it applies, here as in
 * qk_gemm_prefill. Returns QK_EINVAL_TYPE, or QK_EINVAL_SHAPE for rows, cols
 * or M < 1 or cols not a multiple of the block size. */
typedef enum { QK_GEMM_PATH_ROWS = 0, QK_GEMM_PATH_FEW = 3, QK_GEMM_PATH_PREFILL = 4 } qk_gemm_path;
int qk_gemm_kernel_path(int type, int64_t rows, int64_t cols, int64_t M);

/* A static, human-readable name for a status code. */
const char *qk_strerror(int status);

/* The message of the last QK_EHIP (or argument error) on the calling
 * thread; "" if none. The pointer stays valid until the thread's next call.
 * qk_last_error is the same function under a shorter name. */
const char *qk_last_hip_error(void);
const char *qk_last_error(void);

/* Tuning overrides of the type-dispatch table, process-wide, for sweeps and
 * for tests that force one kernel. Each key holds -1 (the table's own
 * choice, the default) or a value:
 *   QK_TUNE_GEMV_STREAM      0: fused GEMVs read rows straight from HBM;
 *                            1: they stream row groups through LDS where the
 *                            streamed mode applies;
 *   QK_TUNE_GEMV_WGS_PER_CU  n >= 1: fused-GEMV workgroups per CU;
 *   QK_TUNE_GEMV_SLOT        32 or 64: lanes per row slot of rows split over
 *                            waves (where that width gives a plan);
 *   QK_TUNE_GEMV_NWR         n >= 1: row waves per GEMV workgroup (if the
 *                            launch bounds allow);
 *   QK_TUNE_GEMM_PATH        a qk_gemm_path value, where it applies;
 *   QK_TUNE_GEMM_KSPLIT      1 or 2: prefill super-blocks split over two
 *                            halves of a workgroup (2) or not (1);
 *   QK_TUNE_FEW_ROWS         8 or 16: few-token weight rows per wave at
 *                            M > 8 (8: two token sets of 8);
 *   QK_TUNE_FEW_KSW          n >= 1: few-token waves per workgroup;
 *   QK_TUNE_FEW_DEPTH        1 or 2: few-token steps of loads in flight;
 *   QK_TUNE_PREFILL_TOKENS   64 or 128: tokens per prefill workgroup.
 * Values are read on every launch, without any other synchronisation: set
 * them while no other thread launches. Results stay within the same
 * tolerance under every setting. qk_set_tuning returns the previous value;
 * both calls return QK_EINVAL_SHAPE for an unknown key or a value below -1.
 * The environment is never read. */
typedef enum {
    QK_TUNE_GEMV_STREAM = 0,
    QK_TUNE_GEMV_WGS_PER_CU = 1,
    QK_TUNE_GEMV_SLOT = 2,
    QK_TUNE_GEMV_NWR = 3,
    QK_TUNE_GEMM_PATH = 4,
    QK_TUNE_GEMM_KSPLIT = 5,
    QK_TUNE_FEW_ROWS = 6,
    QK_TUNE_FEW_KSW = 7,
    QK_TUNE_FEW_DEPTH = 8,
    QK_TUNE_PREFILL_TOKENS = 9,
    QK_TUNE_COUNT = 10
} qk_tune_key;
int qk_set_tuning(int key, int value);
int qk_get_tuning(int key);

#ifdef __cplusplus
}
#endif

#endif /* QK_H */

"""GPU parity over every value the formats' fields can hold.

The workload generators draw Q6_K scales from [-64, 63], positive fp16
scales and q8_0 codes from [-127, 127]. The formats themselves allow more:
Q6_K's scales are int8 ("PicoLM Q6_K量化Bug调试全记录", 原理: int8 scales[16]),
q8_0's codes are int8 (PETIT README, "How the pieces match"), and an fp16 or
fp32 scale may be negative, subnormal or zero. Here every kernel that decodes
weights runs on blocks drawn over those whole ranges (synth.blocks(...,
full=True): Q6_K scales -128..127, q8_0/Q8_0_F16 codes -128..127, scales
with random signs, 1/8 subnormal, 1/32 zero; q8_0 fp32 scales down to
subnormals),
against the oracle: dequantisation bit for bit, every GEMV read mode
(direct, streamed, wide-row, generic), the grouped launch, and every GEMM
path (few-token at every M from 1 to 16, prefill at M = 17, 64 and 512, row
kernel) element by element within |y - y_ref| <= 1e-4 * sum|w*x| + 1e-6, at
the full 2048 x 5632, 5632 x 2048 and 4096 x 11008 shapes."""
import numpy as np
import pytest

from block_quantized_weight_gemv_amd import synth
from gpu_helpers import assert_gemv_close, check_guard, guarded, to_dev

pytestmark = pytest.mark.gpu

Q4_0, Q8_0, Q4_K, Q6_K = 1, 2, 3, 4
Q8_0_F16, Q5_1, Q5_K, Q2_K, Q3_K = 5, 6, 7, 8, 9
ALL = [Q4_0, Q8_0, Q4_K, Q6_K, Q8_0_F16, Q5_1, Q5_K, Q2_K, Q3_K]


@pytest.fixture(scope="module")
def qk():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_quantized_weight_gemv_amd import qk as mod

    return mod


def full_matrix(t, rows, cols, seed):
    return synth.matrix(t, rows, cols, seed, stream=50 + t, full=True)


@pytest.mark.parametrize("t", ALL, ids=lambda t: synth.NAMES[t])
def test_dequant_full_range_bit_exact(qk, orc, t):
    import torch

    nb = 2048
    blocks = synth.blocks(t, nb, synth.rng(7, t), full=True)
    n = nb * synth.BLOCK_ELEMS[t]
    buf, out = guarded(n)
    qk.qk_dequantize_row(t, to_dev(blocks), n, out)
    torch.cuda.synchronize()
    check_guard(buf, n)
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), orc.dequantize_row(t, blocks, n).view(np.uint32))


def run_gemv(qk, t, W, rows, cols, x):
    import torch

    buf, y = guarded(rows)
    qk.qk_gemv(t, to_dev(W), rows, cols, to_dev(x), y)
    torch.cuda.synchronize()
    check_guard(buf, rows)
    return y.cpu().numpy()


# decode-pass and config shapes (direct / streamed), wide rows, the generic
# kernel (more than 512 units per row), odd Q6_K block counts at odd row
# counts, and the ggml formats
GEMV = [(Q6_K, 2048, 5632), (Q6_K, 256, 2048), (Q6_K, 32000, 2048), (Q4_K, 5632, 2048), (Q4_K, 512, 2048),
        (Q8_0, 2048, 2048), (Q8_0, 5632, 2048), (Q4_0, 2048, 2048), (Q6_K, 4096, 11008), (Q4_K, 4096, 14336),
        (Q6_K, 3, 256 * 130), (Q4_K, 3, 256 * 130), (Q6_K, 255, 768), (Q6_K, 1, 256), (Q6_K, 4095, 11008),
        (Q8_0_F16, 512, 2048), (Q5_1, 512, 2048), (Q5_K, 512, 2048), (Q2_K, 512, 2048), (Q3_K, 512, 2048)]


@pytest.mark.parametrize("mode", ["auto", "direct", "streamed"])
@pytest.mark.parametrize("t,rows,cols", GEMV, ids=[f"{synth.NAMES[t]}-{r}x{c}" for t, r, c in GEMV])
def test_gemv_full_range(qk, orc, t, rows, cols, mode):
    W = full_matrix(t, rows, cols, seed=rows + cols)
    x = synth.vector(cols, seed=rows + cols)
    with qk.tuning(gemv_stream={"auto": None, "direct": 0, "streamed": 1}[mode]):
        y = run_gemv(qk, t, W, rows, cols, x)
    y_ref, a = orc.gemv(t, W, rows, cols, x)
    assert_gemv_close(y, y_ref, a, f"full-range {synth.NAMES[t]} {rows}x{cols} {mode}")


def test_gemv_batch_full_range(qk, orc):
    """One decoder layer's grouped launches (Q4_K and Q6_K sharing launches)
    over full-range blocks."""
    import torch

    layer = [(Q4_K, 2048, 2048, 0), (Q4_K, 256, 2048, 0), (Q6_K, 256, 2048, 0), (Q4_K, 2048, 2048, 1),
             (Q4_K, 5632, 2048, 2), (Q4_K, 5632, 2048, 2), (Q6_K, 2048, 5632, 3)]
    xs = {i: synth.vector(c, seed=90 + i) for _, _, c, i in layer}
    xd = {i: to_dev(v) for i, v in xs.items()}
    Ws = [full_matrix(t, r, c, seed=91 + k) for k, (t, r, c, _) in enumerate(layer)]
    ys = [torch.empty(r, device="cuda") for _, r, _, _ in layer]
    Wd = [to_dev(W) for W in Ws]
    qk.qk_gemv_batch([(t, Wd[k], r, c, xd[i], ys[k]) for k, (t, r, c, i) in enumerate(layer)])
    torch.cuda.synchronize()
    for k, (t, r, c, i) in enumerate(layer):
        y_ref, a = orc.gemv(t, Ws[k], r, c, xs[i])
        assert_gemv_close(ys[k].cpu().numpy(), y_ref, a, f"batch full-range {synth.NAMES[t]} {r}x{c}")


def run_gemm(qk, t, Wd, rows, cols, X, M):
    import torch

    buf, Y = guarded(M * rows)
    qk.qk_gemm_prefill(t, Wd, rows, cols, to_dev(X.view(np.int16)), M, Y)
    torch.cuda.synchronize()
    check_guard(buf, M * rows)
    return Y.cpu().numpy().reshape(M, rows)


@pytest.mark.parametrize("t,rows,cols", [(Q6_K, 2048, 5632), (Q4_K, 5632, 2048), (Q6_K, 4096, 11008)],
                         ids=["q6k-2048x5632", "q4k-5632x2048", "q6k-4096x11008"])
@pytest.mark.parametrize("rpw", [None, 8, 16], ids=["rows-auto", "rows-8", "rows-16"])
def test_few_token_every_m_full_range_full_shape(qk, orc, t, rows, cols, rpw):
    """The few-token kernel at every M from 1 to 16 on the whole matrix,
    every output checked; above 8 tokens with the rows per wave the
    launcher picks and with 8 (two token sets) and 16 forced."""
    W = full_matrix(t, rows, cols, seed=17)
    Wd = to_dev(W)
    Ms = range(1, 17) if rows * cols <= 2048 * 5632 else (1, 2, 3, 5, 8, 11, 16)
    with qk.tuning(gemm_path=qk.QK_GEMM_PATH_FEW, few_rows=rpw):
        for M in Ms:
            X = synth.bf16_matrix(M, cols, seed=300 + M)
            Y = run_gemm(qk, t, Wd, rows, cols, X, M)
            Y_ref, A = orc.gemm(t, W, rows, cols, X, M)
            assert_gemv_close(Y, Y_ref, A, f"few-token full-range {synth.NAMES[t]} {rows}x{cols} M={M} rows={rpw}")


@pytest.mark.parametrize("t,rows,cols", [(Q6_K, 2048, 5632), (Q4_K, 5632, 2048), (Q6_K, 4096, 11008),
                                          (Q6_K, 4095, 11008), (Q8_0_F16, 5632, 2048)],
                         ids=["q6k-2048x5632", "q4k-5632x2048", "q6k-4096x11008", "q6k-4095x11008",
                              "q8_0_f16-5632x2048"])
@pytest.mark.parametrize("M", [17, 64, 512])
@pytest.mark.parametrize("ksplit,tok", [(None, None), (1, None), (2, None), (None, 64), (1, 128), (2, 128)],
                         ids=["ks-auto", "ks-1", "ks-2", "tok-64", "tok-128-ks-1", "tok-128-ks-2"])
def test_prefill_full_range_full_shape(qk, orc, t, rows, cols, M, ksplit, tok):
    """The prefill kernel at M = 17, 64 and 512 on the whole matrix, with
    either tile width and split; every output checked below M = 512, and at
    M = 512 every output of 256 sampled weight rows (the first and the last
    among them)."""
    W = full_matrix(t, rows, cols, seed=18)
    X = synth.bf16_matrix(M, cols, seed=400 + M)
    with qk.tuning(gemm_path=qk.QK_GEMM_PATH_PREFILL, gemm_ksplit=ksplit, prefill_tokens=tok):
        Y = run_gemm(qk, t, to_dev(W), rows, cols, X, M)
    if M < 512:
        Y_ref, A = orc.gemm(t, W, rows, cols, X, M)
        assert_gemv_close(Y, Y_ref, A, f"prefill full-range {synth.NAMES[t]} {rows}x{cols} M={M}")
        return
    rb = synth.row_bytes(t, cols)
    sample = sorted(set([0, 1, rows - 1] + list(synth.rng(18, 5).integers(0, rows, 253))))
    Ws = np.concatenate([W[r * rb:(r + 1) * rb] for r in sample])
    Y_ref, A = orc.gemm(t, Ws, len(sample), cols, X, M)
    assert_gemv_close(Y[:, sample], Y_ref, A, f"prefill full-range {synth.NAMES[t]} {rows}x{cols} M={M} sampled")


GGML = [(Q5_K, 5632, 2048), (Q2_K, 5632, 2048), (Q3_K, 2048, 5632), (Q3_K, 4095, 11008), (Q5_1, 5632, 2048)]


@pytest.mark.parametrize("t,rows,cols", GGML, ids=[f"{synth.NAMES[t]}-{r}x{c}" for t, r, c in GGML])
def test_ggml_few_token_every_m_full_range_full_shape(qk, orc, t, rows, cols):
    """Q5_K, Q2_K, Q3_K and Q5_1 on the few-token kernel at every M from 1
    to 16 (the 7B down shape at a few M) on the whole matrix, every output
    checked (Q3_K 4095 x 11008: 43 blocks per row, odd rows start 2 bytes
    past a 4-byte boundary)."""
    W = full_matrix(t, rows, cols, seed=21)
    Wd = to_dev(W)
    Ms = range(1, 17) if rows * cols <= 2048 * 5632 else (1, 5, 8, 13, 16)
    with qk.tuning(gemm_path=qk.QK_GEMM_PATH_FEW):
        for M in Ms:
            X = synth.bf16_matrix(M, cols, seed=700 + M)
            Y = run_gemm(qk, t, Wd, rows, cols, X, M)
            Y_ref, A = orc.gemm(t, W, rows, cols, X, M)
            assert_gemv_close(Y, Y_ref, A, f"few-token full-range {synth.NAMES[t]} {rows}x{cols} M={M}")


@pytest.mark.parametrize("t,rows,cols", GGML, ids=[f"{synth.NAMES[t]}-{r}x{c}" for t, r, c in GGML])
@pytest.mark.parametrize("M", [17, 512])
@pytest.mark.parametrize("ksplit,tok", [(None, None), (2, 64), (1, 128)], ids=["auto", "tok-64-ks-2", "tok-128-ks-1"])
def test_ggml_prefill_full_range_full_shape(qk, orc, t, rows, cols, M, ksplit, tok):
    """Q5_K, Q2_K, Q3_K and Q5_1 on the prefill kernel on the whole matrix:
    every output at M = 17, every output of 256 sampled rows at M = 512."""
    W = full_matrix(t, rows, cols, seed=22)
    X = synth.bf16_matrix(M, cols, seed=800 + M)
    with qk.tuning(gemm_path=qk.QK_GEMM_PATH_PREFILL, gemm_ksplit=ksplit, prefill_tokens=tok):
        Y = run_gemm(qk, t, to_dev(W), rows, cols, X, M)
    if M < 512:
        Y_ref, A = orc.gemm(t, W, rows, cols, X, M)
        assert_gemv_close(Y, Y_ref, A, f"prefill full-range {synth.NAMES[t]} {rows}x{cols} M={M}")
        return
    rb = synth.row_bytes(t, cols)
    sample = sorted(set([0, 1, rows - 1] + list(synth.rng(22, 5).integers(0, rows, 253))))
    Ws = np.concatenate([W[r * rb:(r + 1) * rb] for r in sample])
    Y_ref, A = orc.gemm(t, Ws, len(sample), cols, X, M)
    assert_gemv_close(Y[:, sample], Y_ref, A, f"prefill full-range {synth.NAMES[t]} {rows}x{cols} M={M} sampled")


@pytest.mark.parametrize("t", [Q8_0, Q4_0, Q8_0_F16, Q5_1, Q5_K, Q2_K, Q3_K], ids=lambda t: synth.NAMES[t])
@pytest.mark.parametrize("M", [3, 40])
def test_row_kernel_full_range(qk, orc, t, M):
    rows, cols = 96, 2048
    W = full_matrix(t, rows, cols, seed=19)
    X = synth.bf16_matrix(M, cols, seed=500 + M)
    with qk.tuning(gemm_path=qk.QK_GEMM_PATH_ROWS):  # (every format defaults to the MFMA kernels here)
        Y = run_gemm(qk, t, to_dev(W), rows, cols, X, M)
    Y_ref, A = orc.gemm(t, W, rows, cols, X, M)
    assert_gemv_close(Y, Y_ref, A, f"row kernel full-range {synth.NAMES[t]} M={M}")


PATHS = [(Q6_K, 130, 2816), (Q6_K, 65, 768), (Q4_K, 131, 2048), (Q8_0, 131, 2048), (Q8_0, 65, 768),
         (Q4_0, 130, 1280), (Q4_0, 33, 256), (Q8_0_F16, 131, 2048), (Q8_0_F16, 65, 768), (Q5_1, 131, 2048),
         (Q5_1, 65, 768), (Q5_K, 131, 2048), (Q2_K, 131, 2048), (Q3_K, 131, 2816), (Q3_K, 65, 768)]


@pytest.mark.parametrize("path", ["few", "prefill", "rows"])
@pytest.mark.parametrize("t,rows,cols", PATHS, ids=[f"{synth.NAMES[t]}-{r}x{c}" for t, r, c in PATHS])
def test_gemm_paths_full_range(qk, orc, t, rows, cols, path):
    """Every GEMM path forced on one matrix (ragged row tiles; odd Q6_K and
    Q3_K block counts with odd row counts, so that half of the rows start
    2 bytes past a 4-byte boundary; q8_0 and GGUF Q8_0 codes -128..127 and
    every format's scales of either sign, subnormal or zero, on the MFMA
    kernels too)."""
    W = full_matrix(t, rows, cols, seed=20)
    Wd = to_dev(W)
    force = {"few": qk.QK_GEMM_PATH_FEW, "prefill": qk.QK_GEMM_PATH_PREFILL, "rows": qk.QK_GEMM_PATH_ROWS}[path]
    with qk.tuning(gemm_path=force):
        for M in ((1, 7, 16) if path == "few" else (1, 16, 33, 100)):
            X = synth.bf16_matrix(M, cols, seed=600 + M)
            Y = run_gemm(qk, t, Wd, rows, cols, X, M)
            Y_ref, A = orc.gemm(t, W, rows, cols, X, M)
            assert_gemv_close(Y, Y_ref, A, f"{path} full-range {synth.NAMES[t]} {rows}x{cols} M={M}")

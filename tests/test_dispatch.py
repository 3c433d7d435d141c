"""The type-dispatch table on the host (no GPU): qk_gemv_kernel_path and
qk_gemm_kernel_path report the kernel qk_gemv / qk_gemm_prefill runs for a
format and shape, from the same decisions the launchers take. Pins each rule
at its edges. GEMV:

* the fused kernels take rows of up to 512 units (64-weight units for the
  K-quants, 32-weight blocks for the others); one unit more runs the generic
  kernel;
* rows wider than 6144 columns run the wide-row kernel;
* q4_0 and Q8_0_F16 need an even block count per row; Q3_K an even block
  count or an even row count (the matrix's last block must not start on a
  4-byte boundary); Q6_K takes any shape;
* launches of at least 128 MiB whose rows one wave covers stream their row
  groups through LDS, except q4_0, and only when the matrix is a whole
  number of 16-byte pieces; the tuning key QK_TUNE_GEMV_STREAM overrides;
* bad types and shapes are errors.

GEMM: Q4_K and Q6_K take the few-token kernel for M <= 16 and the prefill
kernel above, at every shape; every other format the row kernel;
QK_TUNE_GEMM_PATH forces a kernel where it applies.
"""
import pytest

from block_quantized_weight_gemv_amd import qk

Q4_0, Q8_0, Q4_K, Q6_K = 1, 2, 3, 4
Q8_0_F16, Q5_1, Q5_K, Q2_K, Q3_K = 5, 6, 7, 8, 9
GENERIC, FUSED, STREAMED, WIDE = qk.QK_PATH_GENERIC, qk.QK_PATH_FUSED, qk.QK_PATH_STREAMED, qk.QK_PATH_WIDE
MiB = 1 << 20


@pytest.fixture(autouse=True)
def no_override():
    for k in range(8):
        assert qk.qk_get_tuning(k) == -1, "a tuning override leaked from another test"


def rows_for(t, cols, nbytes):
    """The fewest rows of cols columns that make at least nbytes."""
    rb = qk.qk_row_bytes(t, cols)
    return -(-nbytes // rb)


CASES = [
    # the decode pass and the configurations' shapes: direct
    (Q4_K, 512, 2048, FUSED), (Q6_K, 2048, 5632, FUSED), (Q4_K, 5632, 2048, FUSED), (Q6_K, 32000, 2048, FUSED),
    (Q8_0, 5632, 2048, FUSED), (Q4_0, 5632, 2048, FUSED),
    # units per row: 512 is the widest fused row, one more is generic
    (Q4_K, 9, 32768, WIDE), (Q4_K, 9, 32768 + 256, GENERIC), (Q8_0, 7, 16384, WIDE), (Q8_0, 7, 16384 + 32, GENERIC),
    (Q5_1, 3, 16384, WIDE), (Q5_1, 3, 16416, GENERIC),
    # the register staging holds 6144 columns; wider rows take the wide-row kernel
    (Q4_K, 64, 6144, FUSED), (Q4_K, 64, 6400, WIDE), (Q6_K, 4096, 11008, WIDE), (Q8_0, 40, 6144, FUSED),
    (Q8_0, 40, 6176, WIDE),
    # block-count parity
    (Q4_0, 8, 96, GENERIC), (Q4_0, 8, 128, FUSED), (Q8_0_F16, 8, 96, GENERIC), (Q8_0_F16, 8, 128, FUSED),
    (Q6_K, 255, 768, FUSED), (Q6_K, 256, 768, FUSED), (Q6_K, 1, 256, FUSED), (Q6_K, 2, 256, FUSED),
    (Q6_K, 4095, 11008, WIDE), (Q3_K, 255, 768, GENERIC), (Q3_K, 256, 768, FUSED),
    (Q3_K, 63, 11008, GENERIC), (Q3_K, 64, 11008, WIDE), (Q4_K, 255, 768, FUSED), (Q2_K, 255, 768, FUSED),
    (Q5_K, 255, 768, FUSED),
]


@pytest.mark.parametrize("t,rows,cols,path", CASES, ids=[f"{t}-{r}x{c}" for t, r, c, _ in CASES])
def test_kernel_path(t, rows, cols, path):
    assert qk.qk_gemv_kernel_path(t, rows, cols) == path


def test_streamed_threshold():
    """128 MiB of packed weights switches rows that one wave covers to the
    streamed mode; rows split over waves (5632 columns), q4_0, and the wide
    rows never stream."""
    for t in (Q4_K, Q6_K, Q8_0, Q5_K, Q8_0_F16):
        r = rows_for(t, 2048, 128 * MiB)
        r += r % 2
        assert qk.qk_gemv_kernel_path(t, r, 2048) == STREAMED, t
        assert qk.qk_gemv_kernel_path(t, r - 16, 2048) == FUSED, t
    assert qk.qk_gemv_kernel_path(Q4_0, rows_for(Q4_0, 2048, 1 << 30), 2048) == FUSED
    assert qk.qk_gemv_kernel_path(Q6_K, rows_for(Q6_K, 5632, 1 << 30), 5632) == FUSED
    assert qk.qk_gemv_kernel_path(Q4_K, rows_for(Q4_K, 14336, 1 << 30), 14336) == WIDE


def test_streamed_needs_whole_16_byte_pieces():
    """Q6_K rows of 3 blocks are 630 bytes: 300000 rows make a whole number
    of 16-byte pieces, 300002 do not (the direct mode then)."""
    assert (300000 * 630) % 16 == 0 and (300002 * 630) % 16 != 0
    assert qk.qk_gemv_kernel_path(Q6_K, 300000, 768) == STREAMED
    assert qk.qk_gemv_kernel_path(Q6_K, 300002, 768) == FUSED


def test_stream_override():
    big = rows_for(Q4_K, 2048, 1 << 30)
    with qk.tuning(gemv_stream=0):
        assert qk.qk_gemv_kernel_path(Q4_K, big, 2048) == FUSED
    with qk.tuning(gemv_stream=1):
        assert qk.qk_gemv_kernel_path(Q4_K, 512, 2048) == STREAMED
        assert qk.qk_gemv_kernel_path(Q4_0, 512, 2048) == FUSED  # q4_0 never streams
        assert qk.qk_gemv_kernel_path(Q6_K, 2048, 5632) == FUSED  # nor rows split over waves


def test_transformed_input_follows_the_fused_kernels():
    """A transformed input (RMSNorm / SwiGLU inside the GEMV) is offered for
    the K-quant and q4_0/q8_0 families wherever their fused kernels run."""
    for t, r, c, path in CASES:
        if t in (Q4_K, Q6_K, Q4_0, Q8_0):
            assert qk.qk_gemv_input_supported(t, r, c) == (path != GENERIC), (t, r, c)
        else:
            assert not qk.qk_gemv_input_supported(t, r, c)


def test_errors():
    with pytest.raises(qk.QkError):
        qk.qk_gemv_kernel_path(10, 4, 256)
    with pytest.raises(qk.QkError):
        qk.qk_gemv_kernel_path(Q4_K, 4, 255)
    with pytest.raises(qk.QkError):
        qk.qk_gemv_kernel_path(Q4_K, 0, 256)
    assert qk.lib.qk_gemv_kernel_path(10, 4, 256) == qk.QK_EINVAL_TYPE
    assert qk.lib.qk_gemv_kernel_path(Q4_K, 4, 100) == qk.QK_EINVAL_SHAPE


GEMM = [
    (Q4_K, 5632, 2048, 2, qk.QK_GEMM_PATH_FEW), (Q4_K, 5632, 2048, 16, qk.QK_GEMM_PATH_FEW),
    (Q4_K, 5632, 2048, 17, qk.QK_GEMM_PATH_PREFILL), (Q4_K, 5632, 2048, 512, qk.QK_GEMM_PATH_PREFILL),
    (Q6_K, 2048, 5632, 8, qk.QK_GEMM_PATH_FEW), (Q6_K, 2048, 5632, 512, qk.QK_GEMM_PATH_PREFILL),
    (Q6_K, 4096, 11008, 8, qk.QK_GEMM_PATH_FEW), (Q6_K, 4096, 11008, 512, qk.QK_GEMM_PATH_PREFILL),
    (Q6_K, 4095, 11008, 8, qk.QK_GEMM_PATH_FEW), (Q6_K, 4095, 11008, 512, qk.QK_GEMM_PATH_PREFILL),
    (Q6_K, 1, 256, 5, qk.QK_GEMM_PATH_FEW), (Q6_K, 1, 256, 50, qk.QK_GEMM_PATH_PREFILL),
    (Q6_K, 4095, 5632, 8, qk.QK_GEMM_PATH_FEW), (Q4_K, 4095, 11008, 8, qk.QK_GEMM_PATH_FEW),
    (Q4_K, 1, 256, 1, qk.QK_GEMM_PATH_FEW),
    # 2^26 columns and more: the row kernel (the MFMA kernels' buffers stay under 2 GiB)
    (Q4_K, 4, (1 << 26) - 256, 8, qk.QK_GEMM_PATH_FEW), (Q4_K, 4, 1 << 26, 8, qk.QK_GEMM_PATH_ROWS),
    (Q6_K, 4, 1 << 26, 512, qk.QK_GEMM_PATH_ROWS),
    # q8_0 and q4_0: the MFMA kernels when a row is whole 256-column steps
    (Q8_0, 2048, 2048, 8, qk.QK_GEMM_PATH_FEW), (Q4_0, 2048, 2048, 512, qk.QK_GEMM_PATH_PREFILL),
    (Q8_0, 5632, 2048, 16, qk.QK_GEMM_PATH_FEW), (Q4_0, 5632, 2048, 17, qk.QK_GEMM_PATH_PREFILL),
    (Q8_0, 64, 2080, 8, qk.QK_GEMM_PATH_ROWS), (Q4_0, 64, 96, 512, qk.QK_GEMM_PATH_ROWS),
    # the ggml formats: the same rule (the K-quants' rows are always whole steps)
    (Q8_0_F16, 64, 2048, 4, qk.QK_GEMM_PATH_FEW), (Q8_0_F16, 5632, 2048, 512, qk.QK_GEMM_PATH_PREFILL),
    (Q8_0_F16, 64, 2080, 8, qk.QK_GEMM_PATH_ROWS),
    (Q5_K, 2048, 2048, 512, qk.QK_GEMM_PATH_PREFILL), (Q5_K, 2048, 2048, 16, qk.QK_GEMM_PATH_FEW),
    (Q5_1, 64, 2048, 4, qk.QK_GEMM_PATH_FEW), (Q5_1, 64, 2048, 17, qk.QK_GEMM_PATH_PREFILL),
    (Q5_1, 64, 2080, 4, qk.QK_GEMM_PATH_ROWS), (Q5_1, 64, 96, 512, qk.QK_GEMM_PATH_ROWS),
    (Q2_K, 64, 2048, 64, qk.QK_GEMM_PATH_PREFILL), (Q2_K, 64, 2048, 1, qk.QK_GEMM_PATH_FEW),
    (Q3_K, 64, 2048, 8, qk.QK_GEMM_PATH_FEW), (Q3_K, 65, 768, 100, qk.QK_GEMM_PATH_PREFILL),
    (Q3_K, 4, 1 << 26, 8, qk.QK_GEMM_PATH_ROWS),
]


@pytest.mark.parametrize("t,rows,cols,M,path", GEMM, ids=[f"{t}-{r}x{c}-M{m}" for t, r, c, m, _ in GEMM])
def test_gemm_kernel_path(t, rows, cols, M, path):
    assert qk.qk_gemm_kernel_path(t, rows, cols, M) == path


def test_gemm_path_override():
    with qk.tuning(gemm_path=qk.QK_GEMM_PATH_ROWS):
        assert qk.qk_gemm_kernel_path(Q4_K, 5632, 2048, 512) == qk.QK_GEMM_PATH_ROWS
    with qk.tuning(gemm_path=qk.QK_GEMM_PATH_FEW):
        assert qk.qk_gemm_kernel_path(Q4_K, 5632, 2048, 8) == qk.QK_GEMM_PATH_FEW
        # the few-token kernel takes M <= 16: larger M keeps the table's choice
        assert qk.qk_gemm_kernel_path(Q4_K, 5632, 2048, 64) == qk.QK_GEMM_PATH_PREFILL
    with qk.tuning(gemm_path=qk.QK_GEMM_PATH_PREFILL):
        assert qk.qk_gemm_kernel_path(Q6_K, 4095, 11008, 8) == qk.QK_GEMM_PATH_PREFILL
        assert qk.qk_gemm_kernel_path(Q8_0, 64, 2048, 8) == qk.QK_GEMM_PATH_PREFILL
        assert qk.qk_gemm_kernel_path(Q8_0_F16, 64, 2048, 8) == qk.QK_GEMM_PATH_PREFILL
        assert qk.qk_gemm_kernel_path(Q5_K, 64, 2048, 8) == qk.QK_GEMM_PATH_PREFILL
        # no MFMA kernel for a q8_0 or Q5_1 row of 65 blocks
        assert qk.qk_gemm_kernel_path(Q8_0, 64, 2080, 64) == qk.QK_GEMM_PATH_ROWS
        assert qk.qk_gemm_kernel_path(Q5_1, 64, 2080, 64) == qk.QK_GEMM_PATH_ROWS


def test_gemm_path_errors():
    assert qk.lib.qk_gemm_kernel_path(10, 4, 256, 4) == qk.QK_EINVAL_TYPE
    assert qk.lib.qk_gemm_kernel_path(Q4_K, 4, 100, 4) == qk.QK_EINVAL_SHAPE
    assert qk.lib.qk_gemm_kernel_path(Q4_K, 4, 256, 0) == qk.QK_EINVAL_SHAPE

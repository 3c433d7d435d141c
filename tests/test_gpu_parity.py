"""GPU parity: every kernel through the C ABI against the CPU oracle.

Dequantisation is compared bit for bit; GEMV/GEMM outputs element by element
within |y - y_ref| <= 1e-4 * sum|w*x| + 1e-6. Shapes cover several tiles and
ragged row tails, the full TinyLlama-1.1B shapes of the decode-step weight
pass, both GEMV code paths (even and odd block counts per row), and the
degenerate cases (one row, one block, empty matrices)."""
import numpy as np
import pytest

import pins
from block_quantized_weight_gemv_amd import synth
from gpu_helpers import assert_gemv_close, check_guard, gemv_case, guarded, to_dev

pytestmark = pytest.mark.gpu

Q4_0, Q8_0, Q4_K, Q6_K = 1, 2, 3, 4
ALL = [Q4_K, Q6_K, Q8_0, Q4_0]
QK = {Q4_K: 256, Q6_K: 256, Q8_0: 32, Q4_0: 32}


@pytest.fixture(scope="module")
def qk():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_quantized_weight_gemv_amd import qk as mod

    return mod


def run_dequant(qk, t, blocks_np, n):
    import torch

    buf, out = guarded(n)
    qk.qk_dequantize_row(t, to_dev(blocks_np), n, out)
    torch.cuda.synchronize()
    check_guard(buf, n)
    return out.cpu().numpy()


def run_gemv(qk, t, W_np, rows, cols, x_np):
    import torch

    buf, y = guarded(rows)
    qk.qk_gemv(t, to_dev(W_np), rows, cols, to_dev(x_np), y)
    torch.cuda.synchronize()
    check_guard(buf, rows)
    return y.cpu().numpy()


# ------------------------------------------------------------------ dequant

@pytest.mark.parametrize("t", ALL, ids=lambda t: synth.NAMES[t])
@pytest.mark.parametrize("nblocks", [1, 3, 64, 4097])
def test_dequant_bit_exact(qk, orc, t, nblocks):
    blocks = synth.blocks(t, nblocks, synth.rng(100 + nblocks, t))
    n = nblocks * QK[t]
    got = run_dequant(qk, t, blocks, n)
    ref = orc.dequantize_row(t, blocks, n)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_q6k_one_million(qk, orc):
    """The 2^20-weight Q6_K dequantisation check (4096 blocks)."""
    blocks = synth.matrix(Q6_K, 1, 1 << 20, seed=1, stream=7)
    got = run_dequant(qk, Q6_K, blocks, 1 << 20)
    ref = orc.dequantize_row(Q6_K, blocks, 1 << 20)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("name,t,n", [("q4k_h1.json", Q4_K, 256), ("q6k_h2.json", Q6_K, 256),
                                      ("q6k_h3.json", Q6_K, 256), ("q8_0_hand.json", Q8_0, 32),
                                      ("q4_0_hand.json", Q4_0, 32)])
def test_dequant_hand_blocks(qk, orc, name, t, n):
    blk = pins.block_of(pins.golden(name))
    got = run_dequant(qk, t, blk, n)
    assert np.array_equal(got.view(np.uint32), orc.dequantize_row(t, blk, n).view(np.uint32))


@pytest.mark.parametrize("t", ALL, ids=lambda t: synth.NAMES[t])
def test_dequant_extreme_scales(qk, orc, t):
    """Subnormal, zero and largest fp16 scales: still bit-exact."""
    blocks = synth.blocks(t, 16, synth.rng(5, t))
    if t == Q4_K:
        blocks[:8, 0:2] = np.array([0x0001, 0x03FF, 0x7BFF, 0x0000, 0x0400, 0x8001, 0xFBFF, 0x3C00],
                                   dtype=np.uint16).view(np.uint8).reshape(-1, 2)
        blocks[:8, 2:4] = blocks[:8, 0:2][::-1]
    elif t == Q6_K:
        blocks[:8, 208:210] = np.array([0x0001, 0x03FF, 0x7BFF, 0x0000, 0x0400, 0x8001, 0xFBFF, 0x3C00],
                                       dtype=np.uint16).view(np.uint8).reshape(-1, 2)
    elif t == Q4_0:
        blocks[:8, 0:2] = np.array([0x0001, 0x03FF, 0x7BFF, 0x0000, 0x0400, 0x8001, 0xFBFF, 0x3C00],
                                   dtype=np.uint16).view(np.uint8).reshape(-1, 2)
    else:
        blocks[:4, 0:4] = np.array([1e-30, 3.0e30, -2.5, 0.0], dtype=np.float32).view(np.uint8).reshape(-1, 4)
    n = 16 * QK[t]
    got = run_dequant(qk, t, blocks, n)
    assert np.array_equal(got.view(np.uint32), orc.dequantize_row(t, blocks, n).view(np.uint32))


# ------------------------------------------------------------------ GEMV

# (rows, cols) per format: tiles, ragged row tails, one row, one block,
# even and odd blocks per row, and more than 64 / more than 256 units per row.
SHAPES = {
    Q4_K: [(1, 256), (3, 512), (17, 2048), (255, 2048), (512, 2048), (33, 5632), (7, 1280), (5, 256 * 70)],
    Q6_K: [(1, 256), (3, 512), (17, 2048), (255, 768), (64, 5632), (9, 1280), (5, 256 * 70), (130, 2048)],
    Q8_0: [(1, 32), (3, 64), (17, 2048), (255, 96), (40, 5632), (7, 32 * 300), (2, 32 * 33)],
    Q4_0: [(1, 32), (3, 64), (17, 2048), (255, 96), (40, 5632), (7, 32 * 300), (2, 32 * 33), (5, 32 * 31)],
}
CASES = [(t, r, c) for t in ALL for (r, c) in SHAPES[t]]


@pytest.fixture(params=["auto", "streamed", "direct"])
def gemv_mode(request, qk):
    """Both ways the fused GEMV reads its rows (QK_TUNE_GEMV_STREAM):
    straight from HBM into registers, or streamed through LDS (where it
    applies; the library uses it by itself only for launches of >= 128
    MiB)."""
    val = {"auto": None, "streamed": 1, "direct": 0}[request.param]
    with qk.tuning(gemv_stream=val):
        yield request.param


@pytest.mark.parametrize("t,rows,cols", CASES, ids=[f"{synth.NAMES[t]}-{r}x{c}" for t, r, c in CASES])
def test_gemv_matches_oracle(qk, orc, t, rows, cols, gemv_mode):
    W, x = gemv_case(t, rows, cols, seed=rows * 7 + cols)
    y = run_gemv(qk, t, W, rows, cols, x)
    y_ref, a = orc.gemv(t, W, rows, cols, x)
    assert_gemv_close(y, y_ref, a, f"{synth.NAMES[t]} {rows}x{cols}")


# The configurations' full shapes (the TinyLlama-1.1B decode pass and the
# q8_0/q4_0 shapes), compared on every output.
FULL = [(Q4_K, 512, 2048, 0), (Q6_K, 2048, 5632, 1), (Q8_0, 2048, 2048, 2), (Q8_0, 5632, 2048, 2),
        (Q4_0, 2048, 2048, 2), (Q4_0, 5632, 2048, 2), (Q4_K, 2048, 2048, 3), (Q4_K, 256, 2048, 3),
        (Q6_K, 256, 2048, 3), (Q4_K, 5632, 2048, 3), (Q6_K, 32000, 2048, 3)]


@pytest.mark.parametrize("t,rows,cols,seed", FULL, ids=[f"{synth.NAMES[t]}-{r}x{c}" for t, r, c, s in FULL])
def test_gemv_full_shapes(qk, orc, t, rows, cols, seed, gemv_mode):
    W, x = gemv_case(t, rows, cols, seed)
    y = run_gemv(qk, t, W, rows, cols, x)
    y_ref, a = orc.gemv(t, W, rows, cols, x)
    assert_gemv_close(y, y_ref, a, f"{synth.NAMES[t]} {rows}x{cols}")


@pytest.mark.parametrize("t,rows,cols", [(Q4_K, 40, 2048), (Q6_K, 40, 5632), (Q8_0, 9, 2048), (Q4_0, 9, 2048),
                                          (Q6_K, 5, 1280), (Q4_0, 5, 32 * 31)])
def test_gemv_unit_vector_gives_column(qk, orc, t, rows, cols, gemv_mode):
    """x = e_k returns column k of the dequantised matrix exactly (IEEE
    equality: a -0.0 weight summed from +0 is +0, as in the oracle's GEMV)."""
    W, _ = gemv_case(t, rows, cols, seed=3)
    rb = len(W) // rows
    deq = np.stack([orc.dequantize_row(t, W[r * rb:(r + 1) * rb], cols) for r in range(rows)])
    for k in (0, 1, 31, 32, cols // 2 + 17, cols - 1):
        e = np.zeros(cols, dtype=np.float32)
        e[k] = 1.0
        y = run_gemv(qk, t, W, rows, cols, e)
        assert np.array_equal(y, deq[:, k]), k
        y_ref, _ = orc.gemv(t, W, rows, cols, e)
        assert np.array_equal(y.astype(np.float64).view(np.uint64), y_ref.view(np.uint64)), k


# Matrices past the size where the library streams rows through LDS by
# itself (>= 128 MiB), at the widths where it does; outputs checked on a
# sample of rows, including the first and the last, computed by the oracle.
BIG = [(Q4_K, 2048, 2048 * 64 + 5), (Q6_K, 2048, 1680 * 48 + 4), (Q8_0, 2048, 2304 * 40 + 8)]


@pytest.mark.parametrize("t,cols,rows", BIG, ids=[f"{synth.NAMES[t]}-{r}x{c}" for t, c, r in BIG])
def test_gemv_large_sampled(qk, orc, t, cols, rows):
    import torch

    rb = synth.row_bytes(t, cols)
    assert rows * rb >= 128 << 20
    # a seeded block of rows tiled over the matrix
    base_rows = 4096
    blk = synth.matrix(t, base_rows, cols, seed=12, stream=t)
    reps = -(-rows // base_rows)
    Wd = to_dev(blk).repeat(reps)[: rows * rb].contiguous()
    x = synth.vector(cols, seed=12)
    buf, y = guarded(rows)
    qk.qk_gemv(t, Wd, rows, cols, to_dev(x), y)
    torch.cuda.synchronize()
    check_guard(buf, rows)
    yh = y.cpu().numpy()
    sample = sorted(set([0, 1, 4095, 4096, rows - 2, rows - 1] + list(synth.rng(12, 98).integers(0, rows, 60))))
    for r in sample:
        b = r % base_rows
        yr, ar = orc.gemv(t, blk[b * rb:(b + 1) * rb], 1, cols, x)
        assert_gemv_close(yh[r:r + 1], yr, ar, f"row {r}")


def test_gemv_h1_sum(qk):
    """The hand block H1 against x = 1 gives exactly 50000."""
    blk = pins.block_of(pins.golden("q4k_h1.json"))
    y = run_gemv(qk, Q4_K, blk, 1, 256, np.ones(256, dtype=np.float32))
    assert y[0] == 50000.0


def test_gemv_integer_exact(qk, orc):
    """d = dmin = 1 and small integer x: every partial sum is an integer
    below 2^24, so the GPU result equals the oracle exactly."""
    rows, cols = 64, 2048
    W = synth.matrix(Q4_K, rows, cols, seed=9).reshape(-1, 144)
    W[:, 0:4] = np.array([0x3C00, 0x3C00], dtype=np.uint16).view(np.uint8)
    W = W.reshape(-1)
    x = synth.rng(9, 1).integers(-3, 4, cols).astype(np.float32)
    y = run_gemv(qk, Q4_K, W, rows, cols, x)
    y_ref, _ = orc.gemv(Q4_K, W, rows, cols, x)
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_gemv_empty_and_zero_cols(qk):
    import torch

    y = torch.full((5,), 7.0, device="cuda")
    qk.qk_gemv(Q4_K, None, 0, 2048, None, y)  # no rows: nothing written
    qk.qk_gemv(Q4_K, None, 5, 0, None, y)     # no columns: empty sums
    torch.cuda.synchronize()
    assert y.cpu().tolist() == [0.0] * 5


def test_gemv_on_side_stream(qk, orc):
    """Work enqueued on a non-default torch stream is ordered on that stream."""
    import torch

    W, x = gemv_case(Q6_K, 2048, 2048, seed=21)
    Wd, xd = to_dev(W), to_dev(x)
    y = torch.empty(2048, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y.fill_(float("nan"))
        for _ in range(3):
            qk.qk_gemv(Q6_K, Wd, 2048, 2048, xd, y)
        y2 = y * 1.0
    s.synchronize()
    y_ref, a = orc.gemv(Q6_K, W, 2048, 2048, x)
    assert_gemv_close(y2.cpu().numpy(), y_ref, a, "side stream")


# ------------------------------------------------------------------ batched GEMV

BATCH = [
    # (type, rows, cols, x id): shared and distinct x, mixed formats, a 4-row
    # and a 1-row matrix, Q6_K with 5 blocks per row (fused with an even row
    # count, the generic kernel with an odd one), an empty one
    (Q4_K, 2048, 2048, 0), (Q4_K, 256, 2048, 0), (Q6_K, 256, 2048, 0), (Q4_K, 4, 2048, 0),
    (Q4_K, 1, 2048, 1), (Q6_K, 130, 1280, 2), (Q6_K, 131, 1280, 2), (Q8_0, 40, 2048, 0), (Q4_K, 0, 2048, 0),
    (Q6_K, 2048, 5632, 3), (Q6_K, 64, 5632, 3),
    # formats sharing a launch: q4_0 with q8_0, Q6_K listed before Q4_K at a
    # width whose rows are split over waves, and q4_0/q8_0 split three ways
    (Q8_0, 300, 2048, 5), (Q4_0, 257, 2048, 5), (Q8_0, 3, 2048, 5),
    (Q6_K, 100, 5632, 6), (Q4_K, 129, 5632, 6),
    (Q4_0, 33, 6144, 7), (Q8_0, 65, 6144, 7),
] + [(Q4_K, 17 + i, 2048, 4) for i in range(10)]  # more than 4 in one group


def test_gemv_batch_matches_oracle(qk, orc, gemv_mode):
    import torch

    xs = {}
    for _, _, c, xi in BATCH:
        xs.setdefault(xi, synth.vector(c, seed=50 + xi))
    xd = {k: to_dev(v) for k, v in xs.items()}
    items, host, bufs = [], [], []
    for i, (t, r, c, xi) in enumerate(BATCH):
        W = synth.matrix(t, r, c, seed=60, stream=i) if r else np.zeros(16, dtype=np.uint8)
        buf, y = guarded(max(r, 1))
        Wd = to_dev(W)
        items.append((t, Wd, r, c, xd[xi], y))
        host.append((t, W, r, c, xs[xi]))
        bufs.append((buf, Wd))
    qk.qk_gemv_batch(items)
    torch.cuda.synchronize()
    for (t, W, r, c, x), (buf, _), item in zip(host, bufs, items):
        check_guard(buf, max(r, 1))
        if r == 0:
            continue
        y_ref, a = orc.gemv(t, W, r, c, x)
        assert_gemv_close(item[5].cpu().numpy(), y_ref, a, f"batch {synth.NAMES[t]} {r}x{c}")


def test_gemv_batch_equals_single_calls(qk, gemv_mode):
    """Grouped launches compute exactly what the single calls compute."""
    import torch

    x = to_dev(synth.vector(2048, seed=70))
    mats = [(Q4_K, 2048), (Q4_K, 256), (Q4_K, 5632), (Q4_K, 5632)]
    Ws = [to_dev(synth.matrix(t, r, 2048, seed=71, stream=i)) for i, (t, r) in enumerate(mats)]
    yb = [torch.empty(r, device="cuda") for _, r in mats]
    ys = [torch.empty(r, device="cuda") for _, r in mats]
    qk.qk_gemv_batch([(t, W, r, 2048, x, y) for (t, r), W, y in zip(mats, Ws, yb)])
    for (t, r), W, y in zip(mats, Ws, ys):
        qk.qk_gemv(t, W, r, 2048, x, y)
    torch.cuda.synchronize()
    for a, b in zip(yb, ys):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ GEMM

GEMM = [(Q4_K, 64, 2048, 1), (Q4_K, 64, 2048, 2), (Q6_K, 48, 5632, 4), (Q4_K, 33, 2048, 8), (Q6_K, 17, 2048, 16),
        (Q4_K, 20, 2048, 17), (Q8_0, 19, 2048, 5), (Q4_0, 21, 2048, 3), (Q6_K, 9, 1280, 7), (Q4_K, 130, 2048, 64),
        (Q6_K, 5, 512, 3), (Q4_K, 1, 256, 1), (Q4_K, 47, 2304, 15), (Q6_K, 31, 4608, 9), (Q4_K, 16, 6144, 16),
        (Q6_K, 70, 2048, 100), (Q4_K, 129, 1024, 65), (Q6_K, 200, 512, 130), (Q4_K, 65, 768, 33),
        # odd Q6_K block counts at even and odd row counts; wide rows
        (Q6_K, 64, 768, 2), (Q6_K, 64, 768, 16), (Q6_K, 64, 768, 70), (Q6_K, 65, 768, 8), (Q6_K, 65, 768, 40),
        (Q6_K, 2, 256, 5), (Q6_K, 2, 256, 33), (Q6_K, 64, 11008, 8), (Q6_K, 130, 11008, 64),
        (Q4_K, 48, 14336, 16), (Q4_K, 70, 14336, 100)]


@pytest.fixture(params=["auto", "few", "prefill", "prefill_ksplit", "prefill_one_k", "prefill_t64", "prefill_t128",
                        "prefill_t128_ksplit", "rows"])
def gemm_path(request, qk):
    """Every GEMM code path the library can choose (QK_TUNE_GEMM_PATH; the
    few-token kernel where M <= 16), and the prefill kernel with and without
    the super-blocks split over two workgroups (QK_TUNE_GEMM_KSPLIT), with
    64- and 128-token tiles (QK_TUNE_PREFILL_TOKENS)."""
    P = qk.QK_GEMM_PATH_PREFILL
    path, ks, tok = {"auto": (None, None, None), "few": (qk.QK_GEMM_PATH_FEW, None, None),
                     "prefill": (P, None, None), "prefill_ksplit": (P, 2, None), "prefill_one_k": (P, 1, None),
                     "prefill_t64": (P, None, 64), "prefill_t128": (P, 1, 128), "prefill_t128_ksplit": (P, 2, 128),
                     "rows": (qk.QK_GEMM_PATH_ROWS, None, None)}[request.param]
    with qk.tuning(gemm_path=path, gemm_ksplit=ks, prefill_tokens=tok):
        yield request.param


@pytest.mark.parametrize("t,rows,cols,M", GEMM, ids=[f"{synth.NAMES[t]}-{r}x{c}-M{m}" for t, r, c, m in GEMM])
def test_gemm_matches_oracle(qk, orc, t, rows, cols, M, gemm_path):
    import torch

    W = synth.matrix(t, rows, cols, seed=M)
    X = synth.bf16_matrix(M, cols, seed=M)
    buf, Y = guarded(M * rows)
    qk.qk_gemm_prefill(t, to_dev(W), rows, cols, to_dev(X.view(np.int16)), M, Y)
    torch.cuda.synchronize()
    check_guard(buf, M * rows)
    Y_ref, A = orc.gemm(t, W, rows, cols, X, M)
    assert_gemv_close(Y.cpu().numpy().reshape(M, rows), Y_ref, A, f"gemm M={M}")


@pytest.mark.parametrize("t,rows,cols", [(Q4_K, 40, 2048), (Q6_K, 34, 2560), (Q6_K, 18, 1280), (Q6_K, 34, 5632),
                                          (Q4_K, 33, 5632), (Q6_K, 17, 1280), (Q8_0, 40, 2048), (Q4_0, 33, 1280)],
                         ids=["q4k-40x2048", "q6k-34x2560", "q6k-18x1280-odd-blocks", "q6k-34x5632-22-blocks",
                              "q4k-33x5632-22-blocks", "q6k-17x1280-odd-blocks-odd-rows", "q8_0-40x2048",
                              "q4_0-33x1280"])
@pytest.mark.parametrize("ksw", [None, "1", "3", "8"], ids=["ksw-auto", "ksw-1", "ksw-3", "ksw-8"])
@pytest.mark.parametrize("rows_per_wave", [None, 8, 16], ids=["rows-auto", "rows-8", "rows-16"])
@pytest.mark.parametrize("depth", [1, 2], ids=["depth-1", "depth-2"])
def test_few_token_every_m(qk, orc, t, rows, cols, ksw, rows_per_wave, depth):
    """The few-token kernel at every M from 1 to 16: 8 weight rows per wave
    in two slices with X tiles of 1, 2, 4 or 8 tokens per slice (the
    fewest that cover M), so each tile runs at its full and its ragged M;
    above 8 tokens both the 16-row single-slice kernel and the 8-row kernel
    with two token sets (forced, and the launcher's choice); ragged last
    row groups; the default number of waves per workgroup and 1, 3 (uneven
    super-block split, steps with idle slices) and 8 (X tiles of more than
    48 KiB of LDS); one and two steps of loads in flight; rows of 22
    super-blocks and odd block and row counts; against the oracle, twice in
    a row (bit-identical)."""
    with qk.tuning(gemm_path=qk.QK_GEMM_PATH_FEW, few_ksw=None if ksw is None else int(ksw),
                   few_rows=rows_per_wave, few_depth=depth):
        few_token_every_m(qk, orc, t, rows, cols, ksw, rows_per_wave)


def few_token_every_m(qk, orc, t, rows, cols, ksw, rpw):
    import torch

    W = synth.matrix(t, rows, cols, seed=rows)
    Wd = to_dev(W)
    assert qk.qk_gemm_kernel_path(t, rows, cols, 16) == qk.QK_GEMM_PATH_FEW
    for M in range(1, 17):
        X = synth.bf16_matrix(M, cols, seed=100 + M)
        buf, Y = guarded(M * rows)
        Xd = to_dev(X.view(np.int16))
        qk.qk_gemm_prefill(t, Wd, rows, cols, Xd, M, Y)
        torch.cuda.synchronize()
        check_guard(buf, M * rows)
        Y_ref, A = orc.gemm(t, W, rows, cols, X, M)
        y1 = Y.cpu().numpy().reshape(M, rows)
        assert_gemv_close(y1, Y_ref, A, f"few-token M={M} ksw={ksw} rows={rpw}")
        qk.qk_gemm_prefill(t, Wd, rows, cols, Xd, M, Y)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().reshape(M, rows), y1), f"repeat differs at M={M}"


@pytest.mark.parametrize("t,rows,cols", [(Q4_K, 5632, 2048), (Q6_K, 2048, 5632), (Q6_K, 4096, 11008),
                                          (Q8_0, 5632, 2048), (Q4_0, 5632, 2048)])
@pytest.mark.parametrize("M", [2, 4, 8, 16, 512])
def test_gemm_full_shapes_sampled(qk, orc, t, rows, cols, M):
    """The multi-token shapes at full size; outputs checked on a sample of
    weight rows (every M) computed by the oracle one row at a time."""
    import torch

    W = synth.matrix(t, rows, cols, seed=4, stream=t)
    X = synth.bf16_matrix(M, cols, seed=4)
    Y = torch.empty(M * rows, device="cuda")
    qk.qk_gemm_prefill(t, to_dev(W), rows, cols, to_dev(X.view(np.int16)), M, Y)
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy().reshape(M, rows)
    rb = len(W) // rows
    sample = sorted(set([0, 1, rows - 1] + list(synth.rng(4, 99).integers(0, rows, 40))))
    for r in sample:
        Yr, Ar = orc.gemm(t, W[r * rb:(r + 1) * rb], 1, cols, X, M)
        assert_gemv_close(Yh[:, r], Yr[:, 0], Ar[:, 0], f"gemm row {r}")


@pytest.mark.parametrize("t,rows,cols,M", [(Q4_K, 200, 2048, 300), (Q6_K, 130, 5632, 130), (Q8_0, 70, 2048, 200),
                                            (Q4_0, 64, 1280, 129)],
                         ids=["q4k-200x2048-M300", "q6k-130x5632-M130", "q8_0-70x2048-M200", "q4_0-64x1280-M129"])
@pytest.mark.parametrize("ksplit,tok", [(1, 64), (2, 64), (1, 128), (2, 128)],
                         ids=["t64-ks1", "t64-ks2", "t128-ks1", "t128-ks2"])
def test_prefill_repeats_bit_exact(qk, orc, t, rows, cols, M, ksplit, tok):
    """The prefill kernel gives the same bits call after call, also where
    two workgroups add their halves into Y (two addends to a zeroed Y)."""
    import torch

    W = to_dev(synth.matrix(t, rows, cols, seed=M))
    X = to_dev(synth.bf16_matrix(M, cols, seed=M).view(np.int16))
    Y = torch.empty(M * rows, device="cuda")
    with qk.tuning(gemm_path=qk.QK_GEMM_PATH_PREFILL, gemm_ksplit=ksplit, prefill_tokens=tok):
        qk.qk_gemm_prefill(t, W, rows, cols, X, M, Y)
        first = Y.clone()
        for _ in range(3):
            Y.fill_(float("nan"))
            qk.qk_gemm_prefill(t, W, rows, cols, X, M, Y)
            torch.cuda.synchronize()
            assert torch.equal(Y, first)


def test_gemm_m1_equals_gemv(qk, orc):
    import torch

    rows, cols = 300, 2048
    W = synth.matrix(Q4_K, rows, cols, seed=31)
    X = synth.bf16_matrix(1, cols, seed=31)
    x = (X.astype(np.uint32) << 16).view(np.float32).reshape(-1)
    Y = torch.empty(rows, device="cuda")
    qk.qk_gemm_prefill(Q4_K, to_dev(W), rows, cols, to_dev(X.view(np.int16)), 1, Y)
    y = run_gemv(qk, Q4_K, W, rows, cols, x)
    torch.cuda.synchronize()
    y_ref, a = orc.gemv(Q4_K, W, rows, cols, x)
    assert_gemv_close(Y.cpu().numpy(), y_ref, a, "gemm M=1")
    assert_gemv_close(y, y_ref, a, "gemv")


# ------------------------------------------------------------------ GGUF upload

def test_gguf_upload_then_gemv(qk, orc, tmp_path):
    """Weights written into a GGUF file (tests/gguf_writer.py), read back by
    the library's reader, uploaded with qk_gguf_upload and multiplied in
    place: the uploaded bytes equal the written ones and the GEMV matches the
    oracle on them."""
    import os

    import torch

    import gguf_writer as gw

    mats = [("blk.0.attn_q.weight", Q4_K, gw.Q4_K, 48, 2048), ("blk.0.ffn_down.weight", Q6_K, gw.Q6_K, 40, 5632),
            ("blk.0.attn_v.weight", Q4_0, gw.Q4_0, 33, 2048)]
    host = {n: synth.matrix(t, r, c, seed=80 + i, stream=t) for i, (n, t, _, r, c) in enumerate(mats)}
    blob = gw.build([("general.alignment", gw.UINT32, 64)],
                    [(n, [c, r], gt, host[n].tobytes()) for n, t, gt, r, c in mats], alignment=64)
    path = os.path.join(tmp_path, "w.gguf")
    with open(path, "wb") as fh:
        fh.write(blob)
    with qk.GgufFile(path) as f:
        for n, t, _, r, c in mats:
            info = f.tensor(n)
            assert info["qk_type"] == t and info["dims"] == [c, r]
            Wd = torch.empty(info["nbytes"], dtype=torch.uint8, device="cuda")
            f.upload(n, Wd)
            torch.cuda.synchronize()
            assert np.array_equal(Wd.cpu().numpy(), host[n])
            x = synth.vector(c, seed=81)
            buf, y = guarded(r)
            qk.qk_gemv(info["qk_type"], Wd, r, c, to_dev(x), y)
            torch.cuda.synchronize()
            check_guard(buf, r)
            y_ref, a = orc.gemv(t, host[n], r, c, x)
            assert_gemv_close(y.cpu().numpy(), y_ref, a, f"gguf {n}")

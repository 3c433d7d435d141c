"""GPU parity for wide rows and odd block counts through the C ABI against
the CPU oracle (|y - y_ref| <= 1e-4 * sum|w*x| + 1e-6 for every output).

Rows wider than 6144 columns run the wide-row kernel: x staged in LDS in
batches, each row split over up to 8 waves (up to 512 units of 64 or 32
weights), the wave partials added in LDS in a fixed order. Q6_K and Q3_K rows
with an odd number of blocks take the fused kernel when the row count is
even (the matrix's last block then ends on a 4-byte boundary) and the generic
kernel otherwise. Shapes: the down projections of 7B-8B models (11008, 14336
and 18944 columns), the widest row the kernel takes (512 units), one unit
past it (generic), ragged row tails, grouped launches and transformed inputs
at these widths, and a one-layer decode step at 4096 x 11008 shapes."""
import numpy as np
import pytest

from block_quantized_weight_gemv_amd import synth
from gpu_helpers import assert_gemv_close, check_guard, gemv_case, guarded, to_dev

pytestmark = pytest.mark.gpu

Q4_0, Q8_0, Q4_K, Q6_K = 1, 2, 3, 4
Q8_0_F16, Q5_1, Q5_K, Q2_K, Q3_K = 5, 6, 7, 8, 9


@pytest.fixture(scope="module")
def qk():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_quantized_weight_gemv_amd import qk as mod

    return mod


def run_gemv(qk, t, W_np, rows, cols, x_np):
    import torch

    buf, y = guarded(rows)
    qk.qk_gemv(t, to_dev(W_np), rows, cols, to_dev(x_np), y)
    torch.cuda.synchronize()
    check_guard(buf, rows)
    return y.cpu().numpy()


# (type, rows, cols): widths just past the register staging, 7B-8B down
# projections, the widest fused row (512 units: 32768 columns of 64-weight
# units, 16384 of 32-weight blocks) and one unit more (generic kernel).
WIDE = [
    (Q4_K, 64, 6400), (Q4_K, 130, 11008), (Q4_K, 33, 14336), (Q4_K, 17, 18944), (Q4_K, 9, 32768),
    (Q4_K, 3, 33024),
    (Q6_K, 64, 11008), (Q6_K, 65, 11008), (Q6_K, 32, 14336), (Q6_K, 16, 18944), (Q6_K, 8, 32768),
    (Q6_K, 130, 6400),
    (Q8_0, 40, 8192), (Q8_0, 7, 16384), (Q8_0, 3, 16416),
    (Q4_0, 40, 8192), (Q4_0, 5, 16384), (Q4_0, 6, 32 * 301),
    (Q5_K, 33, 14336), (Q2_K, 33, 14336), (Q3_K, 64, 11008), (Q3_K, 63, 11008),
    (Q5_1, 17, 8192), (Q8_0_F16, 17, 8192), (Q8_0_F16, 9, 16384),
]


@pytest.mark.parametrize("t,rows,cols", WIDE, ids=[f"{synth.NAMES[t]}-{r}x{c}" for t, r, c in WIDE])
def test_wide_gemv_matches_oracle(qk, orc, t, rows, cols):
    W, x = gemv_case(t, rows, cols, seed=rows + cols)
    y = run_gemv(qk, t, W, rows, cols, x)
    y_ref, a = orc.gemv(t, W, rows, cols, x)
    assert_gemv_close(y, y_ref, a, f"{synth.NAMES[t]} {rows}x{cols}")


# Odd block counts per row of the 2-byte aligned K-quants (rows then start
# alternately 4-byte aligned and 2 bytes past): Q6_K is fused at every row
# count; Q3_K with an even row count, else the generic kernel; one, three,
# five and 43 blocks per row.
ODD = [(t, r, c) for t in (Q6_K, Q3_K) for (r, c) in [(2, 256), (1, 256), (256, 768), (255, 768), (130, 1280),
                                                      (4096, 768), (10, 256 * 43)]]


@pytest.mark.parametrize("t,rows,cols", ODD, ids=[f"{synth.NAMES[t]}-{r}x{c}" for t, r, c in ODD])
@pytest.mark.parametrize("mode", ["auto", "streamed"])
def test_odd_block_rows_match_oracle(qk, orc, t, rows, cols, mode):
    with qk.tuning(gemv_stream=1 if mode == "streamed" else None):
        W, x = gemv_case(t, rows, cols, seed=3 * rows + cols)
        y = run_gemv(qk, t, W, rows, cols, x)
    y_ref, a = orc.gemv(t, W, rows, cols, x)
    assert_gemv_close(y, y_ref, a, f"{synth.NAMES[t]} {rows}x{cols} {mode}")


def test_fused_path_taken(qk):
    """The shapes above that should be fused are (a transformed input is
    offered exactly where the fused kernel runs, for Q4_K and Q6_K)."""
    assert qk.qk_gemv_input_supported(Q6_K, 4096, 11008)
    assert qk.qk_gemv_input_supported(Q4_K, 4096, 14336)
    assert qk.qk_gemv_input_supported(Q6_K, 3584, 18944)
    assert qk.qk_gemv_input_supported(Q4_K, 9, 32768)
    assert qk.qk_gemv_input_supported(Q6_K, 256, 768)
    assert qk.qk_gemv_input_supported(Q6_K, 255, 768)
    assert qk.qk_gemv_kernel_path(Q6_K, 255, 768) == qk.QK_PATH_FUSED
    assert qk.qk_gemv_kernel_path(Q3_K, 255, 768) == qk.QK_PATH_GENERIC
    assert not qk.qk_gemv_input_supported(Q4_K, 3, 33024)


@pytest.mark.parametrize("t,rows,cols", [(Q6_K, 4096, 11008), (Q4_K, 4096, 14336), (Q6_K, 3584, 18944)],
                         ids=["q6k-llama2-7b-down", "q4k-llama3-8b-down", "q6k-qwen2-7b-down"])
def test_wide_full_shapes(qk, orc, t, rows, cols):
    """Full down-projection shapes of 7B-8B models, every output."""
    W, x = gemv_case(t, rows, cols, seed=9)
    y = run_gemv(qk, t, W, rows, cols, x)
    y_ref, a = orc.gemv(t, W, rows, cols, x)
    assert_gemv_close(y, y_ref, a, f"{synth.NAMES[t]} {rows}x{cols}")


def test_wide_batch_matches_oracle(qk, orc):
    """Grouped launches at wide widths: Q4_K with Q6_K (odd block count,
    even and odd row counts) against one x, q4_0 with q8_0 against another,
    and an unfusable member (q4_0 with an odd block count) run on its own."""
    import torch

    spec = [(Q4_K, 300, 11008, 0), (Q6_K, 64, 11008, 0), (Q4_K, 5, 11008, 0), (Q6_K, 3, 11008, 0),
            (Q4_0, 129, 9600, 1), (Q8_0, 40, 9600, 1), (Q4_0, 7, 9632, 2)]
    xs = {0: synth.vector(11008, seed=31), 1: synth.vector(9600, seed=32), 2: synth.vector(9632, seed=34)}
    xd = {k: to_dev(v) for k, v in xs.items()}
    items, host = [], []
    for i, (t, r, c, xi) in enumerate(spec):
        W = synth.matrix(t, r, c, seed=33, stream=i)
        buf, y = guarded(r)
        items.append((t, to_dev(W), r, c, xd[xi], y))
        host.append((t, W, r, c, xs[xi], buf))
    qk.qk_gemv_batch(items)
    torch.cuda.synchronize()
    for (t, W, r, c, x, buf), item in zip(host, items):
        check_guard(buf, r)
        y_ref, a = orc.gemv(t, W, r, c, x)
        assert_gemv_close(item[5].cpu().numpy(), y_ref, a, f"batch {synth.NAMES[t]} {r}x{c}")


@pytest.mark.parametrize("kind", ["add_rmsnorm", "swiglu"])
@pytest.mark.parametrize("mats,cols", [([(Q4_K, 700), (Q4_K, 64), (Q6_K, 64)], 8192),
                                       ([(Q6_K, 4096)], 11008), ([(Q4_0, 33), (Q8_0, 65)], 16384)],
                         ids=["q4k-q6k-8192", "q6k-11008", "q4_0-q8_0-16384"])
def test_wide_gemv_batch_input(qk, orc, kind, mats, cols):
    """Transformed inputs (RMSNorm of x + aux, or silu(x) * aux) staged by
    the wide-row kernel, against the oracle's GEMV of the oracle's x'."""
    import torch

    g = synth.rng(51, cols)
    x = g.standard_normal(cols).astype(np.float32)
    aux = g.standard_normal(cols).astype(np.float32)
    nw = g.uniform(0.5, 1.5, cols).astype(np.float32)
    xd, auxd, nwd = to_dev(x), to_dev(aux), to_dev(nw)
    x_out = torch.full((cols,), float("nan"), device="cuda")
    Ws = [synth.matrix(t, r, cols, seed=52 + i, stream=t) for i, (t, r) in enumerate(mats)]
    ys = [torch.full((r,), float("nan"), device="cuda") for _, r in mats]
    descs = [(t, to_dev(W), r, cols, xd, y) for (t, r), W, y in zip(mats, Ws, ys)]
    if kind == "add_rmsnorm":
        inp = qk.make_gemv_input(qk.QK_INPUT_ADD_RMSNORM, auxd, nwd, 1e-5, x_out)
        xp = orc.rmsnorm(x + aux, nw, 1e-5)
    else:
        inp = qk.make_gemv_input(qk.QK_INPUT_SWIGLU, auxd)
        xp = orc.swiglu(x, aux).astype(np.float32)
    assert all(qk.qk_gemv_input_supported(t, r, cols) for t, r in mats)
    qk.qk_gemv_batch_input(descs, inp)
    torch.cuda.synchronize()
    for (t, r), W, y in zip(mats, Ws, ys):
        ref, a = orc.gemv(t, W, r, cols, xp)
        assert_gemv_close(y.cpu().numpy(), ref, a, f"{kind} {synth.NAMES[t]} {r}x{cols}")
    if kind == "add_rmsnorm":
        assert np.array_equal(x_out.cpu().numpy(), x + aux)


def test_wide_repeat_is_deterministic(qk):
    """The split-row combine has a fixed order: repeated calls agree bit for
    bit."""
    import torch

    W, x = gemv_case(Q6_K, 4096, 11008, seed=4)
    Wd, xd = to_dev(W), to_dev(x)
    y0 = torch.empty(4096, device="cuda")
    y1 = torch.empty(4096, device="cuda")
    qk.qk_gemv(Q6_K, Wd, 4096, 11008, xd, y0)
    for _ in range(3):
        qk.qk_gemv(Q6_K, Wd, 4096, 11008, xd, y1)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)


def test_step_with_wide_ffn(qk, orc):
    """One layer at Llama-2-7B widths (4096 wide, 32 heads of 128, FFN 11008:
    the down projection is a wide Q6_K row with 43 blocks), two positions,
    against the oracle's step, eager and from a captured graph."""
    from block_quantized_weight_gemv_amd.step import DecodeStep, StepConfig, synthetic_weights
    from oracle.step import OracleStep

    cfg = StepConfig(dim=4096, n_layers=1, n_heads=32, n_kv_heads=32, ffn=11008, vocab=512, max_pos=8)
    w = synthetic_weights(cfg, seed=12)
    gpu, ref = DecodeStep(cfg, w), OracleStep(orc, cfg, w)
    assert gpu.fused
    eager = []
    for pos, t in enumerate([3, 300]):
        got = gpu.forward(t, pos).cpu().numpy().astype(np.float64)
        lr, a, _ = ref.forward(t, pos)
        ratio = np.abs(got - lr) / a
        assert ratio.max() <= 1e-3, (pos, float(ratio.max()))
        eager.append(got)
    g2 = DecodeStep(cfg, w)
    g2.capture()
    for pos, t in enumerate([3, 300]):
        assert np.array_equal(g2.forward(t, pos).cpu().numpy().astype(np.float64), eager[pos]), pos

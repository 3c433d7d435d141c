"""GPU parity of the decode step around the GEMVs and of the encoder, through
the C ABI (include/qk_step.h) against the CPU oracle.

Tolerances (fp32 kernels against fp64 definitions):
* RMSNorm: |out - ref| <= 1e-5 |ref| + 1e-30 (the sum of squares is a tree of
  fp32 adds, relative error ~1e-6; one sqrt, one divide, two multiplies);
* RoPE tables: within 1 fp32 ulp of the fp64 values rounded (both round
  fp64 cos/sin of the same fp64 angle; the libraries may differ by an fp64
  ulp, which can move the fp32 rounding by one);
* RoPE rotation: |r0 - ref| <= 2^-22 (|x0 c| + |x1 s|) and |r1 - ref| <=
  2^-22 (|x0 s| + |x1 c|) (+ 1e-30; two products and one sum in fp32,
  possibly fused); the cached K equals the kernel's
  rotated k rounded to fp16 and is within one fp16 step of the oracle's; the
  cached V is bit-exact;
* attention: |out - ref| <= 1e-4 sum_t p_t |V[t]| + 1e-6 (the GEMV rule with
  softmax weights: 64- or 128-term fp32 dot products, fp32 exp, a running
  rescale per position);
* SwiGLU: |out - ref| <= 2e-6 |ref| + 1e-37;
* the encoder: bit-exact (its integer codes are decided by the same fp32
  operations on both sides);
* the whole step (logits): |l - ref| <= 1e-3 sum|w x| of the output matrix
  per logit — each operation's own error is ~1e-6 relative and the layers
  carry it forward; measured worst ~1e-5.
"""
import numpy as np
import pytest

from block_quantized_weight_gemv_amd import synth
from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu

Q8_0, Q4_0 = 2, 1


@pytest.fixture(scope="module")
def qk():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_quantized_weight_gemv_amd import qk as mod

    return mod


def dev_pos(p):
    import torch

    return torch.tensor([p], dtype=torch.int32, device="cuda")


# ------------------------------------------------------------------ RMSNorm

@pytest.mark.parametrize("n", [1, 5, 256, 2048, 5632, 65536])
def test_rmsnorm(qk, orc, n):
    import torch

    g = synth.rng(40, n)
    x = (g.standard_normal(n) * 3).astype(np.float32)
    w = g.uniform(0.5, 1.5, n).astype(np.float32)
    out = torch.empty(n, device="cuda")
    qk.qk_rmsnorm(to_dev(x), to_dev(w), n, 1e-5, out)
    torch.cuda.synchronize()
    ref = orc.rmsnorm(x, w, 1e-5).astype(np.float64)
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1e-5 * np.abs(ref) + 1e-30)


def test_add_rmsnorm_and_in_place_norm(qk, orc):
    import torch

    n = 2048
    g = synth.rng(41, 0)
    x = g.standard_normal(n).astype(np.float32)
    r = g.standard_normal(n).astype(np.float32)
    w = g.uniform(0.5, 1.5, n).astype(np.float32)
    xd, out = to_dev(x), torch.empty(n, device="cuda")
    qk.qk_add_rmsnorm(xd, to_dev(r), to_dev(w), n, 1e-5, out)
    torch.cuda.synchronize()
    s = x + r  # fp32 additions
    assert np.array_equal(xd.cpu().numpy(), s)
    ref = orc.rmsnorm(s, w, 1e-5).astype(np.float64)
    assert np.all(np.abs(out.cpu().numpy() - ref) <= 1e-5 * np.abs(ref) + 1e-30)
    xd2 = to_dev(x)
    qk.qk_rmsnorm(xd2, to_dev(w), n, 1e-5, xd2)  # out aliasing x
    torch.cuda.synchronize()
    ref2 = orc.rmsnorm(x, w, 1e-5).astype(np.float64)
    assert np.all(np.abs(xd2.cpu().numpy() - ref2) <= 1e-5 * np.abs(ref2) + 1e-30)


# ------------------------------------------------------------------ RoPE

def ulps(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, -(a & 0x7FFFFFFF), a)
    b = np.where(b < 0, -(b & 0x7FFFFFFF), b)
    return np.abs(a - b)


@pytest.mark.parametrize("head_dim", [64, 128])
def test_rope_tables(qk, orc, head_dim):
    import torch

    P = 2048
    c = torch.empty(P * head_dim // 2, device="cuda")
    s = torch.empty_like(c)
    qk.qk_rope_tables(P, head_dim, 10000.0, c, s)
    torch.cuda.synchronize()
    ch, sh = c.cpu().numpy().reshape(P, -1), s.cpu().numpy().reshape(P, -1)
    for p in [0, 1, 2, 17, 511, 1000, 2047]:
        rc, rs = orc.rope_table(p, head_dim, 10000.0)
        assert ulps(ch[p], rc).max() <= 1 and ulps(sh[p], rs).max() <= 1, p


@pytest.mark.parametrize("nh,nkv,hd,pos", [(32, 4, 64, 0), (32, 4, 64, 77), (4, 2, 128, 2047), (8, 8, 64, 5)])
def test_rope_kv(qk, orc, nh, nkv, hd, pos):
    import torch

    P = 2048
    g = synth.rng(42, nh + pos)
    q = g.standard_normal(nh * hd).astype(np.float32)
    k = g.standard_normal(nkv * hd).astype(np.float32)
    v = g.standard_normal(nkv * hd).astype(np.float32)
    c = torch.empty(P * hd // 2, device="cuda")
    s = torch.empty_like(c)
    qk.qk_rope_tables(P, hd, 10000.0, c, s)
    stride = nkv * hd + 8
    kc = torch.zeros(P * stride, dtype=torch.int16, device="cuda")
    vc = torch.zeros_like(kc)
    qd, kd = to_dev(q), to_dev(k)
    qk.qk_rope_kv(qd, kd, to_dev(v), dev_pos(pos), P, c, s, nh, nkv, hd, kc, vc, stride)
    torch.cuda.synchronize()
    ct = c.cpu().numpy().reshape(P, -1)[pos]
    st = s.cpu().numpy().reshape(P, -1)[pos]
    for x, got, heads in ((q, qd.cpu().numpy(), nh), (k, kd.cpu().numpy(), nkv)):
        ref = orc.rope(x, heads, hd, ct, st).astype(np.float64)
        x2 = x.reshape(-1, 2).astype(np.float64)
        cc = np.tile(ct, heads).astype(np.float64)
        ss = np.tile(st, heads).astype(np.float64)
        # r0 = x0 c - x1 s and r1 = x0 s + x1 c, each with its own scale
        b0 = 2.0 ** -22 * (np.abs(x2[:, 0] * cc) + np.abs(x2[:, 1] * ss)) + 1e-30
        b1 = 2.0 ** -22 * (np.abs(x2[:, 0] * ss) + np.abs(x2[:, 1] * cc)) + 1e-30
        err = np.abs(got.reshape(-1, 2) - ref.reshape(-1, 2))
        assert np.all(err[:, 0] <= b0) and np.all(err[:, 1] <= b1)
    kch = kc.cpu().numpy().view(np.uint16).reshape(P, stride)
    vch = vc.cpu().numpy().view(np.uint16).reshape(P, stride)
    assert np.array_equal(kch[pos, :nkv * hd], kd.cpu().numpy().astype(np.float16).view(np.uint16))
    kref = orc.halves(orc.rope(k, nkv, hd, ct, st))
    assert np.max(np.abs(kch[pos, :nkv * hd].astype(np.int64) - kref.astype(np.int64))) <= 1
    assert np.array_equal(vch[pos, :nkv * hd], orc.halves(v))
    others = np.ones(P, bool)
    others[pos] = False
    assert not kch[others].any() and not vch[others].any() and not kch[pos, nkv * hd:].any()


def test_rope_kv_position_out_of_range_writes_nothing(qk):
    import torch

    P, hd = 16, 64
    c = torch.empty(P * hd // 2, device="cuda")
    s = torch.empty_like(c)
    qk.qk_rope_tables(P, hd, 10000.0, c, s)
    for bad in (P, -1, 1 << 30):
        q = torch.ones(4 * hd, device="cuda")
        k = torch.ones(hd, device="cuda")
        kc = torch.zeros(P * hd, dtype=torch.int16, device="cuda")
        vc = torch.zeros_like(kc)
        out = torch.full((4 * hd,), 7.0, device="cuda")
        qk.qk_rope_kv(q, k, torch.ones(hd, device="cuda"), dev_pos(bad), P, c, s, 4, 1, hd, kc, vc, hd)
        ws = torch.zeros(qk.qk_attention_workspace_bytes(4, hd, P) // 4, device="cuda")
        qk.qk_attention(q, kc, vc, dev_pos(bad), P, 4, 1, hd, hd, ws, out)
        torch.cuda.synchronize()
        assert torch.all(q == 1) and torch.all(k == 1) and not kc.any() and not vc.any()
        assert torch.all(out == 7.0)


# ------------------------------------------------------------------ attention

ATT = [(32, 4, 64, 0), (32, 4, 64, 1), (32, 4, 64, 255), (32, 4, 64, 256), (32, 4, 64, 1000),
       (32, 4, 64, 2047), (4, 4, 128, 300), (8, 1, 128, 2047), (2, 2, 64, 700)]


@pytest.mark.parametrize("nh,nkv,hd,pos", ATT, ids=[f"{a}h{b}kv{c}d-pos{d}" for a, b, c, d in ATT])
def test_attention(qk, orc, nh, nkv, hd, pos):
    import torch

    P = 2048
    g = synth.rng(43, pos * 7 + hd)
    stride = nkv * hd + (8 if nh == 2 else 0)
    kc = (g.standard_normal((P, stride)) * 2).astype(np.float16)
    vc = g.standard_normal((P, stride)).astype(np.float16)
    kc[pos + 1:] = 6.0e4  # rows past the position must not be read
    vc[pos + 1:] = -6.0e4
    q = g.standard_normal(nh * hd).astype(np.float32)
    out = torch.empty(nh * hd, device="cuda")
    nbytes = qk.qk_attention_workspace_bytes(nh, hd, P)
    ws = torch.full((nbytes // 4,), float("nan"), device="cuda")  # scratch: no contents needed
    ref, a = orc.attention(q, kc.view(np.uint16), vc.view(np.uint16), nh, nkv, hd, pos + 1, stride)
    Kd, Vd, qd, pd = to_dev(kc.view(np.int16)), to_dev(vc.view(np.int16)), to_dev(q), dev_pos(pos)
    for rep in range(3):  # repeated calls on one workspace
        out.fill_(float("nan"))
        qk.qk_attention(qd, Kd, Vd, pd, P, nh, nkv, hd, stride, ws, out)
        torch.cuda.synchronize()
        err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= 1e-4 * a + 1e-6), (rep, float(np.nanmax(err / (1e-4 * a + 1e-6))))


@pytest.mark.parametrize("P,pos,hd", [(20000, 19999, 64), (20000, 5000, 128), (65536, 40000, 64), (65536, 65535, 128)],
                         ids=["cap20000-pos19999", "cap20000-pos5000-hd128", "cap65536-pos40000", "cap65536-pos65535-hd128"])
def test_attention_long_cache(qk, orc, P, pos, hd):
    """Caches of more than 16384 rows take chunks of 128 or 256 positions
    (at most 256 chunks per head)."""
    import torch

    nh, nkv = 8, 2
    g = synth.rng(44, pos + hd)
    stride = nkv * hd
    kc = np.full((P, stride), 6.0e4, dtype=np.float16)  # rows past the position must not be read
    vc = np.full((P, stride), -6.0e4, dtype=np.float16)
    kc[:pos + 1] = (g.standard_normal((pos + 1, stride)) * 2).astype(np.float16)
    vc[:pos + 1] = g.standard_normal((pos + 1, stride)).astype(np.float16)
    q = g.standard_normal(nh * hd).astype(np.float32)
    out = torch.full((nh * hd,), float("nan"), device="cuda")
    ws = torch.full((qk.qk_attention_workspace_bytes(nh, hd, P) // 4,), float("nan"), device="cuda")
    qk.qk_attention(to_dev(q), to_dev(kc.view(np.int16)), to_dev(vc.view(np.int16)), dev_pos(pos), P, nh, nkv, hd,
                    stride, ws, out)
    torch.cuda.synchronize()
    ref, a = orc.attention(q, kc.view(np.uint16), vc.view(np.uint16), nh, nkv, hd, pos + 1, stride)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= 1e-4 * a + 1e-6), float(np.nanmax(err / (1e-4 * a + 1e-6)))


@pytest.mark.parametrize("nh,nkv,hd,pos", [(32, 4, 64, 0), (32, 4, 64, 255), (32, 4, 64, 256), (32, 4, 64, 2047),
                                          (8, 2, 128, 700), (32, 32, 128, 63), (32, 32, 128, 64)])
def test_attention_rope(qk, orc, nh, nkv, hd, pos):
    """RoPE, the cache store and attention in one call, against the oracle
    run as separate steps (rotate, round to fp16 into row pos, attend)."""
    import torch

    P = 2048
    g = synth.rng(49, pos + hd)
    stride = nkv * hd
    kc = (g.standard_normal((P, stride)) * 2).astype(np.float16)
    vc = g.standard_normal((P, stride)).astype(np.float16)
    kc[pos:] = 6.0e4  # row pos is written by the call; later rows must not be read
    vc[pos:] = -6.0e4
    q = g.standard_normal(nh * hd).astype(np.float32)
    k = g.standard_normal(nkv * hd).astype(np.float32)
    v = g.standard_normal(nkv * hd).astype(np.float32)
    c = torch.empty(P * hd // 2, device="cuda")
    s = torch.empty_like(c)
    qk.qk_rope_tables(P, hd, 10000.0, c, s)
    ws = torch.full((qk.qk_attention_workspace_bytes(nh, hd, P) // 4,), float("nan"), device="cuda")
    Kd, Vd = to_dev(kc.view(np.int16)), to_dev(vc.view(np.int16))
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = torch.full((nh * hd,), float("nan"), device="cuda")
    qk.qk_attention_rope(qd, kd, vd, dev_pos(pos), P, c, s, nh, nkv, hd, Kd, Vd, stride, ws, out)
    torch.cuda.synchronize()
    assert np.array_equal(qd.cpu().numpy(), q) and np.array_equal(kd.cpu().numpy(), k)
    ct = c.cpu().numpy().reshape(P, -1)[pos]
    st = s.cpu().numpy().reshape(P, -1)[pos]
    kref = orc.halves(orc.rope(k, nkv, hd, ct, st))
    krow = Kd.cpu().numpy().view(np.uint16).reshape(P, stride)
    vrow = Vd.cpu().numpy().view(np.uint16).reshape(P, stride)
    assert np.max(np.abs(krow[pos].astype(np.int64) - kref.astype(np.int64))) <= 1
    assert np.array_equal(vrow[pos], orc.halves(v))
    assert np.array_equal(krow[:pos], kc.view(np.uint16)[:pos]) and np.array_equal(krow[pos + 1:], kc.view(np.uint16)[pos + 1:])
    kc2 = kc.view(np.uint16).copy()
    vc2 = vc.view(np.uint16).copy()
    kc2[pos], vc2[pos] = krow[pos], vrow[pos]  # the row the call wrote (within one fp16 step of the oracle's)
    ref, a = orc.attention(orc.rope(q, nh, hd, ct, st), kc2, vc2, nh, nkv, hd, pos + 1, stride)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= 1e-4 * a + 1e-6), float(np.nanmax(err / (1e-4 * a + 1e-6)))


# ------------------------------------------------------------------ SwiGLU

def test_swiglu(qk, orc):
    import torch

    n = 5632 * 3 + 7
    g = synth.rng(44, 0)
    gate = (g.standard_normal(n) * 4).astype(np.float32)
    gate[:6] = [0, 100, -100, 88, -88, 1e-30]
    up = g.standard_normal(n).astype(np.float32)
    out = torch.empty(n, device="cuda")
    qk.qk_swiglu(to_dev(gate), to_dev(up), n, out)
    torch.cuda.synchronize()
    ref = orc.swiglu(gate, up)
    assert np.all(np.abs(out.cpu().numpy() - ref) <= 2e-6 * np.abs(ref) + 1e-37)


# ------------------------------------------------------------------ encoder

def encoder_input(n, seed):
    g = synth.rng(45, seed)
    x = (g.standard_normal(n) * np.exp2(g.integers(-12, 12, n))).astype(np.float32)
    b = x.reshape(-1, 32)
    b[0] = 0.0  # all-zero block: d = 0
    b[1] = (np.arange(32) - 15.5) * 2.0 ** -7  # halfway points on the q8_0 grid of block 1
    b[1, 0] = 127 * 2.0 ** -7
    b[2] = np.float32(-3.0)  # all equal (negative): q4_0 maps them to code 0
    b[3, 5] = np.float32(1e-38)
    b[4, :] = np.float32(3e38) * np.sign(b[4, :] + 1e-3)
    return x


@pytest.mark.parametrize("t", [Q8_0, Q4_0], ids=["q8_0", "q4_0"])
@pytest.mark.parametrize("n", [32 * 8, 32 * 1001, 1 << 20])
def test_quantize_bit_exact(qk, orc, t, n):
    import torch

    x = encoder_input(n, n + t)
    bb = 36 if t == Q8_0 else 18
    out = torch.zeros(n // 32 * bb + 16, dtype=torch.uint8, device="cuda")
    qk.qk_quantize_row(t, to_dev(x), n, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = orc.quantize(t, x)
    bad = np.flatnonzero((got[:n // 32 * bb] != ref).reshape(-1, bb).any(axis=1))
    assert bad.size == 0, (bad[:4].tolist(), got[:n // 32 * bb].reshape(-1, bb)[bad[:2]].tolist(),
                           ref.reshape(-1, bb)[bad[:2]].tolist())
    assert not got[n // 32 * bb:].any()


def test_quantize_then_gemv_round_trip(qk, orc):
    """Weights quantised on the GPU and multiplied by the library's GEMV agree
    with the oracle's GEMV of the same blocks (the exporter's output serves
    the engine)."""
    import torch

    rows, cols = 300, 2048
    wf = synth.rng(46, 0).standard_normal(rows * cols).astype(np.float32) * 0.02
    x = synth.vector(cols, seed=46)
    for t in (Q8_0, Q4_0):
        bb = 36 if t == Q8_0 else 18
        W = torch.empty(rows * cols // 32 * bb, dtype=torch.uint8, device="cuda")
        qk.qk_quantize_row(t, to_dev(wf), rows * cols, W)
        y = torch.empty(rows, device="cuda")
        qk.qk_gemv(t, W, rows, cols, to_dev(x), y)
        torch.cuda.synchronize()
        Wh = W.cpu().numpy()
        assert np.array_equal(Wh, orc.quantize(t, wf))
        ref, a = orc.gemv(t, Wh, rows, cols, x)
        assert np.all(np.abs(y.cpu().numpy() - ref) <= 1e-4 * a + 1e-6)


# ------------------------------------------------------------------ GEMVs with a transformed input

INPUT = [(3, [(3, 2048), (3, 256), (4, 256)], 2048), (3, [(3, 5632), (3, 5632)], 2048), (4, [(4, 2048)], 5632),
         (1, [(2, 300), (1, 17)], 2048), (4, [(4, 32000)], 2048)]


@pytest.mark.parametrize("kind", ["add_rmsnorm", "swiglu"])
@pytest.mark.parametrize("case", range(len(INPUT)))
def test_gemv_batch_input(qk, orc, kind, case):
    """y = W x' with x' = RMSNorm(x + aux) * w (and x + aux written to
    x_out) or x' = silu(x) * aux, in one launch, against the oracle's GEMV of
    the oracle's x' (whose fp32 rounding may differ by an ulp from the
    kernel's: well inside the GEMV tolerance)."""
    import torch

    _, mats, cols = INPUT[case]
    g = synth.rng(47, case)
    x = g.standard_normal(cols).astype(np.float32)
    aux = g.standard_normal(cols).astype(np.float32)
    nw = g.uniform(0.5, 1.5, cols).astype(np.float32)
    xd, auxd, nwd = to_dev(x), to_dev(aux), to_dev(nw)
    x_out = torch.full((cols,), float("nan"), device="cuda")
    Ws = [synth.matrix(t, r, cols, seed=48 + i, stream=t) for i, (t, r) in enumerate(mats)]
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
        err = np.abs(y.cpu().numpy() - ref)
        assert np.all(err <= 1e-4 * a + 1e-6), (t, r, float(np.max(err / (1e-4 * a + 1e-6))))
    if kind == "add_rmsnorm":
        assert np.array_equal(x_out.cpu().numpy(), x + aux)


def test_gemv_input_supported(qk):
    assert qk.qk_gemv_input_supported(3, 2048, 2048) and qk.qk_gemv_input_supported(4, 2048, 5632)
    assert qk.qk_gemv_input_supported(4, 10, 256)  # Q6_K, odd blocks per row: fused at any row count
    assert qk.qk_gemv_input_supported(4, 11, 256)
    assert qk.qk_gemv_input_supported(3, 10, 8192) and qk.qk_gemv_input_supported(4, 4096, 11008)  # wide rows
    assert not qk.qk_gemv_input_supported(1, 11, 96)  # q4_0 with an odd block count: generic kernel
    assert not qk.qk_gemv_input_supported(7, 10, 2048)  # Q5_K: no transformed-input kernel
    assert not qk.qk_gemv_input_supported(3, 10, 256 * 129)  # more than 512 units per row


# ------------------------------------------------------------------ the whole step

def small_config(dim: int):
    """A 3-layer model 512 or 256 wide (at 256 the Q6_K matrices have one
    block per row, an odd count: the fused kernels take them when the row
    count is even, as here)."""
    from block_quantized_weight_gemv_amd.step import StepConfig

    if dim == 512:
        return StepConfig(dim=512, n_layers=3, n_heads=8, n_kv_heads=2, ffn=1024, vocab=300, max_pos=32)
    return StepConfig(dim=256, n_layers=3, n_heads=4, n_kv_heads=2, ffn=512, vocab=300, max_pos=32)


@pytest.mark.parametrize("dim,fused", [(512, True), (256, False), (256, True)],
                         ids=["fused", "separate", "fused-one-block-rows"])
def test_step_matches_oracle_and_graph_replays(qk, orc, dim, fused):
    """A 3-layer model over 10 positions: the GPU step's logits against the
    oracle's step, then the same sequence through a captured graph, which
    must reproduce the eager logits bit for bit."""
    from block_quantized_weight_gemv_amd.step import DecodeStep, synthetic_weights
    from oracle.step import OracleStep

    cfg = small_config(dim)
    w = synthetic_weights(cfg, seed=7)
    gpu, ref = DecodeStep(cfg, w, fuse=fused), OracleStep(orc, cfg, w)
    assert gpu.fused == fused
    toks = [1, 20, 299, 5, 5, 77, 0, 123, 200, 42]
    eager = []
    for pos, t in enumerate(toks):
        got = gpu.forward(t, pos).cpu().numpy().astype(np.float64)
        lr, a, _ = ref.forward(t, pos)
        ratio = np.abs(got - lr) / a
        assert ratio.max() <= 1e-3, (pos, float(ratio.max()))
        eager.append(got)
    g2 = DecodeStep(cfg, w, fuse=fused)
    g2.capture()
    for pos, t in enumerate(toks):
        assert np.array_equal(g2.forward(t, pos).cpu().numpy().astype(np.float64), eager[pos]), pos


def test_step_full_size_first_positions(qk, orc):
    """TinyLlama-1.1B shapes (22 layers, 2048 wide, 32/4 heads, FFN 5632,
    32000 tokens): the first two positions' logits against the oracle, every
    logit compared."""
    from block_quantized_weight_gemv_amd.step import DecodeStep, StepConfig, synthetic_weights
    from oracle.step import OracleStep

    cfg = StepConfig(max_pos=64)
    w = synthetic_weights(cfg, seed=8)
    gpu, ref = DecodeStep(cfg, w), OracleStep(orc, cfg, w)
    assert gpu.fused
    gpu.capture()
    for pos, t in enumerate([9, 31000]):
        got = gpu.forward(t, pos).cpu().numpy().astype(np.float64)
        lr, a, _ = ref.forward(t, pos)
        ratio = np.abs(got - lr) / a
        assert ratio.max() <= 1e-3, (pos, float(ratio.max()))

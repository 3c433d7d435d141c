"""The persistent decode pass (qk_gemv_pass_*) on the GPU, through the C ABI.

* A pass gives, bit for bit, what qk_gemv_batch gives stage by stage: on a
  TinyLlama-1.1B-shaped pass of 3 layers plus the output matrix (each
  stage with its own x) and on a chain in which every stage's x is the
  previous stage's y (the dependency the pass is for: stale or early reads
  of x would change the bits), over several runs with new inputs, and from
  a replayed HIP graph; every stage is also within the GEMV tolerance of the
  oracle on the x it read.
* A chain with the decode step's input transforms (RMSNorm with and without
  weights, SwiGLU of two earlier outputs) at TinyLlama-1.1B shapes: every
  stage within the GEMV tolerance of the oracle applied to the oracle's
  transform of the outputs the stage read; repeated runs and graph replays
  give the same bits.
* A run whose waits are forced to give up at once (spin limit 0, set from
  the host) still ends and is reported (qk_gemv_pass_gave_up); the next run
  with the default limit is exact again.
"""
import numpy as np
import pytest

from block_quantized_weight_gemv_amd import synth
from gpu_helpers import assert_gemv_close, to_dev

pytestmark = pytest.mark.gpu

Q4_K, Q6_K = 3, 4


@pytest.fixture(scope="module")
def qk():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_quantized_weight_gemv_amd import qk as mod

    return mod


LAYER = [[("q", Q4_K, 2048, 2048), ("k", Q4_K, 256, 2048), ("v", Q6_K, 256, 2048)], [("o", Q4_K, 2048, 2048)],
         [("gate", Q4_K, 5632, 2048), ("up", Q4_K, 5632, 2048)], [("down", Q6_K, 2048, 5632)]]


def decode_stages(n_layers, seed):
    """Stages of a 1.1B-shaped pass: per layer q/k/v, o, gate/up, down, then
    the output matrix; host weights and one x per stage."""
    stages = []
    for l in range(n_layers):
        for st in LAYER:
            stages.append([(f"{l}.{n}", t, r, c) for n, t, r, c in st])
    stages.append([("lm_head", Q6_K, 32000, 2048)])
    W = {n: synth.matrix(t, r, c, seed, stream=i) for i, (n, t, r, c) in enumerate(g for st in stages for g in st)}
    xs = [synth.vector(st[0][3], seed, stream=500 + s) for s, st in enumerate(stages)]
    return stages, W, xs


def test_decode_pass_equals_grouped_launches(qk, orc):
    import torch

    stages, W, xs = decode_stages(3, seed=11)
    Wd = {n: to_dev(w) for n, w in W.items()}
    xd = [to_dev(x) for x in xs]
    y_pass = {n: torch.full((r,), float("nan"), device="cuda") for st in stages for n, _, r, _ in st}
    y_batch = {n: torch.full((r,), float("nan"), device="cuda") for st in stages for n, _, r, _ in st}
    p = qk.GemvPass([[(t, Wd[n], r, c, xd[s], y_pass[n]) for n, t, r, c in st] for s, st in enumerate(stages)])
    assert p.grid > 0
    for _ in range(2):
        p.run()
    for s, st in enumerate(stages):
        qk.qk_gemv_batch([(t, Wd[n], r, c, xd[s], y_batch[n]) for n, t, r, c in st])
    torch.cuda.synchronize()
    assert not p.gave_up()
    for s, st in enumerate(stages):
        for n, t, r, c in st:
            assert torch.equal(y_pass[n], y_batch[n]), n
            if n.startswith("0.") or n == "lm_head":
                y_ref, a = orc.gemv(t, W[n], r, c, xs[s])
                assert_gemv_close(y_pass[n].cpu().numpy(), y_ref, a, f"pass {n}")
    p.close()


def chain_stages(seed, n_stages=12):
    """A chain: stage s reads the y of stage s - 1. Widths alternate 2048 and
    5632 (rows of split and unsplit plans) with both formats and two GEMVs
    in some stages; the block scales are small (x0.03) so that the values
    stay of order one along the chain."""
    dims = [2048]
    spec = []
    for s in range(n_stages):
        cols = dims[-1]
        rows = 5632 if (s % 3 == 1) else 2048
        t = Q6_K if s % 2 else Q4_K
        spec.append((t, rows, cols))
        dims.append(rows)
    W = [synth.matrix(t, r, c, seed, stream=s, scale=0.03) for s, (t, r, c) in enumerate(spec)]
    side = [synth.matrix(Q4_K if t == Q6_K else Q6_K, 256, c, seed, stream=100 + s, scale=0.03)
            for s, (t, r, c) in enumerate(spec)]
    return spec, W, side


@pytest.mark.parametrize("mode", ["eager", "graph"])
def test_chained_pass_reads_each_stage_output(qk, orc, mode):
    import torch

    spec, W, side = chain_stages(seed=12)
    Wd = [to_dev(w) for w in W]
    Sd = [to_dev(w) for w in side]
    x0 = torch.empty(2048, device="cuda")
    ys = [torch.full((r,), float("nan"), device="cuda") for _, r, _ in spec]
    zs = [torch.full((256,), float("nan"), device="cuda") for _ in spec]  # a second GEMV per stage, same x
    stages = []
    for s, (t, r, c) in enumerate(spec):
        x = x0 if s == 0 else ys[s - 1]
        stage = [(t, Wd[s], r, c, x, ys[s])]
        if s % 4 != 3:
            stage.append((Q4_K if t == Q6_K else Q6_K, Sd[s], 256, c, x, zs[s]))
        stages.append(stage)
    p = qk.GemvPass(stages)
    ref_y = [torch.empty_like(y) for y in ys]
    ref_z = [torch.empty_like(z) for z in zs]

    graph = None
    if mode == "graph":
        x0.copy_(torch.from_numpy(synth.vector(2048, 12, stream=1)).cuda())
        p.run()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            p.run()
    for run in range(4):
        xin = synth.vector(2048, 12, stream=10 + run)
        x0.copy_(torch.from_numpy(xin).cuda())
        for y in ys + zs:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        if graph is not None:
            graph.replay()
        else:
            p.run()
        torch.cuda.synchronize()
        assert not p.gave_up()
        # the same chain with one qk_gemv per matrix, in order on the stream
        xr = x0
        for s, (t, r, c) in enumerate(spec):
            qk.qk_gemv(t, Wd[s], r, c, xr, ref_y[s])
            if s % 4 != 3:
                qk.qk_gemv(Q4_K if t == Q6_K else Q6_K, Sd[s], 256, c, xr, ref_z[s])
            xr = ref_y[s]
        torch.cuda.synchronize()
        for s in range(len(spec)):
            assert torch.equal(ys[s], ref_y[s]), f"run {run} stage {s}"
            if s % 4 != 3:
                assert torch.equal(zs[s], ref_z[s]), f"run {run} stage {s} (second GEMV)"
        # every stage against the oracle on the x it read
        xh = xin
        for s, (t, r, c) in enumerate(spec):
            y_ref, a = orc.gemv(t, W[s], r, c, xh)
            yh = ys[s].cpu().numpy()
            assert_gemv_close(yh, y_ref, a, f"chain stage {s}")
            xh = yh
    p.close()


def test_forced_give_up_ends_and_is_reported(qk):
    """Spin limit 0: every wait gives up at once. The run still ends (the
    synchronisation returns), it is reported, and the next run with the
    default limit is exact again."""
    import torch

    spec, W, _ = chain_stages(seed=13, n_stages=6)
    Wd = [to_dev(w) for w in W]
    x0 = to_dev(synth.vector(2048, 13, stream=1))
    ys = [torch.empty(r, device="cuda") for _, r, _ in spec]
    stages = [[(t, Wd[s], r, c, x0 if s == 0 else ys[s - 1], ys[s])] for s, (t, r, c) in enumerate(spec)]
    p = qk.GemvPass(stages)
    p.set_spin_limit(0)
    p.run()
    torch.cuda.synchronize()
    assert p.gave_up()
    p.set_spin_limit(1 << 16)
    p.run()
    torch.cuda.synchronize()
    assert not p.gave_up()
    ref = torch.empty_like(ys[-1])
    xr = x0
    for s, (t, r, c) in enumerate(spec):
        out = ref if s == len(spec) - 1 else torch.empty(r, device="cuda")
        qk.qk_gemv(t, Wd[s], r, c, xr, out)
        xr = out
    torch.cuda.synchronize()
    assert torch.equal(ys[-1], ref)
    p.close()


def decode_chain(qk, n_layers, seed, eps=1e-5):
    """A chained 1.1B-shaped pass: per layer q/k/v read RMSNorm(the previous
    down output) with weights (layer 0: x0 as it is), o reads RMSNorm(q)
    (standing in for the attention output), gate/up RMSNorm(o), down
    SwiGLU(gate, up); then the output matrix reads RMSNorm(the last down).
    Returns host weights, device tensors and the pass's stages and inputs."""
    import torch

    spec = []
    for l in range(n_layers):
        spec.append([(f"{l}.q", Q4_K, 2048, 2048), (f"{l}.k", Q4_K, 256, 2048), (f"{l}.v", Q6_K, 256, 2048)])
        spec.append([(f"{l}.o", Q4_K, 2048, 2048)])
        spec.append([(f"{l}.gate", Q4_K, 5632, 2048), (f"{l}.up", Q4_K, 5632, 2048)])
        spec.append([(f"{l}.down", Q6_K, 2048, 5632)])
    spec.append([("lm_head", Q6_K, 32000, 2048)])
    W = {n: synth.matrix(t, r, c, seed, stream=i) for i, (n, t, r, c) in enumerate(g for st in spec for g in st)}
    Wd = {n: to_dev(w) for n, w in W.items()}
    y = {n: torch.full((r,), float("nan"), device="cuda") for st in spec for n, _, r, _ in st}
    x0 = to_dev(synth.vector(2048, seed, stream=7))
    nw = to_dev(np.abs(synth.vector(2048, seed, stream=8)) + np.float32(0.5))
    stages, inputs, src = [], [], []
    for s, st in enumerate(spec):
        head = st[0][0]
        l = head.split(".")[0]
        if head.endswith(".q"):
            if l == "0":
                x, inp, sr = x0, None, ("x0",)
            else:
                x, inp, sr = y[f"{int(l) - 1}.down"], (qk.QK_PASS_IN_RMSNORM, None, nw, eps), ("norm_w", f"{int(l) - 1}.down")
        elif head.endswith(".o"):
            x, inp, sr = y[f"{l}.q"], (qk.QK_PASS_IN_RMSNORM, None, None, eps), ("norm", f"{l}.q")
        elif head.endswith(".gate"):
            x, inp, sr = y[f"{l}.o"], (qk.QK_PASS_IN_RMSNORM, None, None, eps), ("norm", f"{l}.o")
        elif head.endswith(".down"):
            x, inp, sr = y[f"{l}.gate"], (qk.QK_PASS_IN_SWIGLU, y[f"{l}.up"], None, 0.0), ("swiglu", f"{l}.gate", f"{l}.up")
        else:
            x, inp, sr = y[f"{n_layers - 1}.down"], (qk.QK_PASS_IN_RMSNORM, None, None, eps), ("norm", f"{n_layers - 1}.down")
        stages.append([(t, Wd[n], r, c, x, y[n]) for n, t, r, c in st])
        inputs.append(inp)
        src.append(sr)
    return spec, W, y, x0, nw, stages, inputs, src


@pytest.mark.parametrize("mode", ["eager", "graph"])
def test_transformed_chain_matches_oracle(qk, orc, mode):
    import torch

    eps = 1e-5
    spec, W, y, x0, nw, stages, inputs, src = decode_chain(qk, 2, seed=21, eps=eps)
    p = qk.GemvPass(stages, inputs)
    first = None
    graph = None
    if mode == "graph":
        p.run()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            p.run()
    for run in range(3):
        for t in y.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay() if graph is not None else p.run()
        torch.cuda.synchronize()
        assert not p.gave_up()
        got = {n: t.cpu().numpy() for n, t in y.items()}
        if first is None:
            first = got
        else:
            for n in got:
                assert np.array_equal(got[n].view(np.uint32), first[n].view(np.uint32)), f"run {run}: {n} changed"
    # every stage against the oracle on the oracle's transform of what it read
    nwh = nw.cpu().numpy()
    for st, sr in zip(spec, src):
        if sr[0] == "x0":
            xh = x0.cpu().numpy()
        elif sr[0] == "norm_w":
            xh = orc.rmsnorm(first[sr[1]], nwh, eps)
        elif sr[0] == "norm":
            xh = orc.rmsnorm(first[sr[1]], np.ones(first[sr[1]].size, np.float32), eps)
        else:
            xh = orc.swiglu(first[sr[1]], first[sr[2]]).astype(np.float32)
        assert np.all(np.isfinite(xh))
        for n, t, r, c in st:
            y_ref, a = orc.gemv(t, W[n], r, c, xh)
            assert_gemv_close(first[n], y_ref, a, f"{mode} stage {n}")
    p.close()

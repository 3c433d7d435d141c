"""Helpers for the GPU parity tests: device copies of seeded inputs, guard
words around outputs, and the oracle comparison."""
from __future__ import annotations

import numpy as np

import oracle
from block_quantized_weight_gemv_amd import synth

CANARY = np.float32(-1.2345678e29)


def to_dev(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def guarded(n: int, guard: int = 64):
    """A device fp32 buffer of n + 2*guard values filled with a canary, and
    the 16-byte aligned view of its middle n values."""
    import torch

    buf = torch.full((n + 2 * guard,), float(CANARY), dtype=torch.float32, device="cuda")
    return buf, buf[guard:guard + n]


def check_guard(buf, n: int, guard: int = 64):
    h = buf.cpu().numpy()
    assert np.all(h[:guard] == CANARY), "write before the output"
    assert np.all(h[guard + n:] == CANARY), "write past the output"


def gemv_case(t: int, rows: int, cols: int, seed: int):
    W = synth.matrix(t, rows, cols, seed, stream=0)
    x = synth.vector(cols, seed)
    return W, x


def assert_gemv_close(y_gpu: np.ndarray, y_ref: np.ndarray, absacc: np.ndarray, what: str):
    ok, worst = oracle.within_tolerance(y_gpu, y_ref, absacc)
    assert ok, f"{what}: worst |err| / (1e-4*sum|w*x| + 1e-6) = {worst:.3g}"
    return worst

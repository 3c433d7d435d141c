"""The seeded input generators (block_quantized_weight_gemv_amd/synth.py),
on the host: the full-range mode reaches every extreme value the formats'
fields can hold, and the default mode keeps the workload's ranges."""
import numpy as np

from block_quantized_weight_gemv_amd import synth

Q4_0, Q8_0, Q4_K, Q6_K = 1, 2, 3, 4
Q8_0_F16 = 5


def test_generator_reaches_the_whole_range():
    """The full-range blocks do hold the extreme values (checked on the
    host, on the bytes the tests below upload)."""
    b = synth.blocks(Q6_K, 4096, synth.rng(1, 1), full=True)
    sc = b[:, 192:208].view(np.int8)
    assert sc.min() == -128 and sc.max() == 127
    d = b[:, 208:210].copy().view(np.uint16).ravel()
    assert (d >> 15).any() and ((d & 0x7C00) == 0).any() and ((d & 0x7FFF) == 0).any() and (d == 0x8000).any()
    q = synth.blocks(Q8_0, 4096, synth.rng(1, 2), full=True)
    assert q[:, 4:].view(np.int8).min() == -128
    s = q[:, 0:4].copy().view(np.float32).ravel()
    assert (s < 0).any() and (np.abs(s) < 1.2e-38).any()  # fp32 subnormal scales
    q = synth.blocks(Q8_0_F16, 4096, synth.rng(1, 3), full=True)
    assert q[:, 2:].view(np.int8).min() == -128


def test_default_ranges():
    b = synth.blocks(Q6_K, 4096, synth.rng(1, 1))
    sc = b[:, 192:208].view(np.int8)
    assert sc.min() == -64 and sc.max() == 63
    d = b[:, 208:210].copy().view(np.float16).astype(np.float64).ravel()
    assert d.min() >= 0.9999e-4 and d.max() <= 1.0001e-3
    q = synth.blocks(Q8_0, 4096, synth.rng(1, 2))
    assert q[:, 4:].view(np.int8).min() == -127

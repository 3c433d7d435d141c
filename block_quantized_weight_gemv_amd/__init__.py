"""Block-quantized weight GEMV for AMD MI355X (gfx950).

The product is the C-ABI library ``libqk.so`` (hand-written HIP kernels,
declared in ``include/qk.h``); :mod:`.qk` is its thin ctypes binding,
:mod:`.synth` draws seeded synthetic inputs and :mod:`.rocprof` is the
rocprofv3 harness behind the committed profiles. The binding is imported lazily
so that the input generator can be used without loading the GPU library.
"""
from __future__ import annotations

import importlib

__all__ = ["qk", "synth", "build", "rocprof"]


def __getattr__(name):
    if name in ("qk", "synth", "build", "rocprof"):
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)

"""qasi -- query-aware sparse KV index, selection and sparse decode for MI355X (gfx950).

The computation lives in libqasi.so (hand-written HIP kernels behind a C ABI, see
include/qasi.h).  `api` is the torch-tensor binding; `synth` draws seeded inputs.
The binding is imported lazily so that input generation works without the library.
"""
from __future__ import annotations

import importlib

__all__ = ["api", "synth", "build_lib"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)

"""One-GPU join-agg engine for AMD Instinct MI355X (gfx950).

Every operation (contraction, attention, RMSNorm, SwiGLU, residual add) runs
as a join of blocked tensor relations into tuples, a per-tuple HIP kernel and
an aggregation by output key, with repartitioning between blockings.  The
compute lives in libja.so (C ABI: include/ja.h); ``binding`` is its ctypes
binding and ``device`` adds torch-allocated device buffers and streams.

Submodules are imported on first use, so ``synth`` (seeded inputs) works
without the built library; touching ``binding`` or ``device`` without
libja.so raises ImportError.
"""
import importlib

__all__ = ["binding", "device", "synth", "block"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)

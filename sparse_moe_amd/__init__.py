"""MI355X-native routed-MoE layer (Gemma 4 26B-A4B shape) with Q4_0 experts.

The compute lives in hand-written HIP kernels for gfx950 behind a C-ABI
library (libsparse_moe_amd.so, declared in include/sparse_moe.h).  The
binding in ``sparse_moe_amd.binding`` only marshals torch tensors into that
ABI; it is imported lazily so that the input generator (``synth``) can be used
without loading the GPU library.
"""
import importlib

__all__ = ["binding", "synth"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)

"""MI355X-native quantized (INT8 QK / FP8 PV) self-attention for video diffusion transformers.

The compute path is the C-ABI library ``libsattn.so`` (hand-written HIP kernels for
gfx950, declared in ``include/sattn.h``); ``binding`` marshals torch tensors into it.
Importing the package loads nothing: the library is opened on first use.
"""
__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in ("binding", "workloads"):
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)

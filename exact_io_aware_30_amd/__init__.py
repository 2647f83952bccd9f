"""MI355X-native exact FlashAttention-2, forward and backward.

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``, header ``include/fa.h``); ``binding`` marshals torch
tensors into it; ``interface`` adds ``flash_attn``, its autograd.Function
and the ``FlashSelfAttention`` module on top.  ``workloads`` draws the
seeded synthetic inputs and counts FLOPs and bytes.  Submodules are imported on demand so that the input
generator can be used where the native library is not built.
"""

__all__ = ["binding", "interface", "workloads"]


def __getattr__(name):
    if name in __all__:
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)

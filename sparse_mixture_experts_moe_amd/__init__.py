"""MI355X-native routed MoE FFN layer: HIP kernels behind a small C ABI.

`sparse_mixture_experts_moe_amd.binding` is the ctypes binding of the C ABI
(same entry-point names as include/moe.h).  It is imported lazily so that the
pure-host helpers (e.g. `costmodel`) work without the built library.
"""
import importlib

__all__ = ["binding", "costmodel"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)

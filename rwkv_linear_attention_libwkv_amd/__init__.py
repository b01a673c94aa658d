"""libwkv for MI355X: the RWKV-4 WKV operator as a C-ABI library with HIP kernels.

``libwkv`` (the ctypes binding) is imported on first attribute access so that
``workloads`` can be used without loading the shared library.
"""
import importlib

__all__ = ["libwkv", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)

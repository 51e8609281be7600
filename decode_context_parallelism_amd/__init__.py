"""dcpmla: decode-context-parallel MLA causal verification for MI355X (gfx950).

The compute lives in ``libdcpmla.so`` (HIP kernels behind the C ABI of
``include/dcpmla.h``); ``ops`` is a thin PyTorch-tensor binding over it and
``build`` compiles it.  ``ops`` is imported lazily so that ``build`` works
before the library exists; importing ``ops`` without the library raises.
"""
import importlib

__all__ = ["ops", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)

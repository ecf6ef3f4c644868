"""MI355X-native Gated DeltaNet mixer core.

The compute path is the C-ABI library ``libgdn.so`` (hand-written HIP kernels
for gfx950, declared in ``include/gdn.h``).  ``binding`` marshals torch tensors
into its argument structs; it loads the library lazily and raises if it is
missing -- there is no fallback path.
"""
import importlib

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(__name__ + "." + name)
    raise AttributeError(name)

"""MI355X-native forward pass of Native Sparse Attention (NSA).

The compute lives in ``libnsa.so`` (HIP kernels for gfx950 behind the C ABI in
``include/nsa.h``); ``ops`` is its Python binding.  ``configs`` names the workloads and
``inputs`` draws their seeded synthetic inputs.  ``ops`` (and with it torch) is loaded on
first attribute access so that the input generators import without a GPU stack.
"""
import importlib

__all__ = ["configs", "inputs", "ops"]


def __getattr__(name):
    if name == "ops":
        return importlib.import_module(__name__ + ".ops")
    raise AttributeError(name)

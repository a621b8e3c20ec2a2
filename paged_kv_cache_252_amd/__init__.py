"""MI355X-native paged decode attention.

The compute lives in a HIP library built for gfx950 (``libpagedkv.so``,
sources under ``csrc/``) behind a small C ABI; ``ops`` is a thin ctypes
binding to it that marshals torch tensors and the current stream.
``inputs`` draws seeded synthetic workloads.  Nothing here computes
attention on the CPU: if the library is missing, ``ops`` raises.
"""

__all__ = ["ops", "inputs"]


def __getattr__(name):
    if name in ("ops", "inputs"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)

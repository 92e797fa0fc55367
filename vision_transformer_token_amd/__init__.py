"""MI355X-native LiSA (Linear Stochastic Attention) forward pass.

The compute path is a hand-written HIP library for gfx950
(``liblisa.so``, C ABI declared in ``include/lisa.h``).  ``lisa`` is the thin
ctypes binding with the library's entry-point names; it is imported lazily so
that CPU-only users of ``workloads`` never load the GPU library.
"""

__all__ = ["lisa", "workloads"]


def __getattr__(name):
    if name in ("lisa", "workloads"):
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)

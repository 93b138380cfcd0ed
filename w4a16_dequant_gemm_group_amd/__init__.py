"""libgq: group-wise INT4 weight quantization and fused W4A16 GEMV/GEMM for
AMD MI355X (gfx950), behind a C ABI (``include/gq.h``).

The Python layer is a thin ctypes binding (``binding``) with the same names as
the C entry points.  Importing the package does not load the shared library;
the first call does, and fails loudly if it has not been built.
"""
__all__ = ["binding"]


def __getattr__(name):
    if name == "binding":
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    from . import binding
    return getattr(binding, name)

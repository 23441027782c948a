"""FluxBin LUT GEMV for MI355X (gfx950): hand-written HIP kernels behind a C ABI.

Importing the package loads nothing.  ``binary_basis_lut_amd.fluxbin`` is the
thin ctypes binding of ``libfluxbin.so`` (argument marshalling only); it raises
when the library has not been built.  ``inputs`` draws seeded synthetic data
and ``accounting`` counts the bytes and operations of one call.
"""

__all__ = ["fluxbin", "inputs", "accounting"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)

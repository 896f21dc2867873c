"""Exact ring-ordered attention forward for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libringattn.so`` (C ABI in
``include/ringattn.h``); :mod:`exact_long_context_amd.ringattn` is its ctypes
binding and :mod:`exact_long_context_amd.api` adds tensor-allocating
conveniences on top.  Build the library with
``python -m exact_long_context_amd.build``.
"""

__all__ = ["ringattn", "api", "build"]


def __getattr__(name):
    # imported on first use so that the build module works before the library exists
    if name in ("ringattn", "api"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)

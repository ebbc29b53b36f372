"""Integer-only training step for AMD MI355X (gfx950).

The computation lives in libionn.so (HIP kernels behind the C ABI declared
in include/ionn.h).  ``ops`` binds each C entry point by name; ``steps``
sequences them into whole training steps.  There is no CPU fallback: the
package raises if the library has not been built.
"""
from ._lib import IonnError, LIB_PATH, header_functions, lib  # noqa: F401

__all__ = ["IonnError", "LIB_PATH", "header_functions", "lib", "ops", "steps"]


def __getattr__(name):
    if name in ("ops", "steps"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)

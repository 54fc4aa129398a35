"""Gated DeltaNet prompt-path recurrence for MI355X (gfx950).

The compute lives in a C-ABI shared library (``libgdn.so``, declared in ``include/gdn.h``)
built from hand-written HIP kernels in ``csrc/``.  ``gdn`` is the thin Python binding over
that library (argument marshalling only), ``inputs`` the seeded synthetic-input generator.

The binding is imported lazily so that the input generator can be used without the
library; every compute call fails loudly if the library has not been built.
"""
from .inputs import (DK, DV, EDGE_LENGTHS, N_K_HEADS, N_V_HEADS, make_inputs,  # noqa: F401
                     make_pre_inputs)

__all__ = ["make_inputs", "make_pre_inputs", "EDGE_LENGTHS", "N_K_HEADS", "N_V_HEADS", "DK", "DV", "gdn"]


def __getattr__(name):
    if name == "gdn":
        import importlib
        return importlib.import_module(__name__ + ".gdn")
    raise AttributeError(name)

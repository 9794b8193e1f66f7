"""MI355X-native Mixture-of-Kittens-style MoE layer: a C-ABI HIP library (libmok.so)
with a thin Python binding.  Importing the package loads nothing; `_lib.load()` loads
the library and fails loudly when it has not been built."""
from . import gen  # noqa: F401

__all__ = ["gen"]

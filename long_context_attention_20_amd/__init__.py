"""MI355X (gfx950) hybrid compressed attention: CSA + HCA + sliding window.

liblca.so (HIP, built in-tree) holds every kernel; this package marshals
torch tensors into its C-ABI (``ops``) and sequences one layer step
(``pipeline.HybridAttention``).  Importing fails loudly when the library has
not been built -- there is no CPU fallback.
"""
from ._lib import LIB_PATH, LCAError, lib  # noqa: F401  (loads liblca.so)
from . import ops  # noqa: F401
from .pipeline import Caches, HybridAttention, n_windows  # noqa: F401

__all__ = ["ops", "HybridAttention", "Caches", "n_windows", "LCAError", "lib", "LIB_PATH"]
